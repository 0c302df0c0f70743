"""fly_decode_amd -- lossless codebook-compressed BF16 weights decoded on MI355X (gfx950).

A thin ctypes binding over ``libcbk.so`` (C ABI declared in ``include/cbk.h`` and, for the
exponent entropy-coded format, ``include/cbk_ec.h``).  Every step of the
hot path runs in the library's HIP kernels; this module only marshals arguments.  PyTorch is used
for device memory and streams: inputs and outputs are torch tensors whose ``data_ptr()`` is handed
to the library, and GPU calls are enqueued on ``torch.cuda.current_stream()``.

If the library has not been built, importing works but every call raises ``RuntimeError``: there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["CBK_OK", "CbkError", "bits_for", "words_for", "compressed_bytes", "encode",
           "Compressed", "decode_bf16", "decode_group", "gemv", "gemv_group", "gemm_small", "library_path",
           "load_library", "ECTensor", "ec_encode", "ec_decode_bf16", "ec_gemv", "ec_build_index",
           "ec_decode_group", "ec_gemv_group", "cap_patterns",
           "GemvChain"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# CBK_LIBRARY names another build of the same library (for side-by-side comparisons)
_LIB_PATH = os.environ.get("CBK_LIBRARY") or os.path.join(_HERE, "libcbk.so")
_lib = None

CBK_OK = 0
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)


class CbkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {load_library().cbk_status_str(status).decode()} (status {status})")


class _Tensor(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_uint64), ("cols", ctypes.c_uint64), ("U", ctypes.c_uint32),
                ("b", ctypes.c_uint32), ("codebook", ctypes.c_void_p), ("words", ctypes.c_void_p)]


class _EncodeJob(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("n", ctypes.c_uint64), ("codebook", ctypes.c_void_p),
                ("words", ctypes.c_void_p), ("words_cap", ctypes.c_uint64), ("meta", ctypes.c_void_p)]


class _GemvPhase(ctypes.Structure):
    _fields_ = [("ts", ctypes.POINTER(_Tensor)), ("count", ctypes.c_uint32), ("x", ctypes.c_void_p),
                ("ys", ctypes.POINTER(ctypes.c_void_p))]


class _GemvChain(ctypes.Structure):
    _fields_ = [("buffer", ctypes.c_void_p), ("phases", ctypes.c_uint32), ("b", ctypes.c_uint32),
                ("grid", ctypes.c_uint32), ("lds_bytes", ctypes.c_uint32), ("x_bytes", ctypes.c_uint32),
                ("device", ctypes.c_uint32)]


class _ECHeader(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64), ("lengths", ctypes.c_uint8 * 256)]


class _ECTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64), ("sm", ctypes.c_void_p),
                ("stream", ctypes.c_void_p), ("gaps", ctypes.c_void_p), ("bases", ctypes.c_void_p),
                ("lut", ctypes.c_void_p), ("max_block_codes", ctypes.c_uint32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libcbk.so (built in-tree by fly_decode_amd/build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run fly_decode_amd/build.py (or "
                               "__graft_entry__.build()) first; there is no fallback path")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.cbk_bits_for.restype = ctypes.c_uint32
        lib.cbk_bits_for.argtypes = [ctypes.c_uint32]
        lib.cbk_words_for.restype = ctypes.c_uint64
        lib.cbk_words_for.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        lib.cbk_compressed_bytes.restype = ctypes.c_uint64
        lib.cbk_compressed_bytes.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        lib.cbk_status_str.restype = ctypes.c_char_p
        lib.cbk_status_str.argtypes = [ctypes.c_int]
        lib.cbk_encode.restype = ctypes.c_int
        lib.cbk_encode.argtypes = [_u16p, ctypes.c_uint64, _u16p, _u32p, _u32p, _u32p,
                                   ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        tp = ctypes.POINTER(_Tensor)
        lib.cbk_decode_bf16.restype = ctypes.c_int
        lib.cbk_decode_bf16.argtypes = [tp, ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_gemv.restype = ctypes.c_int
        lib.cbk_gemv.argtypes = [tp, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_gemv_group.restype = ctypes.c_int
        lib.cbk_gemv_group.argtypes = [tp, ctypes.c_uint32, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]
        lib.cbk_gemm_small.restype = ctypes.c_int
        lib.cbk_gemm_small.argtypes = [tp, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
        lib.cbk_cap_patterns.restype = ctypes.c_int
        lib.cbk_cap_patterns.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                         _u32p]
        lib.cbk_encode_gpu_workspace_bytes.restype = ctypes.c_size_t
        lib.cbk_encode_gpu_workspace_bytes.argtypes = []
        lib.cbk_encode_gpu.restype = ctypes.c_int
        lib.cbk_encode_gpu.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_decode_group.restype = ctypes.c_int
        lib.cbk_decode_group.argtypes = [tp, ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]
        lib.cbk_encode_gpu_group.restype = ctypes.c_int
        lib.cbk_encode_gpu_group.argtypes = [ctypes.POINTER(_EncodeJob), ctypes.c_uint32, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.cbk_encode_gpu_noalloc.restype = ctypes.c_int
        lib.cbk_encode_gpu_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_gemm_group.restype = ctypes.c_int
        lib.cbk_gemm_group.argtypes = [tp, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.c_void_p]
        lib.cbk_gemv_chain_bytes.restype = ctypes.c_size_t
        lib.cbk_gemv_chain_bytes.argtypes = [ctypes.c_uint32]
        lib.cbk_gemv_chain_init.restype = ctypes.c_int
        lib.cbk_gemv_chain_init.argtypes = [ctypes.POINTER(_GemvPhase), ctypes.c_uint32, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.POINTER(_GemvChain)]
        lib.cbk_gemv_chain_run.restype = ctypes.c_int
        lib.cbk_gemv_chain_run.argtypes = [ctypes.POINTER(_GemvChain), ctypes.c_uint32, ctypes.c_void_p]
        lib.cbk_gemv_chain_check.restype = ctypes.c_int
        lib.cbk_gemv_chain_check.argtypes = [ctypes.POINTER(_GemvChain)]
        hp = ctypes.POINTER(_ECHeader)
        for name in ("cbk_ec_spans", "cbk_ec_stream_words", "cbk_ec_gap_words", "cbk_ec_blocks",
                     "cbk_ec_stored_bytes"):
            getattr(lib, name).restype = ctypes.c_uint64
            getattr(lib, name).argtypes = [hp]
        lib.cbk_ec_plan.restype = ctypes.c_int
        lib.cbk_ec_plan.argtypes = [ctypes.c_void_p, ctypes.c_uint64, hp]
        lib.cbk_ec_encode.restype = ctypes.c_int
        lib.cbk_ec_encode.argtypes = [ctypes.c_void_p, hp] + [ctypes.c_void_p] * 5
        lib.cbk_ec_decode_bf16.restype = ctypes.c_int
        lib.cbk_ec_decode_bf16.argtypes = [ctypes.POINTER(_ECTensor), ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_ec_gemv.restype = ctypes.c_int
        lib.cbk_ec_gemv.argtypes = [ctypes.POINTER(_ECTensor), ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_ec_index_bytes.restype = ctypes.c_uint64
        lib.cbk_ec_index_bytes.argtypes = [ctypes.c_uint64]
        lib.cbk_ec_build_index.restype = ctypes.c_int
        lib.cbk_ec_build_index.argtypes = [ctypes.POINTER(_ECTensor), ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_ec_decode_bf16_indexed.restype = ctypes.c_int
        lib.cbk_ec_decode_bf16_indexed.argtypes = [ctypes.POINTER(_ECTensor), ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p]
        lib.cbk_ec_gemv_indexed.restype = ctypes.c_int
        lib.cbk_ec_gemv_indexed.argtypes = [ctypes.POINTER(_ECTensor), ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.cbk_ec_max_block_codes.restype = ctypes.c_uint32
        lib.cbk_ec_max_block_codes.argtypes = [hp, ctypes.c_void_p]
        lib.cbk_ec_decode_group.restype = ctypes.c_int
        lib.cbk_ec_decode_group.argtypes = [ctypes.POINTER(_ECTensor), ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                            ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]
        lib.cbk_ec_gemv_group.restype = ctypes.c_int
        lib.cbk_ec_gemv_group.argtypes = [ctypes.POINTER(_ECTensor), ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                          ctypes.POINTER(ctypes.c_uint64), ctypes.c_uint64, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]
        _lib = lib
    return _lib


def bits_for(U: int) -> int:
    return int(load_library().cbk_bits_for(U))


def words_for(n: int, b: int) -> int:
    return int(load_library().cbk_words_for(n, b))


def compressed_bytes(n: int, U: int) -> int:
    return int(load_library().cbk_compressed_bytes(n, U))


class Compressed:
    """A compressed tensor: codebook (uint16[U]) and words (uint32[words_for(n, b)]).

    Host arrays after ``encode``; ``to(device)`` returns a copy whose arrays are torch tensors on
    that device, ready for the GPU calls."""

    def __init__(self, rows, cols, U, b, codebook, words):
        self.rows, self.cols, self.U, self.b = int(rows), int(cols), int(U), int(b)
        self.codebook, self.words = codebook, words

    @property
    def n(self) -> int:
        return self.rows * self.cols

    @property
    def compressed_bytes(self) -> int:
        return compressed_bytes(self.n, self.U)

    def to(self, device) -> "Compressed":
        import torch
        def put(a, view):
            if isinstance(a, np.ndarray):
                return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(device)
            return a.to(device)
        cb = put(self.codebook, np.int16)
        wd = put(self.words, np.int32)
        return Compressed(self.rows, self.cols, self.U, self.b, cb, wd)

    def _struct(self) -> _Tensor:
        cb = self.codebook.data_ptr() if self.U and self.codebook.numel() else None
        wd = self.words.data_ptr() if self.words.numel() else None
        return _Tensor(self.rows, self.cols, self.U, self.b, cb, wd)


def cap_patterns(w, K: int):
    """cbk_cap_patterns: the lossy capped-codebook step.  Returns (patterns with at most K
    distinct values, same shape as w, uint16; their distinct count)."""
    w = np.ascontiguousarray(w).view(np.uint16)
    out = np.empty_like(w)
    U = ctypes.c_uint32()
    _check(load_library().cbk_cap_patterns(w.ctypes.data if w.size else None, w.size, K,
                                           out.ctypes.data if w.size else None, ctypes.byref(U)),
           "cbk_cap_patterns")
    return out, int(U.value)


def encode(w, rows: int | None = None, cols: int | None = None, cap: int | None = None) -> Compressed:
    """Compress a host array of BF16 bit patterns (numpy uint16/int16, or a CPU torch tensor of
    bfloat16/int16/uint16), shape [rows][cols] (or 1-D with rows/cols given).  With ``cap`` the
    tensor first goes through cbk_cap_patterns (lossy when it has more than cap distinct values)."""
    if hasattr(w, "detach"):
        w = w.detach().contiguous().cpu()
        w = w.view(__import__("torch").int16).numpy()
    w = np.ascontiguousarray(w)
    if w.dtype not in (np.uint16, np.int16):
        raise TypeError("encode expects 16-bit patterns")
    if cap is not None:
        w, _ = cap_patterns(w, cap)
    if rows is None:
        rows, cols = (w.shape if w.ndim == 2 else (1, w.size))
    flat = w.reshape(-1).view(np.uint16)
    if flat.size != rows * cols:
        raise ValueError("rows * cols does not match the array size")
    lib = load_library()
    cb = np.zeros(65536, dtype=np.uint16)
    U, b, need = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint64()
    src = flat.ctypes.data_as(_u16p) if flat.size else None
    st = lib.cbk_encode(src, flat.size, cb.ctypes.data_as(_u16p), ctypes.byref(U), ctypes.byref(b),
                        None, 0, ctypes.byref(need))
    if st not in (CBK_OK, 2):
        raise CbkError(st, "cbk_encode")
    words = np.zeros(need.value, dtype=np.uint32)
    st = lib.cbk_encode(src, flat.size, cb.ctypes.data_as(_u16p), ctypes.byref(U), ctypes.byref(b),
                        words.ctypes.data_as(_u32p) if words.size else None, words.size,
                        ctypes.byref(need))
    if st != CBK_OK:
        raise CbkError(st, "cbk_encode")
    return Compressed(rows, cols, U.value, b.value, cb[:U.value].copy(), words)


def encode_gpu_workspace_bytes() -> int:
    return int(load_library().cbk_encode_gpu_workspace_bytes())


def encode_gpu_launch(w, workspace, codebook, words, meta, stream=None) -> None:
    """Enqueue cbk_encode_gpu on the stream without waiting: w holds n 16-bit patterns; workspace,
    codebook (65536 entries), words (at least words_for(n, 16) words) and meta (two uint32: U, b)
    are device tensors the caller owns."""
    n = w.numel()
    _check(load_library().cbk_encode_gpu(
        ctypes.c_void_p(w.data_ptr() if n else None), n, ctypes.c_void_p(workspace.data_ptr()),
        ctypes.c_void_p(codebook.data_ptr()), ctypes.c_void_p(words.data_ptr()),
        words.numel() * words.element_size() // 4, ctypes.c_void_p(meta.data_ptr()), _stream(stream)),
        "cbk_encode_gpu")


def encode_gpu_group_launch(ws, workspace, codebooks, words, metas, stream=None) -> None:
    """Enqueue cbk_encode_gpu_group: tensors ws[i] encoded into codebooks[i], words[i], metas[i] (as
    ``encode_gpu_launch``), one run of three launches per 8 tensors; workspace holds
    min(len(ws), 8) * encode_gpu_workspace_bytes() bytes."""
    jobs = (_EncodeJob * len(ws))(*[
        _EncodeJob(w.data_ptr() if w.numel() else None, w.numel(), cb.data_ptr(), wd.data_ptr(),
                   wd.numel() * wd.element_size() // 4, m.data_ptr())
        for w, cb, wd, m in zip(ws, codebooks, words, metas)])
    _check(load_library().cbk_encode_gpu_group(jobs, len(ws), ctypes.c_void_p(workspace.data_ptr()),
                                               _stream(stream)), "cbk_encode_gpu_group")


def encode_gpu_noalloc_launch(w, codebook, words, meta, stream=None) -> None:
    """Enqueue cbk_encode_gpu_noalloc: as ``encode_gpu_launch`` with the library's static scratch
    in place of a workspace (nothing is allocated; calls that overlap on one GPU race)."""
    n = w.numel()
    _check(load_library().cbk_encode_gpu_noalloc(
        ctypes.c_void_p(w.data_ptr() if n else None), n, ctypes.c_void_p(codebook.data_ptr()),
        ctypes.c_void_p(words.data_ptr()), words.numel() * words.element_size() // 4,
        ctypes.c_void_p(meta.data_ptr()), _stream(stream)), "cbk_encode_gpu_noalloc")


def encode_gpu(w, rows: int | None = None, cols: int | None = None, stream=None) -> Compressed:
    """Compress BF16 bit patterns already on the GPU (a contiguous bfloat16/int16/uint16 torch
    tensor, shape [rows][cols] or 1-D with rows/cols given) with cbk_encode_gpu.  The result is
    bit-identical to ``encode`` and stays on the device; U and b are read back (one sync)."""
    import torch
    if not w.is_contiguous() or w.element_size() != 2:
        raise ValueError("encode_gpu expects a contiguous tensor of 16-bit patterns")
    if rows is None:
        rows, cols = (tuple(w.shape) if w.dim() == 2 else (1, w.numel()))
    n = w.numel()
    if n != rows * cols:
        raise ValueError("rows * cols does not match the tensor size")
    dev = w.device
    ws = torch.empty(encode_gpu_workspace_bytes(), dtype=torch.uint8, device=dev)
    cb = torch.empty(65536, dtype=torch.int16, device=dev)
    words = torch.empty(max(words_for(n, 16), 4), dtype=torch.int32, device=dev)
    meta = torch.zeros(2, dtype=torch.int32, device=dev)
    encode_gpu_launch(w, ws, cb, words, meta, stream)
    U, b = (int(v) for v in meta.cpu().tolist())
    return Compressed(rows, cols, U, b, cb[:U], words[:words_for(n, b)])


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st, what):
    if st != CBK_OK:
        raise CbkError(st, what)


def decode_bf16(t: Compressed, out=None, stream=None):
    """Standalone decode into a [rows][cols] torch.bfloat16 tensor (exact original bits)."""
    import torch
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device=t.words.device)
    ts = t._struct()
    _check(load_library().cbk_decode_bf16(ctypes.byref(ts), ctypes.c_void_p(out.data_ptr() or None),
                                          _stream(stream)), "cbk_decode_bf16")
    return out


def decode_group(ts, outs=None, stream=None):
    """cbk_decode_group: several tensors decoded into [rows][cols] torch.bfloat16 tensors, one launch
    per run of up to 8 of one width (each output bit-identical to ``decode_bf16``)."""
    import torch
    if outs is None:
        outs = [torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device=t.words.device) for t in ts]
    arr = (_Tensor * len(ts))(*[t._struct() for t in ts])
    ptrs = (ctypes.c_void_p * len(outs))(*[o.data_ptr() or None for o in outs])
    _check(load_library().cbk_decode_group(arr, len(ts), ptrs, _stream(stream)), "cbk_decode_group")
    return outs


def gemv(t: Compressed, x, y=None, stream=None):
    """y[rows] (float32) = W . x for a torch.bfloat16 vector x[cols] on the device."""
    import torch
    if x.dtype != torch.bfloat16 or x.numel() != t.cols or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 vector of length cols")
    if y is None:
        y = torch.empty(t.rows, dtype=torch.float32, device=x.device)
    ts = t._struct()
    _check(load_library().cbk_gemv(ctypes.byref(ts), ctypes.c_void_p(x.data_ptr() or None),
                                   ctypes.c_void_p(y.data_ptr() or None), _stream(stream)),
           "cbk_gemv")
    return y


def gemv_group(ts, x, ys=None, stream=None):
    """ys[i] (float32, rows_i) = W_i . x for tensors that share one bfloat16 vector x."""
    import torch
    ts = list(ts)
    if not ts:
        return []
    K = ts[0].cols
    if x.dtype != torch.bfloat16 or x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 vector of length cols")
    if ys is None:
        ys = [torch.empty(t.rows, dtype=torch.float32, device=x.device) for t in ts]
    arr = (_Tensor * len(ts))(*[t._struct() for t in ts])
    yp = (ctypes.c_void_p * len(ts))(*[y.data_ptr() or None for y in ys])
    _check(load_library().cbk_gemv_group(arr, len(ts), ctypes.c_void_p(x.data_ptr() or None), yp,
                                         _stream(stream)), "cbk_gemv_group")
    return ys


def gemm_small(t: Compressed, X, Y=None, stream=None):
    """Y[batch][rows] (float32) = X . W^T for a torch.bfloat16 X[batch][cols] (row stride may
    exceed cols but must be a multiple of 8)."""
    import torch
    if X.dtype != torch.bfloat16 or X.dim() != 2 or X.shape[1] != t.cols or X.stride(1) != 1:
        raise ValueError("X must be a [batch][cols] bfloat16 matrix with unit column stride")
    batch = X.shape[0]
    if Y is None:
        Y = torch.empty((batch, t.rows), dtype=torch.float32, device=X.device)
    ts = t._struct()
    _check(load_library().cbk_gemm_small(ctypes.byref(ts), ctypes.c_void_p(X.data_ptr() or None),
                                         X.stride(0), batch, ctypes.c_void_p(Y.data_ptr() or None),
                                         Y.stride(0), _stream(stream)), "cbk_gemm_small")
    return Y


def gemm_group(ts, X, Ys=None, stream=None):
    """Ys[i][batch][rows_i] (float32) = X . W_i^T for tensors that share one bfloat16 X[batch][cols]
    (row stride of X may exceed cols but must be a multiple of 8 for the fast kernels)."""
    import torch
    ts = list(ts)
    if not ts:
        return []
    K = ts[0].cols
    if X.dtype != torch.bfloat16 or X.dim() != 2 or X.shape[1] != K or X.stride(1) != 1:
        raise ValueError("X must be a [batch][cols] bfloat16 matrix with unit column stride")
    batch = X.shape[0]
    if Ys is None:
        Ys = [torch.empty((batch, t.rows), dtype=torch.float32, device=X.device) for t in ts]
    arr = (_Tensor * len(ts))(*[t._struct() for t in ts])
    yp = (ctypes.c_void_p * len(ts))(*[Y.data_ptr() or None for Y in Ys])
    ld = (ctypes.c_uint64 * len(ts))(*[Y.stride(0) for Y in Ys])
    _check(load_library().cbk_gemm_group(arr, len(ts), ctypes.c_void_p(X.data_ptr() or None), X.stride(0),
                                         batch, yp, ld, _stream(stream)), "cbk_gemm_group")
    return Ys


class GemvChain:
    """cbk_gemv_chain_*: dependent GEMV phases run by one persistent launch.

    ``phases`` is a list of (tensors, x, ys): device ``Compressed`` tensors that share the
    bfloat16 vector x (same cols and, across the whole chain, the same b), and their float32
    outputs ys (rows_i each).  The library records the device pointers, so every tensor, x and y
    must stay alive (this object keeps references).  ``run()`` enqueues one pass over every phase
    on the current stream; ``check()`` (after synchronizing) returns 0, or CBK_E_TIMEOUT (6) when a
    barrier wait of the last run gave up."""

    def __init__(self, phases, device=None):
        import torch
        phases = [(list(ts), x, list(ys)) for ts, x, ys in phases]
        if not phases:
            raise ValueError("a chain needs at least one phase")
        lib = load_library()
        arr = (_GemvPhase * len(phases))()
        keep = []
        for i, (ts, x, ys) in enumerate(phases):
            if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.numel() != ts[0].cols:
                raise ValueError("x must be a contiguous bfloat16 vector of length cols")
            tarr = (_Tensor * len(ts))(*[t._struct() for t in ts])
            yarr = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
            keep += [tarr, yarr]
            arr[i] = _GemvPhase(tarr, len(ts), x.data_ptr(), yarr)
        nbytes = int(lib.cbk_gemv_chain_bytes(len(phases)))
        dev = device if device is not None else phases[0][1].device
        self.buffer = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        off = (-self.buffer.data_ptr()) % 256
        self._chain = _GemvChain()
        _check(lib.cbk_gemv_chain_init(arr, len(phases), ctypes.c_void_p(self.buffer.data_ptr() + off), nbytes,
                                       ctypes.byref(self._chain)), "cbk_gemv_chain_init")
        self.phases = phases
        self.grid = int(self._chain.grid)

    def run(self, timeout_us: int = 1_000_000, stream=None) -> None:
        _check(load_library().cbk_gemv_chain_run(ctypes.byref(self._chain), timeout_us, _stream(stream)),
               "cbk_gemv_chain_run")

    def check(self) -> int:
        return int(load_library().cbk_gemv_chain_check(ctypes.byref(self._chain)))


# ---- exponent entropy-coded format (include/cbk_ec.h)

class ECTensor:
    """A tensor in the exponent entropy-coded format: code lengths, stream length and the arrays
    sm (uint8[n]), stream (uint32), gaps (uint32), bases (uint32) and lut (uint16[4096]).  Host
    numpy arrays after ``ec_encode``; ``to(device)`` gives torch tensors on the device.
    ``max_block_codes``: the most codes in one block (cbk_ec_max_block_codes), 0 if unknown."""

    def __init__(self, rows, cols, total_bits, lengths, sm, stream, gaps, bases, lut, max_block_codes=0):
        self.rows, self.cols, self.total_bits = int(rows), int(cols), int(total_bits)
        self.lengths = list(lengths)
        self.sm, self.stream, self.gaps, self.bases, self.lut = sm, stream, gaps, bases, lut
        self.max_block_codes = int(max_block_codes)

    @property
    def n(self) -> int:
        return self.rows * self.cols

    def _header(self) -> _ECHeader:
        h = _ECHeader()
        h.n, h.total_bits = self.n, self.total_bits
        for s, l in enumerate(self.lengths):
            h.lengths[s] = l
        return h

    @property
    def stored_bytes(self) -> int:
        return int(load_library().cbk_ec_stored_bytes(ctypes.byref(self._header())))

    def to(self, device) -> "ECTensor":
        import torch

        def put(a, view, pad16=False):
            a = np.ascontiguousarray(a)
            if pad16:  # the decoder may read the sm bytes up to a 16-byte boundary
                a = np.concatenate([a, np.zeros((-a.size) % 16, dtype=a.dtype)])
            return torch.from_numpy(a.view(view)).to(device)
        return ECTensor(self.rows, self.cols, self.total_bits, self.lengths, put(self.sm, np.uint8, True),
                        put(self.stream, np.int32), put(self.gaps, np.int32), put(self.bases, np.int32),
                        put(self.lut, np.int16), self.max_block_codes)

    def _struct(self) -> _ECTensor:
        def ptr(a):
            return a.data_ptr() if a.numel() else None
        return _ECTensor(self.n, self.total_bits, ptr(self.sm), ptr(self.stream), ptr(self.gaps),
                         ptr(self.bases), ptr(self.lut), self.max_block_codes)


def ec_encode(w, rows: int | None = None, cols: int | None = None) -> ECTensor:
    """Host encode (cbk_ec_plan, then cbk_ec_encode) of 16-bit patterns [rows][cols]."""
    if hasattr(w, "detach"):
        w = w.detach().contiguous().cpu().view(__import__("torch").int16).numpy()
    w = np.ascontiguousarray(w)
    if w.dtype not in (np.uint16, np.int16):
        raise TypeError("ec_encode expects 16-bit patterns")
    if rows is None:
        rows, cols = (w.shape if w.ndim == 2 else (1, w.size))
    flat = w.reshape(-1).view(np.uint16)
    if flat.size != rows * cols:
        raise ValueError("rows * cols does not match the array size")
    lib = load_library()
    h = _ECHeader()
    src = flat.ctypes.data if flat.size else None
    _check(lib.cbk_ec_plan(src, flat.size, ctypes.byref(h)), "cbk_ec_plan")
    hp = ctypes.byref(h)
    sm = np.zeros(flat.size, dtype=np.uint8)
    stream = np.zeros(int(lib.cbk_ec_stream_words(hp)), dtype=np.uint32)
    gaps = np.zeros(int(lib.cbk_ec_gap_words(hp)), dtype=np.uint32)
    bases = np.zeros(int(lib.cbk_ec_blocks(hp)), dtype=np.uint32)
    lut = np.zeros(4096, dtype=np.uint16)

    def p(a):
        return a.ctypes.data if a.size else None
    _check(lib.cbk_ec_encode(src, hp, p(sm), p(stream), p(gaps), p(bases), p(lut)), "cbk_ec_encode")
    most = int(lib.cbk_ec_max_block_codes(hp, p(bases)))
    return ECTensor(rows, cols, h.total_bits, list(h.lengths), sm, stream, gaps, bases, lut, most)


def ec_build_index(t: ECTensor, stream=None):
    """cbk_ec_build_index: the span index of a device ECTensor (a uint8 device tensor, one count per
    64-bit span of the code stream), for the one-walk ``ec_decode_bf16`` and ``ec_gemv``."""
    import torch
    lib = load_library()
    index = torch.zeros(max(16, int(lib.cbk_ec_index_bytes(t.total_bits))), dtype=torch.uint8, device=t.sm.device)
    st = t._struct()
    _check(lib.cbk_ec_build_index(ctypes.byref(st), ctypes.c_void_p(index.data_ptr()), _stream(stream)),
           "cbk_ec_build_index")
    return index


def ec_decode_bf16(t: ECTensor, out=None, stream=None, index=None):
    """GPU decode of an ECTensor on the device into a [rows][cols] torch.bfloat16 tensor; with the
    span index from ``ec_build_index``, one walk per span (cbk_ec_decode_bf16_indexed)."""
    import torch
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device=t.sm.device)
    st = t._struct()
    outp = ctypes.c_void_p(out.data_ptr() if out.numel() else None)
    lib = load_library()
    if index is None:
        _check(lib.cbk_ec_decode_bf16(ctypes.byref(st), outp, _stream(stream)), "cbk_ec_decode_bf16")
    else:
        _check(lib.cbk_ec_decode_bf16_indexed(ctypes.byref(st), ctypes.c_void_p(index.data_ptr()), outp,
                                              _stream(stream)), "cbk_ec_decode_bf16_indexed")
    return out


def ec_gemv(t: ECTensor, x, y=None, stream=None, index=None):
    """Fused decode + GEMV for an ECTensor on the device: x bfloat16[cols] -> float32[rows]; with the
    span index, one walk per span (cbk_ec_gemv_indexed)."""
    import torch
    if y is None:
        y = torch.empty(t.rows, dtype=torch.float32, device=t.sm.device)
    st = t._struct()
    xp = ctypes.c_void_p(x.data_ptr() if x.numel() else None)
    yp = ctypes.c_void_p(y.data_ptr() if y.numel() else None)
    lib = load_library()
    if index is None:
        _check(lib.cbk_ec_gemv(ctypes.byref(st), t.rows, t.cols, xp, yp, _stream(stream)), "cbk_ec_gemv")
    else:
        _check(lib.cbk_ec_gemv_indexed(ctypes.byref(st), ctypes.c_void_p(index.data_ptr()), t.rows, t.cols, xp, yp,
                                       _stream(stream)), "cbk_ec_gemv_indexed")
    return y


def _ptrs(items):
    """A ctypes array of device pointers (None for empty tensors)."""
    return (ctypes.c_void_p * len(items))(*[a.data_ptr() if a.numel() else None for a in items])


def ec_decode_group(ts, outs=None, stream=None, indexes=None):
    """cbk_ec_decode_group: several device ECTensors decoded by one launch per run of up to 8 (each
    output bit-identical to ``ec_decode_bf16``); ``indexes``: their span indexes, or None."""
    import torch
    if outs is None:
        outs = [torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device=t.sm.device) for t in ts]
    arr = (_ECTensor * len(ts))(*[t._struct() for t in ts])
    ix = _ptrs(indexes) if indexes is not None else None
    _check(load_library().cbk_ec_decode_group(arr, ix, len(ts), _ptrs(outs), _stream(stream)), "cbk_ec_decode_group")
    return outs


def ec_gemv_group(ts, x, ys=None, stream=None, indexes=None):
    """cbk_ec_gemv_group: fused decode + GEMV of several device ECTensors of equal cols that share
    x, one launch per run of up to 8; ``indexes``: their span indexes, or None."""
    import torch
    if ys is None:
        ys = [torch.empty(t.rows, dtype=torch.float32, device=t.sm.device) for t in ts]
    arr = (_ECTensor * len(ts))(*[t._struct() for t in ts])
    rows = (ctypes.c_uint64 * len(ts))(*[t.rows for t in ts])
    ix = _ptrs(indexes) if indexes is not None else None
    xp = ctypes.c_void_p(x.data_ptr() if x.numel() else None)
    _check(load_library().cbk_ec_gemv_group(arr, ix, len(ts), rows, ts[0].cols if ts else 0, xp, _ptrs(ys),
                                            _stream(stream)), "cbk_ec_gemv_group")
    return ys
