"""CPU tests of the C ABI: the library loads, exports every declared symbol, its host encoder is
byte-identical to the oracle's encoding, and argument validation rejects bad calls before any
HIP call is made (so these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cbk():
    import fly_decode_amd
    if not os.path.exists(fly_decode_amd.library_path()):
        from fly_decode_amd import build
        build.build()
    fly_decode_amd.load_library()
    return fly_decode_amd


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(cbk_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["cbk_encode", "cbk_decode_bf16", "cbk_gemv", "cbk_gemv_group", "cbk_gemm_small", "cbk_gemm_group", "cbk_bits_for",
              "cbk_words_for", "cbk_compressed_bytes", "cbk_status_str", "cbk_encode_gpu",
              "cbk_encode_gpu_workspace_bytes", "cbk_ec_plan", "cbk_ec_encode", "cbk_ec_decode_bf16",
              "cbk_ec_spans", "cbk_ec_stream_words", "cbk_ec_gap_words", "cbk_ec_blocks",
              "cbk_ec_stored_bytes", "cbk_cap_patterns", "cbk_ec_gemv", "cbk_encode_gpu_noalloc",
              "cbk_gemv_chain_bytes", "cbk_gemv_chain_init", "cbk_gemv_chain_run", "cbk_gemv_chain_check"]:
        assert n in names


def test_library_exports_every_declared_symbol(cbk):
    lib = ctypes.CDLL(cbk.library_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_library_does_not_link_the_oracle(cbk):
    data = open(cbk.library_path(), "rb").read()
    assert b"oracle_" not in data


def test_size_helpers_match_oracle(cbk, oracle_mod):
    for U in [0, 1, 2, 3, 4, 5, 255, 256, 257, 4673, 8192, 8193, 65535, 65536]:
        assert cbk.bits_for(U) == oracle_mod.bits_for(U)
    for n in [0, 1, 7, 31, 32, 33, 1000, 1 << 20]:
        for b in range(17):
            w = oracle_mod.stream_words(n, b)
            assert cbk.words_for(n, b) == (w + 3) // 4 * 4
    assert cbk.compressed_bytes(5, 4) == 10 and cbk.compressed_bytes(12, 6) == 17
    assert cbk.compressed_bytes(7, 1) == 2 and cbk.compressed_bytes(0, 0) == 0


def _check_encode(cbk, oracle_mod, w):
    c = cbk.encode(w.reshape(1, -1) if w.ndim == 1 else w)
    e = oracle_mod.encode(w)
    assert c.U == e.U and c.b == e.b
    assert np.array_equal(c.codebook, e.codebook)
    assert np.array_equal(c.words[:e.words.size], e.words)
    assert not c.words[e.words.size:].any()
    assert c.words.size == cbk.words_for(w.size, e.b)
    assert c.compressed_bytes == e.compressed_bytes


@pytest.mark.parametrize("U", [1, 2, 3, 5, 8, 100, 257, 4097, 8193, 32769, 65536])
def test_encoder_byte_parity_distinct_counts(cbk, oracle_mod, U):
    _check_encode(cbk, oracle_mod, synth.with_distinct_count(max(U, 5003), U, seed=[21, U]))


def test_encoder_empty_and_constant(cbk):
    c = cbk.encode(np.zeros((0, 5), dtype=np.uint16))
    assert (c.U, c.b, c.words.size, c.compressed_bytes) == (0, 0, 0, 0)
    c = cbk.encode(np.full((3, 7), 0x3C00, dtype=np.uint16))
    assert (c.U, c.b, c.words.size, c.compressed_bytes) == (1, 0, 0, 2)


def test_encoder_byte_parity_cfg1(cbk, oracle_mod):
    w = synth.workload_tensor(1, 0, synth.WORKLOADS[1][0][0])
    _check_encode(cbk, oracle_mod, w)


def test_encoder_multithreaded_path(cbk, oracle_mod):
    # > 4M fields takes the threaded presence and pack passes
    w = synth.student_t_bf16((1031, 4099), 4.0, 0.02, seed=[22])
    _check_encode(cbk, oracle_mod, w)


def test_encode_capacity_and_invalid(cbk):
    lib = cbk.load_library()
    w = np.array([1, 2, 3, 4, 5], dtype=np.uint16)
    cb = np.zeros(65536, dtype=np.uint16)
    U, b, need = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint64()
    p16 = ctypes.POINTER(ctypes.c_uint16)
    p32 = ctypes.POINTER(ctypes.c_uint32)
    words = np.zeros(2, dtype=np.uint32)
    st = lib.cbk_encode(w.ctypes.data_as(p16), 5, cb.ctypes.data_as(p16), ctypes.byref(U),
                        ctypes.byref(b), words.ctypes.data_as(p32), 2, ctypes.byref(need))
    assert st == 2 and need.value == 4 and U.value == 5 and b.value == 3
    st = lib.cbk_encode(None, 5, cb.ctypes.data_as(p16), ctypes.byref(U), ctypes.byref(b), None, 0,
                        None)
    assert st == 1
    st = lib.cbk_encode(w.ctypes.data_as(p16), 5, None, ctypes.byref(U), ctypes.byref(b), None, 0,
                        None)
    assert st == 1


def _tensor(cbk, rows, cols, U, b, cb=0x1000, words=0x2000):
    return cbk._Tensor(rows, cols, U, b, cb, words)


def test_gpu_calls_validate_before_any_hip_call(cbk):
    """Every invalid argument is rejected on the host (no device is present here)."""
    lib = cbk.load_library()
    T = lambda **kw: ctypes.byref(_tensor(cbk, **{**dict(rows=4, cols=8, U=5, b=3), **kw}))
    X, Y = ctypes.c_void_p(0x4000), ctypes.c_void_p(0x8000)
    assert lib.cbk_gemv(None, X, Y, None) == 1
    assert lib.cbk_gemv(T(b=4), X, Y, None) == 1             # b != bits_for(U)
    assert lib.cbk_gemv(T(U=70000, b=17), X, Y, None) == 1   # U > 65536
    assert lib.cbk_gemv(T(U=0, b=0), X, Y, None) == 1        # empty codebook, non-empty tensor
    assert lib.cbk_gemv(T(cb=0), X, Y, None) == 1            # null codebook
    assert lib.cbk_gemv(T(words=0), X, Y, None) == 1         # null words with b > 0
    assert lib.cbk_gemv(T(words=0x2004), X, Y, None) == 3    # words not 16-byte aligned
    assert lib.cbk_gemv(T(), ctypes.c_void_p(0x4001), Y, None) == 3
    assert lib.cbk_gemv(T(), X, ctypes.c_void_p(0x8002), None) == 3
    assert lib.cbk_gemv(T(), None, Y, None) == 1
    assert lib.cbk_gemv(T(rows=1 << 40, cols=1 << 40), X, Y, None) == 1  # rows*cols overflow
    assert lib.cbk_decode_bf16(T(), None, None) == 1
    assert lib.cbk_decode_bf16(T(), ctypes.c_void_p(0x4001), None) == 3
    assert lib.cbk_gemm_small(T(), X, 8, 0, Y, 4, None) == 1      # batch 0
    assert lib.cbk_gemm_small(T(), X, 8, 17, Y, 4, None) == 1     # batch 17
    assert lib.cbk_gemm_small(T(), X, 4, 2, Y, 4, None) == 1      # ldx < cols
    assert lib.cbk_gemm_small(T(), X, 8, 2, Y, 3, None) == 1      # ldy < rows
    assert lib.cbk_gemm_small(T(), ctypes.c_void_p(0x4001), 8, 2, Y, 4, None) == 3
    # grouped GEMV: all tensors share cols; count 0 is a no-op
    arr = (cbk._Tensor * 2)(_tensor(cbk, 4, 8, 5, 3), _tensor(cbk, 4, 16, 5, 3))
    ys = (ctypes.c_void_p * 2)(0x8000, 0x9000)
    assert lib.cbk_gemv_group(arr, 2, X, ys, None) == 1            # differing cols
    assert lib.cbk_gemv_group(arr, 0, X, ys, None) == 0
    assert lib.cbk_gemv_group(None, 2, X, ys, None) == 1
    arr2 = (cbk._Tensor * 2)(_tensor(cbk, 4, 8, 5, 3), _tensor(cbk, 4, 8, 5, 4))
    assert lib.cbk_gemv_group(arr2, 2, X, ys, None) == 1           # bad b in the second tensor
    ys_bad = (ctypes.c_void_p * 2)(0x8000, 0x9002)
    assert lib.cbk_gemv_group((cbk._Tensor * 2)(_tensor(cbk, 4, 8, 5, 3), _tensor(cbk, 4, 8, 5, 3)),
                              2, X, ys_bad, None) == 3
    # grouped GEMM: shared X, per-tensor Y and leading dimension
    pair = (cbk._Tensor * 2)(_tensor(cbk, 4, 8, 5, 3), _tensor(cbk, 6, 8, 5, 3))
    ld = (ctypes.c_uint64 * 2)(4, 6)
    assert lib.cbk_gemm_group(pair, 0, X, 8, 2, ys, ld, None) == 0                # count 0: no-op
    assert lib.cbk_gemm_group(None, 2, X, 8, 2, ys, ld, None) == 1
    assert lib.cbk_gemm_group(pair, 2, X, 8, 2, ys, None, None) == 1              # null ldys
    assert lib.cbk_gemm_group(pair, 2, X, 8, 0, ys, ld, None) == 1                # batch 0
    assert lib.cbk_gemm_group(pair, 2, X, 8, 17, ys, ld, None) == 1               # batch 17
    assert lib.cbk_gemm_group(pair, 2, X, 4, 2, ys, ld, None) == 1                # ldx < cols
    assert lib.cbk_gemm_group(pair, 2, X, 8, 2, ys, (ctypes.c_uint64 * 2)(4, 5), None) == 1  # ldy < rows
    assert lib.cbk_gemm_group(arr, 2, X, 16, 2, ys, ld, None) == 1                # differing cols
    assert lib.cbk_gemm_group(pair, 2, ctypes.c_void_p(0x4001), 8, 2, ys, ld, None) == 3
    assert lib.cbk_gemm_group(pair, 2, X, 8, 2, ys_bad, ld, None) == 3            # Y not 4-byte aligned
    assert lib.cbk_gemm_group((cbk._Tensor * 2)(_tensor(cbk, 4, 8, 5, 3), _tensor(cbk, 4, 8, 5, 2)),
                              2, X, 8, 2, ys, ld, None) == 1                      # bad b
    # grouped decode: each tensor checked as by cbk_decode_bf16; count 0 is a no-op
    outs = (ctypes.c_void_p * 2)(0x8000, 0x9000)
    assert lib.cbk_decode_group(None, 0, None, None) == 0
    assert lib.cbk_decode_group(None, 2, outs, None) == 1
    assert lib.cbk_decode_group(arr2, 2, outs, None) == 1                        # bad b in the second tensor
    assert lib.cbk_decode_group(arr, 2, (ctypes.c_void_p * 2)(0x8000, None), None) == 1
    assert lib.cbk_decode_group(arr, 2, (ctypes.c_void_p * 2)(0x8000, 0x9001), None) == 3
    # zero-size tensors are accepted without work (no HIP call either)
    assert lib.cbk_gemv(T(rows=0, cols=0, U=0, b=0, cb=0, words=0), None, None, None) == 0
    assert lib.cbk_decode_bf16(T(rows=0, cols=9, U=0, b=0, cb=0, words=0), None, None) == 0


def test_gpu_encoder_validates_before_any_hip_call(cbk):
    """cbk_encode_gpu rejects bad arguments on the host (no device is present here)."""
    lib = cbk.load_library()
    # eight copies of the 65,536-bit presence bitmap
    assert lib.cbk_encode_gpu_workspace_bytes() == 8 * 2048 * 4
    W, WS, CB, WD, M = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
    cap = cbk.words_for(1000, 16)
    assert lib.cbk_encode_gpu(None, 1000, WS, CB, WD, cap, M, None) == 1          # null w
    assert lib.cbk_encode_gpu(W, 1000, None, CB, WD, cap, M, None) == 1           # null workspace
    assert lib.cbk_encode_gpu(W, 1000, WS, None, WD, cap, M, None) == 1           # null codebook
    assert lib.cbk_encode_gpu(W, 1000, WS, CB, None, cap, M, None) == 1           # null words
    assert lib.cbk_encode_gpu(W, 1000, WS, CB, WD, cap, None, None) == 1          # null meta
    assert lib.cbk_encode_gpu(ctypes.c_void_p(0x10008), 1000, WS, CB, WD, cap, M, None) == 3  # w not 16 B
    assert lib.cbk_encode_gpu(W, 1000, ctypes.c_void_p(0x20004), CB, WD, cap, M, None) == 3
    assert lib.cbk_encode_gpu(W, 1000, WS, CB, ctypes.c_void_p(0x40004), cap, M, None) == 3
    assert lib.cbk_encode_gpu(W, 1000, WS, CB, WD, cap - 1, M, None) == 2         # words_cap too small
    assert lib.cbk_encode_gpu(W, 1 << 40, WS, CB, WD, 1 << 62, M, None) == 4      # n beyond the limit


def test_gpu_encoder_group_validates_before_any_hip_call(cbk):
    """cbk_encode_gpu_group checks the array, the count and the workspace, then every job as
    cbk_encode_gpu does, before anything is launched (a failure in the last job is found)."""
    lib = cbk.load_library()
    J = cbk._EncodeJob
    cap = cbk.words_for(1000, 16)
    good = dict(w=0x10000, n=1000, codebook=0x30000, words=0x40000, words_cap=cap, meta=0x50000)

    def jobs(*ds):
        return (J * len(ds))(*[J(**d) for d in ds])
    WS = ctypes.c_void_p(0x20000)
    assert lib.cbk_encode_gpu_group(None, 1, WS, None) == 1
    assert lib.cbk_encode_gpu_group(None, 0, None, None) == 0      # no jobs: no-op
    assert lib.cbk_encode_gpu_group(jobs(good), 1, None, None) == 1
    assert lib.cbk_encode_gpu_group(jobs(good, dict(good, meta=None)), 2, WS, None) == 1
    assert lib.cbk_encode_gpu_group(jobs(good, dict(good, w=0x10008)), 2, WS, None) == 3
    assert lib.cbk_encode_gpu_group(jobs(good, dict(good, words_cap=cap - 1)), 2, WS, None) == 2
    assert lib.cbk_encode_gpu_group(jobs(good, dict(good, n=1 << 40, words_cap=1 << 62)), 2, WS, None) == 4
    assert lib.cbk_encode_gpu_group(jobs(good, good), 2, ctypes.c_void_p(0x20004), None) == 3


def test_gpu_encoder_noalloc_validates_before_any_hip_call(cbk):
    """cbk_encode_gpu_noalloc rejects bad arguments on the host, before it looks up its static
    scratch or launches anything (no device is present here)."""
    lib = cbk.load_library()
    W, CB, WD, M = (ctypes.c_void_p(a) for a in (0x10000, 0x30000, 0x40000, 0x50000))
    cap = cbk.words_for(1000, 16)
    f = lib.cbk_encode_gpu_noalloc
    assert f(None, 1000, CB, WD, cap, M, None) == 1                     # null w
    assert f(W, 1000, None, WD, cap, M, None) == 1                      # null codebook
    assert f(W, 1000, CB, None, cap, M, None) == 1                      # null words
    assert f(W, 1000, CB, WD, cap, None, None) == 1                     # null meta
    assert f(ctypes.c_void_p(0x10008), 1000, CB, WD, cap, M, None) == 3  # w not 16 B aligned
    assert f(W, 1000, CB, ctypes.c_void_p(0x40004), cap, M, None) == 3   # words not 16 B aligned
    assert f(W, 1000, ctypes.c_void_p(0x30001), WD, cap, M, None) == 3   # codebook not 2 B aligned
    assert f(W, 1000, CB, WD, cap - 1, M, None) == 2                    # words_cap too small
    assert f(W, 1 << 40, CB, WD, 1 << 62, M, None) == 4                 # n beyond the limit


def test_gemv_chain_validates_before_any_hip_call(cbk):
    """cbk_gemv_chain_init rejects bad phases and buffers on the host, and the run and check calls
    reject a missing chain, before any HIP call (no device is present here)."""
    lib = cbk.load_library()
    assert lib.cbk_gemv_chain_bytes(0) == 256
    per = lib.cbk_gemv_chain_bytes(1) - 256
    assert per > 0 and lib.cbk_gemv_chain_bytes(128) == 256 + 128 * per
    X, BUF = ctypes.c_void_p(0x4000), ctypes.c_void_p(0x100000)
    need = lib.cbk_gemv_chain_bytes(2)

    def phase(tensors, x=X, ys=None):
        arr = (cbk._Tensor * len(tensors))(*tensors)
        ys = ys or (ctypes.c_void_p * len(tensors))(*[0x8000 + 0x1000 * i for i in range(len(tensors))])
        return cbk._GemvPhase(arr, len(tensors), x, ys), (arr, ys)

    def init(phs, buf=BUF, nbytes=need):
        arr = (cbk._GemvPhase * len(phs))(*[p for p, _ in phs])
        return lib.cbk_gemv_chain_init(arr, len(phs), buf, nbytes, ctypes.byref(cbk._GemvChain()))

    good = lambda rows=4, cols=64, U=5000, b=13: _tensor(cbk, rows, cols, U, b)
    assert init([phase([good()]), phase([good()])], buf=None) == 1                      # null buffer
    assert lib.cbk_gemv_chain_init(None, 1, BUF, need, ctypes.byref(cbk._GemvChain())) == 1
    assert init([]) == 1                                                                # no phases
    assert init([phase([good()]), phase([good()], x=None)]) == 1                        # null x
    assert init([phase([good()]), phase([good(cols=64), good(cols=128)])]) == 1         # differing cols
    assert init([phase([good()]), phase([good(rows=0)])]) == 1                          # empty tensor
    assert init([phase([good()]), phase([good()] * 9)]) == 1                            # more than 8
    assert init([phase([good()]), phase([good(U=200, b=8)])]) == 4                      # b differs
    assert init([phase([good(U=40000, b=16)])]) == 4                                    # b = 16
    assert init([phase([good(cols=96)])]) == 4                                          # cols % 64
    assert init([phase([good(cols=32768 + 64)])]) == 4                                  # cols too large
    assert init([phase([good()]), phase([good()], x=ctypes.c_void_p(0x4008))]) == 3     # x not 16 B
    assert init([phase([good()], ys=(ctypes.c_void_p * 1)(0x8002))]) == 3               # y not 4 B
    assert init([phase([good()]), phase([good()])], buf=ctypes.c_void_p(0x100080)) == 3  # buffer not 256 B
    assert init([phase([good()]), phase([good()])], nbytes=need - 1) == 2               # buffer too small
    assert lib.cbk_gemv_chain_run(None, 1000, None) == 1
    assert lib.cbk_gemv_chain_run(ctypes.byref(cbk._GemvChain()), 1000, None) == 1      # never initialised
    assert lib.cbk_gemv_chain_check(None) == 1
    assert lib.cbk_status_str(6) == b"a chained launch gave up waiting"
