"""CPU oracle for codebook-compressed BF16 weights (TEST INFRASTRUCTURE ONLY).

The plain C reference in ``cbk_oracle.c`` is loaded through ctypes from ``oracle/_build``.
Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may use this
package; the HIP library and its Python binding never import it.  ``build()`` compiles the C
file with gcc.  ``oracle_ref`` is a second, literal pure-Python reading for tiny inputs.

Parity pins for these functions live in ``tests/test_oracle_pins.py``; every function here is
pinned by at least one of: hand-worked examples, brute-force enumeration against the literal
reading, NumPy library routines (unique / searchsorted / packbits / float64 dot), closed forms
(identity codebook, byte codebook), and exact integer GEMV results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cbk_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libcbk_oracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no vector ISA flags)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                        "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_bits_for.restype = ctypes.c_uint32
        lib.oracle_bits_for.argtypes = [ctypes.c_uint32]
        lib.oracle_stream_words.restype = ctypes.c_uint64
        lib.oracle_stream_words.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        lib.oracle_encode.restype = ctypes.c_int
        lib.oracle_encode.argtypes = [_u16p, ctypes.c_uint64, _u16p, _u32p, _u32p, _u32p,
                                      ctypes.c_uint64]
        lib.oracle_decode_range.restype = None
        lib.oracle_decode_range.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u32p,
                                            ctypes.c_uint64, ctypes.c_uint64, _u16p]
        lib.oracle_gemv_rows.restype = None
        lib.oracle_gemv_rows.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u32p,
                                         ctypes.c_uint64, _u16p, ctypes.c_uint64, ctypes.c_uint64,
                                         _f64p, _f64p]
        lib.oracle_gemm_rows.restype = None
        lib.oracle_gemm_rows.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u32p,
                                         ctypes.c_uint64, _u16p, ctypes.c_uint64, ctypes.c_uint32,
                                         ctypes.c_uint64, ctypes.c_uint64, _f64p, _f64p,
                                         ctypes.c_uint64]
        _lib = lib
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


class Encoded:
    """The oracle's encoding of one tensor: sorted codebook, U, b and the packed words."""

    def __init__(self, codebook, U, b, words, n, shape):
        self.codebook, self.U, self.b, self.words, self.n = codebook, U, b, words, n
        self.shape = shape

    @property
    def compressed_bytes(self) -> int:
        """Two bytes per codebook entry plus ceil(n*b/8) bytes of packed indices."""
        return 2 * self.U + (self.n * self.b + 7) // 8


def bits_for(U: int) -> int:
    return int(_load().oracle_bits_for(U))


def stream_words(n: int, b: int) -> int:
    return int(_load().oracle_stream_words(n, b))


def encode(w) -> Encoded:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    shape = w.shape
    flat = w.reshape(-1)
    n = flat.size
    cb = np.zeros(65536, dtype=np.uint16)
    words = np.zeros(max(1, (n * 16 + 31) // 32), dtype=np.uint32)
    U = ctypes.c_uint32(0)
    b = ctypes.c_uint32(0)
    rc = _load().oracle_encode(_p(flat, _u16p), n, _p(cb, _u16p), ctypes.byref(U), ctypes.byref(b),
                               _p(words, _u32p), words.size)
    if rc != 0:
        raise RuntimeError("oracle_encode failed")
    nw = stream_words(n, b.value)
    return Encoded(cb[:U.value].copy(), U.value, b.value, words[:nw].copy(), n, shape)


def _cb_words(e: Encoded):
    cb = np.ascontiguousarray(e.codebook, dtype=np.uint16)
    if cb.size == 0:
        cb = np.zeros(1, dtype=np.uint16)
    words = np.ascontiguousarray(e.words, dtype=np.uint32)
    if words.size == 0:
        words = np.zeros(1, dtype=np.uint32)
    return cb, words


def decode(e: Encoded, i0: int = 0, i1: int | None = None) -> np.ndarray:
    """Weights [i0, i1) of the flat tensor as 16-bit patterns."""
    i1 = e.n if i1 is None else i1
    out = np.zeros(i1 - i0, dtype=np.uint16)
    cb, words = _cb_words(e)
    if i1 > i0:
        _load().oracle_decode_range(_p(cb, _u16p), e.U, e.b, _p(words, _u32p), i0, i1,
                                    _p(out, _u16p))
    return out


def gemv(e: Encoded, x, rows=None):
    """(y, absb) in float64 for the listed rows (all rows by default) of W[rows][cols] . x.

    absb[r] = sum_k |W[r][k] x[k]|, the scale of the per-element tolerance."""
    R, K = e.shape
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
    assert x.size == K
    cb, words = _cb_words(e)
    y = np.zeros(R, dtype=np.float64)
    absb = np.zeros(R, dtype=np.float64)
    lib = _load()
    spans = [(0, R)] if rows is None else [(int(r), int(r) + 1) for r in rows]
    xx = x if x.size else np.zeros(1, dtype=np.uint16)
    for r0, r1 in spans:
        lib.oracle_gemv_rows(_p(cb, _u16p), e.U, e.b, _p(words, _u32p), K, _p(xx, _u16p), r0, r1,
                             _p(y, _f64p), _p(absb, _f64p))
    if rows is None:
        return y, absb
    idx = np.asarray(rows, dtype=np.int64)
    return y[idx], absb[idx]


def gemv_rows_into(e: Encoded, x, r0: int, r1: int, y: np.ndarray, absb: np.ndarray):
    """Raw row-range call (used by the CPU baseline to split rows over threads)."""
    R, K = e.shape
    cb, words = _cb_words(e)
    _load().oracle_gemv_rows(_p(cb, _u16p), e.U, e.b, _p(words, _u32p), K, _p(x, _u16p), r0, r1,
                             _p(y, _f64p), _p(absb, _f64p))


def gemm(e: Encoded, X, rows=None):
    """(Y, absb) in float64, shape [batch][len(rows)] (all rows by default)."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    ys, bs = [], []
    for j in range(X.shape[0]):
        y, a = gemv(e, X[j], rows)
        ys.append(y)
        bs.append(a)
    return np.stack(ys), np.stack(bs)
