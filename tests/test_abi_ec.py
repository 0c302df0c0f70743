"""CPU tests of the exponent entropy-coded format's C ABI (include/cbk_ec.h): the library's host
encoder writes exactly the oracle's bytes, its code lengths are optimal under the 12-bit cap, and
the GPU decode rejects bad arguments before any HIP call (no GPU is needed here)."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import entropy as ec


@pytest.fixture(scope="module")
def cbk():
    import os
    import fly_decode_amd
    if not os.path.exists(fly_decode_amd.library_path()):
        from fly_decode_amd import build
        build.build()
    fly_decode_amd.load_library()
    return fly_decode_amd


def _inputs():
    rng = np.random.default_rng(3)
    return {
        "gaussian_300x777": synth.gaussian_bf16((300, 777), 0.02, seed=[11]),
        "t2_heavy_tail": synth.student_t_bf16((200, 1000), 2.0, 0.02, seed=[12]),
        "t4_workload_like": synth.student_t_bf16((64, 4096), 4.0, 0.02, seed=[13]),
        "constant": np.full((10, 100), 0x3F80, dtype=np.uint16),
        "two_exponents": rng.choice(np.array([0x3F80, 0x4012], dtype=np.uint16), (7, 13)),
        "every_pattern": rng.permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16).reshape(256, 256),
        "specials": rng.choice(np.array([0x7F80, 0xFF80, 0x7FC1, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16), (9, 111)),
        "one": np.array([[0xC2F7]], dtype=np.uint16),
    }


@pytest.mark.parametrize("name", list(_inputs()))
def test_host_encoder_matches_oracle(cbk, name):
    w = _inputs()[name]
    t = cbk.ec_encode(w)
    # optimal under the cap: the same stream length as the oracle's own package-merge lengths
    ref = ec.encode(w)
    assert t.total_bits == ref.total_bits
    assert max(t.lengths) <= ec.L_MAX
    # given the library's lengths, every array equals the oracle's encoding byte for byte
    o = ec.encode_with_lengths(w, t.lengths)
    for a in ("sm", "stream", "gaps", "bases", "lut"):
        assert np.array_equal(getattr(t, a), getattr(o, a)), a
    assert t.stored_bytes == o.stored_bytes
    assert np.array_equal(ec.decode(o), w.reshape(-1)) if w.size <= 70000 else True


def test_empty_tensor(cbk):
    t = cbk.ec_encode(np.zeros((0, 5), dtype=np.uint16))
    assert t.total_bits == 0 and t.stream.size == 0 and t.gaps.size == 0 and t.bases.size == 0
    assert t.lut.size == 4096


def _hdr(cbk, n, total_bits, lengths):
    h = cbk._ECHeader()
    h.n, h.total_bits = n, total_bits
    for s, l in lengths.items():
        h.lengths[s] = l
    return h


def test_encode_rejects_a_header_that_does_not_describe_w(cbk):
    lib = cbk.load_library()
    w = np.array([0x3F80, 0x4000, 0x3F80], dtype=np.uint16)   # exponents 127, 128, 127
    buf = [np.zeros(64, dtype=np.uint8), np.zeros(16, dtype=np.uint32), np.zeros(16, dtype=np.uint32),
           np.zeros(16, dtype=np.uint32), np.zeros(4096, dtype=np.uint16)]
    ptrs = [b.ctypes.data for b in buf]
    ok = _hdr(cbk, 3, 3, {127: 1, 128: 1})
    assert lib.cbk_ec_encode(w.ctypes.data, ctypes.byref(ok), *ptrs) == 0
    assert lib.cbk_ec_encode(w.ctypes.data, ctypes.byref(_hdr(cbk, 3, 4, {127: 1, 128: 1})), *ptrs) == 1  # wrong length sum
    assert lib.cbk_ec_encode(w.ctypes.data, ctypes.byref(_hdr(cbk, 3, 2, {127: 1})), *ptrs) == 1          # 128 has no code
    assert lib.cbk_ec_encode(w.ctypes.data, ctypes.byref(_hdr(cbk, 3, 39, {127: 13, 128: 13})), *ptrs) == 1  # above 12
    assert lib.cbk_ec_encode(w.ctypes.data, ctypes.byref(_hdr(cbk, 3, 3, {127: 1, 128: 1, 5: 1})), *ptrs) == 1  # Kraft > 1
    assert lib.cbk_ec_encode(None, ctypes.byref(ok), *ptrs) == 1
    assert lib.cbk_ec_plan(None, 5, ctypes.byref(ok)) == 1
    assert lib.cbk_ec_plan(w.ctypes.data, 1 << 32, ctypes.byref(ok)) == 4


def test_decode_validates_before_any_hip_call(cbk):
    lib = cbk.load_library()
    T = cbk._ECTensor
    A = 0x10000   # 16-byte aligned stand-ins; nothing is dereferenced on these paths
    good = dict(n=1000, total_bits=3000, sm=A, stream=A, gaps=A, bases=A, lut=A)

    def call(out=A, **kw):
        d = dict(good)
        d.update(kw)
        return lib.cbk_ec_decode_bf16(ctypes.byref(T(**d)), ctypes.c_void_p(out), None)
    assert lib.cbk_ec_decode_bf16(None, ctypes.c_void_p(A), None) == 1
    assert call(n=0, sm=None, stream=None, gaps=None, bases=None, lut=None, out=0) == 0   # empty: no-op
    assert call(n=1 << 32, total_bits=1 << 33) == 4
    for k in ("sm", "stream", "gaps", "bases", "lut"):
        assert call(**{k: None}) == 1, k
    assert call(out=0) == 1
    assert call(total_bits=999) == 1            # fewer bits than weights
    assert call(total_bits=12001) == 1          # more than 12 bits per weight
    for k in ("sm", "stream", "gaps", "bases", "lut"):
        assert call(**{k: A + 8}) == 3, k
    assert call(out=A + 2) == 3


def test_size_helpers(cbk):
    lib = cbk.load_library()
    for bits in [0, 1, 63, 64, 65, 64 * 256, 64 * 256 + 1, 10 ** 7]:
        h = _hdr(cbk, max(1, bits // 3), bits, {})
        spans = (bits + 63) // 64
        assert lib.cbk_ec_spans(ctypes.byref(h)) == spans
        assert lib.cbk_ec_stream_words(ctypes.byref(h)) == 2 * spans
        assert lib.cbk_ec_gap_words(ctypes.byref(h)) == (spans + 7) // 8
        assert lib.cbk_ec_blocks(ctypes.byref(h)) == (spans + 255) // 256


def test_gemv_validates_before_any_hip_call(cbk):
    """cbk_ec_gemv rejects bad arguments on the host (no device is present here)."""
    lib = cbk.load_library()
    T = cbk._ECTensor
    A = 0x10000   # 16-byte aligned stand-ins; nothing is dereferenced on these paths

    def call(n=6400, rows=100, cols=64, x=A, y=A, none=False):
        t = T(n=n, total_bits=3 * n, sm=A, stream=A, gaps=A, bases=A, lut=A)
        return lib.cbk_ec_gemv(None if none else ctypes.byref(t), rows, cols, ctypes.c_void_p(x),
                               ctypes.c_void_p(y), None)
    assert call(none=True) == 1
    assert call(rows=99) == 1                        # rows * cols != n
    assert call(x=0) == 1 and call(y=0) == 1
    assert call(n=6400, rows=200, cols=32) == 4      # fewer than 64 columns
    assert call(n=6000, rows=100, cols=60) == 4      # columns not a multiple of 8
    assert call(x=A + 2) == 3 and call(y=A + 2) == 3
    assert call(n=0, rows=0, cols=64, x=0, y=0) == 0  # nothing to do
    assert call(n=0, rows=8, cols=0, x=0, y=0) == 1   # rows to write need y, even with no columns


def test_span_index_calls_validate_before_any_hip_call(cbk):
    """cbk_ec_build_index and the indexed decode and GEMV reject bad arguments on the host, with the
    same codes as the calls without the index plus a missing or misaligned index."""
    lib = cbk.load_library()
    T = cbk._ECTensor
    A = 0x10000   # 16-byte aligned stand-ins; nothing is dereferenced on these paths
    for bits in [0, 1, 64, 65, 64 * 16, 64 * 16 + 1]:
        spans = (bits + 63) // 64
        assert lib.cbk_ec_index_bytes(bits) == (spans + 15) // 16 * 16
    t = T(n=1000, total_bits=3000, sm=A, stream=A, gaps=A, bases=A, lut=A)
    v = ctypes.c_void_p
    assert lib.cbk_ec_build_index(None, v(A), None) == 1
    assert lib.cbk_ec_build_index(ctypes.byref(t), None, None) == 1
    assert lib.cbk_ec_build_index(ctypes.byref(t), v(A + 1), None) == 3
    assert lib.cbk_ec_build_index(ctypes.byref(T(n=1000, total_bits=999, sm=A, stream=A, gaps=A, bases=A, lut=A)),
                                  v(A), None) == 1
    assert lib.cbk_ec_build_index(ctypes.byref(T(n=0, total_bits=0)), None, None) == 0   # empty: no-op
    assert lib.cbk_ec_decode_bf16_indexed(ctypes.byref(t), None, v(A), None) == 1
    assert lib.cbk_ec_decode_bf16_indexed(ctypes.byref(t), v(A + 8), v(A), None) == 3
    assert lib.cbk_ec_decode_bf16_indexed(ctypes.byref(t), v(A), None, None) == 1
    assert lib.cbk_ec_decode_bf16_indexed(ctypes.byref(t), v(A), v(A + 2), None) == 3
    g = T(n=6400, total_bits=3 * 6400, sm=A, stream=A, gaps=A, bases=A, lut=A)
    assert lib.cbk_ec_gemv_indexed(ctypes.byref(g), None, 100, 64, v(A), v(A), None) == 1
    assert lib.cbk_ec_gemv_indexed(ctypes.byref(g), v(A + 4), 100, 64, v(A), v(A), None) == 3
    assert lib.cbk_ec_gemv_indexed(ctypes.byref(g), v(A), 99, 64, v(A), v(A), None) == 1
    assert lib.cbk_ec_gemv_indexed(ctypes.byref(g), v(A), 200, 32, v(A), v(A), None) == 4


def test_group_calls_validate_before_any_hip_call(cbk):
    """cbk_ec_decode_group and cbk_ec_gemv_group check every tensor as the single calls do, plus
    the arrays and the count, before anything is launched (a failure in the last tensor returns
    its code with nothing enqueued; no device is present here)."""
    lib = cbk.load_library()
    T = cbk._ECTensor
    A = 0x10000   # 16-byte aligned stand-ins; nothing is dereferenced on these paths
    P = ctypes.c_void_p
    good = dict(n=1000, total_bits=3000, sm=A, stream=A, gaps=A, bases=A, lut=A)

    def arr(*ds):
        return (T * len(ds))(*[T(**d) for d in ds])

    def ptrs(*vs):
        return (P * len(vs))(*vs)
    ts = arr(good, good, dict(good, lut=None))
    assert lib.cbk_ec_decode_group(ts, None, 3, ptrs(A, A, A), None) == 1          # last tensor without its table
    assert lib.cbk_ec_decode_group(arr(good, good), None, 2, ptrs(A, A + 2), None) == 3   # misaligned output
    assert lib.cbk_ec_decode_group(arr(good, good), ptrs(A, None), 2, ptrs(A, A), None) == 1  # an index missing
    assert lib.cbk_ec_decode_group(arr(good, good), ptrs(A, A + 8), 2, ptrs(A, A), None) == 3  # misaligned index
    assert lib.cbk_ec_decode_group(None, None, 0, None, None) == 0                  # no tensors: no-op
    assert lib.cbk_ec_decode_group(None, None, 1, ptrs(A), None) == 1
    assert lib.cbk_ec_decode_group(arr(good), None, 1, None, None) == 1
    assert lib.cbk_ec_decode_group(arr(dict(n=0, total_bits=0)), None, 1, ptrs(None), None) == 0  # empty: no-op
    assert lib.cbk_ec_decode_group(arr(good, dict(good, n=1 << 32, total_bits=1 << 33)), None, 2, ptrs(A, A), None) == 4

    g = dict(n=6400, total_bits=3 * 6400, sm=A, stream=A, gaps=A, bases=A, lut=A)
    R = ctypes.c_uint64 * 2
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(100, 99), 64, P(A), ptrs(A, A), None) == 1   # rows * cols != n
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(100, 100), 64, P(A), ptrs(A, A + 2), None) == 3  # misaligned y
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(100, 100), 64, P(A + 8), ptrs(A, A), None) == 3  # misaligned x
    assert lib.cbk_ec_gemv_group(arr(g, g), ptrs(A, None), 2, R(100, 100), 64, P(A), ptrs(A, A), None) == 1
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(200, 200), 32, P(A), ptrs(A, A), None) == 4   # cols < 64
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, None, 64, P(A), ptrs(A, A), None) == 1
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(100, 100), 64, P(A), None, None) == 1
    assert lib.cbk_ec_gemv_group(None, None, 0, None, 64, None, None, None) == 0  # no tensors: no-op
    assert lib.cbk_ec_gemv_group(arr(g, g), None, 2, R(100, 100), 64, None, ptrs(A, A), None) == 1  # no x


def test_max_block_codes_and_its_check(cbk):
    """cbk_ec_max_block_codes is the largest per-block code count that bases gives (the last block
    counted up to n), 0 for an empty tensor; a tensor claiming more than a block can hold (16,384)
    is rejected before any HIP call."""
    import synth
    lib = cbk.load_library()
    rng = np.random.default_rng(9)
    cases = [synth.gaussian_bf16((300, 777), 0.02, seed=[91]),
             rng.choice(np.array([0x3F80, 0x4012], dtype=np.uint16), (1, 64 * 256 * 3 + 11)),
             np.full((10, 1000), 0x3F80, dtype=np.uint16), np.array([[0x3F80]], dtype=np.uint16)]
    for w in cases:
        t = cbk.ec_encode(w)
        want = int(np.diff(np.append(t.bases.astype(np.int64), w.size)).max())
        assert t.max_block_codes == want, (w.shape, t.max_block_codes, want)
    assert cbk.ec_encode(np.zeros((0, 8), dtype=np.uint16)).max_block_codes == 0
    assert lib.cbk_ec_max_block_codes(None, None) == 0
    T = cbk._ECTensor
    A = 0x10000
    bad = T(n=1000, total_bits=3000, sm=A, stream=A, gaps=A, bases=A, lut=A, max_block_codes=16385)
    assert lib.cbk_ec_decode_bf16(ctypes.byref(bad), ctypes.c_void_p(A), None) == 1
    ok = T(n=1000, total_bits=3000, sm=A, stream=A, gaps=A, bases=A, lut=A, max_block_codes=16384)
    assert lib.cbk_ec_decode_bf16_indexed(ctypes.byref(ok), None, ctypes.c_void_p(A), None) == 1  # (no index)
