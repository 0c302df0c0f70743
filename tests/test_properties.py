"""Property-based CPU tests (Hypothesis): random shapes, ragged row lengths, every width b = 0..16
and distinct counts up to 65,536.

* The library's host encoder (cbk_encode) is byte-identical to the C oracle's encoding, and both
  decode back to the input (the oracle's decoder).
* On tiny inputs both equal the literal bit-string reading (oracle/oracle_ref.py).
* The size helpers agree with the definitions: b = bits_for(U), 2U + ceil(n b / 8) bytes, and the
  word count rounded up to 16 bytes.
* The capped codebook (cbk_cap_patterns) equals its oracle on random tensors and caps.

The derandomized profile keeps the cases fixed from run to run.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import synth
from oracle import oracle_ref

SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(scope="module")
def cbk():
    import os
    import fly_decode_amd
    if not os.path.exists(fly_decode_amd.library_path()):
        from fly_decode_amd import build
        build.build()
    fly_decode_amd.load_library()
    return fly_decode_amd


@st.composite
def tensors(draw, max_n=40000):
    """(patterns [rows][cols], U): a width b in 0..16, a distinct count U of that width, a shape
    with at least U weights (cols need not be a multiple of anything)."""
    b = draw(st.integers(0, 16))
    U = 1 if b == 0 else draw(st.integers(2 ** (b - 1) + 1, 2 ** b))
    n_min = max(U, 1)
    n = draw(st.integers(n_min, max(n_min, min(max_n, 4 * U + 64))))
    cols = draw(st.integers(1, n))
    rows = -(-n // cols)
    seed = draw(st.integers(0, 2 ** 31))
    w = synth.with_distinct_count(rows * cols, min(U, rows * cols), seed=[seed])
    return w.reshape(rows, cols), U


@settings(max_examples=60, **SETTINGS)
@given(tensors())
def test_encoder_equals_oracle_and_round_trips(cbk, oracle_mod, wt):
    w, U = wt
    c = cbk.encode(w)
    e = oracle_mod.encode(w)
    assert (c.U, c.b) == (e.U, e.b) == (U, oracle_mod.bits_for(U))
    assert np.array_equal(c.codebook, e.codebook)
    nw = oracle_mod.stream_words(w.size, e.b)
    assert np.array_equal(c.words[:nw], e.words[:nw])
    assert not np.any(c.words[nw:])  # the 16-byte padding is zero
    stream_words = (w.size * e.b + 31) // 32
    assert c.words.size == cbk.words_for(w.size, e.b) == (stream_words + 3) // 4 * 4
    assert c.compressed_bytes == 2 * U + (w.size * e.b + 7) // 8
    assert np.array_equal(oracle_mod.decode(e).reshape(w.shape), w)


@settings(max_examples=150, **SETTINGS)
@given(st.lists(st.integers(0, 0xFFFF), min_size=0, max_size=24))
def test_tiny_inputs_equal_the_literal_reading(cbk, oracle_mod, vals):
    w = np.asarray(vals, dtype=np.uint16)
    cb, U, b, words = oracle_ref.encode(vals)
    c = cbk.encode(w.reshape(1, -1) if w.size else w.reshape(0, 1))
    e = oracle_mod.encode(w)
    assert (c.U, c.b) == (e.U, e.b) == (U, b)
    assert list(c.codebook) == list(e.codebook) == cb
    nw = len(words)
    assert [int(v) for v in c.words[:nw]] == [int(v) for v in e.words[:nw]] == words
    assert oracle_ref.decode(cb, b, words, len(vals)) == [int(v) for v in vals]


@settings(max_examples=200, **SETTINGS)
@given(st.integers(0, 65536), st.integers(0, 1 << 34))
def test_size_helpers(cbk, U, n):
    b = cbk.bits_for(U)
    assert b == (0 if U <= 1 else (U - 1).bit_length())
    assert cbk.compressed_bytes(n, U) == 2 * U + (n * b + 7) // 8 == oracle_ref.compressed_bytes(n, U)
    assert cbk.words_for(n, b) == ((n * b + 31) // 32 + 3) // 4 * 4


@settings(max_examples=40, **SETTINGS)
@given(st.integers(1, 3000), st.integers(1, 600), st.integers(0, 2 ** 31))
def test_capped_codebook_equals_oracle(cbk, K, distinct, seed):
    from oracle import capped
    n = max(distinct, 2000)
    w = synth.with_distinct_count(n, distinct, seed=[seed], exponents=synth.finite_exponents(distinct))
    got, U = cbk.cap_patterns(w, K)
    ref = capped.cap(w, K)
    assert np.array_equal(got, ref)
    assert U == len(np.unique(ref)) == min(distinct, K)
