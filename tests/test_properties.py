"""Property-based CPU tests (Hypothesis): random shapes, ragged row lengths, every width b = 0..16
and distinct counts up to 65,536.

* The library's host encoder (cbk_encode) is byte-identical to the C oracle's encoding, and both
  decode back to the input (the oracle's decoder).
* On tiny inputs both equal the literal bit-string reading (oracle/oracle_ref.py).
* The size helpers agree with the definitions: b = bits_for(U), 2U + ceil(n b / 8) bytes, and the
  word count rounded up to 16 bytes.
* The capped codebook (cbk_cap_patterns) equals its oracle on random tensors and caps.
* The exponent entropy-coded encoder equals its oracle on random exponent distributions (one
  exponent to a skew the 12-bit cap binds), and its largest per-block code count matches the bases.

The derandomized profile keeps the cases fixed from run to run.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, example, given, settings
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


@st.composite
def ec_tensors(draw, max_n=30000):
    """BF16 patterns whose exponents take k distinct values with geometric frequencies (ratio r),
    random signs and mantissas: from one exponent (one-bit codes) to heavy skew and long codes."""
    k = draw(st.integers(1, 40))
    r = draw(st.floats(0.3, 1.0))
    n = draw(st.integers(0, max_n))
    seed = draw(st.integers(0, 2 ** 31))
    rng = np.random.default_rng(seed)
    exps = rng.choice(np.arange(256), size=k, replace=False)
    p = r ** np.arange(k)
    e = exps[rng.choice(k, size=n, p=p / p.sum())].astype(np.uint16)
    sm = rng.integers(0, 256, size=n).astype(np.uint16)
    w = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)
    return w.astype(np.uint16).reshape(1, n)


def _ec_example(n, k, r, seed):
    rng = np.random.default_rng(seed)
    exps = rng.choice(np.arange(256), size=k, replace=False)
    p = r ** np.arange(k)
    e = exps[rng.choice(k, size=n, p=p / p.sum())].astype(np.uint16)
    sm = rng.integers(0, 256, size=n).astype(np.uint16)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16).reshape(1, n)


def _ec_capped(k, seed):
    """k exponents with counts 2^(k-1), ..., 2, 1 (shuffled): an uncapped Huffman code would reach
    k - 1 bits, so the 12-bit cap binds."""
    rng = np.random.default_rng(seed)
    exps = rng.choice(np.arange(256), size=k, replace=False)
    e = rng.permutation(np.repeat(exps, 2 ** np.arange(k - 1, -1, -1))).astype(np.uint16)
    sm = rng.integers(0, 256, size=e.size).astype(np.uint16)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16).reshape(1, e.size)


@settings(max_examples=40, **SETTINGS)
@given(ec_tensors())
@example(_ec_example(50000, 1, 1.0, 1))      # one exponent: one-bit codes, 16,384 per full block
@example(_ec_capped(16, 2))                  # a skew that the 12-bit cap binds (65,535 weights)
@example(_ec_example(40000, 12, 0.8, 3))     # weights-like spread over several blocks
def test_entropy_encoder_equals_oracle(cbk, w):
    """The library's exponent entropy-coded encoder on random exponent distributions: the oracle's
    optimal stream length under the 12-bit cap, a prefix code (Kraft sum at most 1), every array
    byte-identical to the oracle's encoding with the same lengths, and the largest per-block code
    count (cbk_ec_max_block_codes) equal to the one the bases give."""
    from oracle import entropy as ec
    t = cbk.ec_encode(w)
    n = w.size
    assert t.total_bits == ec.encode(w).total_bits
    present = [l for l in t.lengths if l]
    assert all(1 <= l <= ec.L_MAX for l in present)
    assert sum(2.0 ** -l for l in present) <= 1.0 + 1e-12
    o = ec.encode_with_lengths(w, t.lengths)
    for a in ("sm", "stream", "gaps", "bases", "lut"):
        assert np.array_equal(getattr(t, a), getattr(o, a)), a
    want = int(np.diff(np.append(t.bases.astype(np.int64), n)).max()) if n else 0
    assert t.max_block_codes == want
