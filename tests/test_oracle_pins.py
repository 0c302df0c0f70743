"""Pins for the CPU oracle: checks against what the pages and mathematics fix, not against itself.

Sources of truth used here (none is the oracle's own code):
  * hand-worked examples in tests/golden/worked_examples.json (derivations written out there);
  * the literal pure-Python reading in oracle/oracle_ref.py, by brute-force enumeration;
  * NumPy library routines: unique (sorted distinct set), searchsorted (position), packbits with
    little bit order (LSB-first packing), int64 / float64 matrix products;
  * closed forms: identity codebook (packed words == raw 16-bit stream), byte codebook
    (packed bytes == values), b = bit_length(U - 1);
  * the pages' ranges: 12-13 bits per weight and a 10-25 % size reduction (Codebook-Quantization
    digest, "Key points" and competitor table); the DFloat11 page's observation that the BF16
    exponent carries only about 2.6 bits and the whole weight about 11 bits (section on the
    DFloat11 breakthrough), used as a sanity range for the synthetic generator.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import oracle_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _hex(vals):
    return [int(v, 16) for v in vals]


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def numpy_encode(w):
    """The format written with NumPy library routines only (independent of the C oracle)."""
    w = np.asarray(w, dtype=np.uint16).reshape(-1)
    cb = np.unique(w)
    U = cb.size
    b = 0 if U <= 1 else int(U - 1).bit_length()
    idx = np.searchsorted(cb, w).astype(np.uint64)
    if b == 0 or w.size == 0:
        return cb, U, b, np.zeros(0, dtype=np.uint32), idx
    bits = ((idx[:, None] >> np.arange(b, dtype=np.uint64)[None, :]) & 1).astype(np.uint8)
    packed = np.packbits(bits.reshape(-1), bitorder="little")
    nwords = (w.size * b + 31) // 32
    buf = np.zeros(nwords * 4, dtype=np.uint8)
    buf[:packed.size] = packed
    return cb, U, b, buf.view("<u4").astype(np.uint32), idx


# ----------------------------------------------------------------------------- worked examples
@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_worked_example_oracle(oracle_mod, ex):
    w = np.array(_hex(ex["w"]), dtype=np.uint16)
    e = oracle_mod.encode(w)
    assert e.U == ex["U"] and e.b == ex["b"]
    assert e.codebook.tolist() == _hex(ex["codebook"])
    assert e.words.tolist() == _hex(ex["words"])
    assert e.words.astype("<u4").tobytes().hex() == ex["le_bytes"]
    assert e.compressed_bytes == ex["compressed_bytes"]
    assert oracle_mod.decode(e).tolist() == w.tolist()


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_worked_example_literal(ex):
    w = _hex(ex["w"])
    cb, U, b, words = oracle_ref.encode(w)
    assert (cb, U, b) == (_hex(ex["codebook"]), ex["U"], ex["b"])
    assert words == _hex(ex["words"])
    assert oracle_ref.decode(cb, b, words, len(w)) == w
    assert oracle_ref.compressed_bytes(len(w), U) == ex["compressed_bytes"]


# ------------------------------------------------------------------------------- brute force
ALPHABET = [0x0000, 0x8000, 0x0001, 0x7F80, 0x7FC1]  # +0, -0, subnormal, +Inf, NaN payload


def test_brute_force_all_short_sequences(oracle_mod):
    """Every sequence of length <= 4 over a 5-pattern alphabet (781 tensors)."""
    count = 0
    for n in range(0, 5):
        for seq in itertools.product(ALPHABET, repeat=n):
            w = np.array(seq, dtype=np.uint16)
            e = oracle_mod.encode(w)
            cb, U, b, words = oracle_ref.encode(list(seq))
            assert e.codebook.tolist() == cb and e.U == U and e.b == b
            assert e.words.tolist() == words
            assert oracle_mod.decode(e).tolist() == list(seq)
            assert e.compressed_bytes == 2 * U + (n * b + 7) // 8
            count += 1
    assert count == 781


# ------------------------------------------------------------------- library-routine route
DISTINCT = [1, 2, 3, 4, 5, 8, 9, 17, 100, 255, 256, 257, 1000, 4096, 4097, 8192, 8193,
            16385, 32768, 32769, 65536]


@pytest.mark.parametrize("U", DISTINCT)
def test_against_numpy_route(oracle_mod, U):
    n = max(U, 3001) + (U % 7)  # odd lengths, every field straddle pattern
    w = synth.with_distinct_count(n, U, seed=[7, U])
    e = oracle_mod.encode(w)
    cb, U2, b, words, idx = numpy_encode(w)
    assert e.U == U == U2 and e.b == b
    assert np.array_equal(e.codebook, cb)
    assert np.array_equal(e.words, words)
    assert np.array_equal(oracle_mod.decode(e), w)
    # decode of a sub-range
    assert np.array_equal(oracle_mod.decode(e, 17, n - 5), w[17:n - 5])


@pytest.mark.parametrize("U", [0, 1, 2, 3, 4, 5, 7, 8, 9, 255, 256, 257, 65535, 65536])
def test_bits_for_closed_form(oracle_mod, U):
    expect = 0 if U <= 1 else int(U - 1).bit_length()
    assert oracle_mod.bits_for(U) == expect
    if U >= 2:
        assert 2 ** expect >= U > 2 ** (expect - 1)


def test_bits_transitions(oracle_mod):
    for k in range(0, 17):
        assert oracle_mod.bits_for(2 ** k) == k
        if k < 16:
            assert oracle_mod.bits_for(2 ** k + 1) == k + 1


# ------------------------------------------------------------------------------ closed forms
def test_identity_codebook_is_raw_stream(oracle_mod):
    """All 65,536 patterns present: codebook[i] = i, so b = 16 and the words are the raw stream."""
    rng = np.random.default_rng(11)
    w = np.concatenate([rng.permutation(65536), rng.integers(0, 65536, 999)]).astype(np.uint16)
    e = oracle_mod.encode(w)
    assert e.U == 65536 and e.b == 16
    assert np.array_equal(e.codebook, np.arange(65536, dtype=np.uint16))
    raw = np.zeros(e.words.size * 2, dtype=np.uint16)
    raw[:w.size] = w
    assert np.array_equal(e.words.view(np.uint16), raw)


def test_byte_codebook_is_low_bytes(oracle_mod):
    """Values 0..255 all present: index == value, b = 8, packed bytes == the values."""
    rng = np.random.default_rng(12)
    w = np.concatenate([rng.permutation(256), rng.integers(0, 256, 1001)]).astype(np.uint16)
    e = oracle_mod.encode(w)
    assert e.b == 8 and e.U == 256
    assert np.array_equal(e.words.view(np.uint8)[:w.size], w.astype(np.uint8))
    assert not e.words.view(np.uint8)[w.size:].any()


def test_padding_bits_are_zero(oracle_mod):
    for U, n in [(3, 1), (6, 11), (5000, 777), (70, 33)]:
        w = synth.with_distinct_count(n + U, U, seed=[3, U, n])[:n] if n >= U else None
        if w is None:
            w = synth.with_distinct_count(U, U, seed=[3, U])[:n]
        e = oracle_mod.encode(w)
        used = n * e.b
        if e.words.size:
            tail_bits = e.words.size * 32 - used
            last = int(e.words[-1])
            assert tail_bits < 32
            assert last >> (32 - tail_bits) == 0 if tail_bits else True


def test_corrupt_index_reading(oracle_mod):
    """An index >= U (never written by the encoder) decodes to 0x7FC0, the reading taken where the
    pages say nothing about corrupt indices."""
    e = oracle_mod.encode(np.array([0x1111, 0x2222, 0x3333, 0x1111], dtype=np.uint16))
    assert e.b == 2 and e.U == 3
    words = e.words.copy()
    words[0] |= 3 << 2  # field 1 -> index 3
    bad = oracle_mod.Encoded(e.codebook, e.U, e.b, words, e.n, e.shape)
    assert oracle_mod.decode(bad).tolist() == [0x1111, 0x7FC0, 0x3333, 0x1111]
    assert oracle_ref.decode(e.codebook.tolist(), 2, words.tolist(), 4) == [0x1111, 0x7FC0, 0x3333, 0x1111]


# ------------------------------------------------------------------ ranges from the pages
def test_gaussian_tensor_width_and_ratio(oracle_mod):
    """1024x1024 N(0, 0.02): b in 12..13 bits and a 10-25 % reduction vs raw BF16."""
    w = synth.workload_tensor(1, 0, synth.WORKLOADS[1][0][0])
    e = oracle_mod.encode(w)
    assert e.b in (12, 13)
    ratio = e.compressed_bytes / (2 * w.size)
    assert 0.75 <= ratio <= 0.90
    eff = 8 * e.compressed_bytes / w.size
    assert 11.0 <= eff <= 13.1
    assert np.array_equal(oracle_mod.decode(e), w.reshape(-1))


def test_generator_information_content():
    """Sanity of the synthetic weights against the DFloat11 page: exponent ~2.6 bits, total ~11."""
    w = synth.gaussian_bf16((1 << 20,), 0.02, seed=[2, 0, 0])

    def entropy(v):
        _, c = np.unique(v, return_counts=True)
        p = c / c.sum()
        return float(-(p * np.log2(p)).sum())

    h_exp = entropy((w >> 7) & 0xFF)
    h_all = entropy(w)
    assert 2.0 < h_exp < 3.2
    assert 9.5 < h_all < 12.0


# ---------------------------------------------------------------------------------- GEMV
def _int_bf16(vals):
    return synth.f32_to_bf16(np.asarray(vals, dtype=np.float32))


def test_gemv_integer_exact(oracle_mod):
    rng = np.random.default_rng(5)
    R, K = 37, 301
    Wi = rng.integers(-8, 8, size=(R, K))
    xi = rng.integers(-4, 5, size=K)
    e = oracle_mod.encode(_int_bf16(Wi))
    y, absb = oracle_mod.gemv(e, _int_bf16(xi))
    assert np.array_equal(y, (Wi.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64))
    assert np.array_equal(absb, np.abs(Wi * xi[None, :]).sum(1).astype(np.float64))


def test_gemv_one_hot_selects_column(oracle_mod):
    w = synth.gaussian_bf16((29, 64), 0.02, seed=[9])
    e = oracle_mod.encode(w)
    for k in (0, 13, 63):
        x = np.zeros(64, dtype=np.float32)
        x[k] = 1.0
        y, _ = oracle_mod.gemv(e, _int_bf16(x))
        assert np.array_equal(y, synth.bf16_to_f32(w[:, k]).astype(np.float64))


def test_gemv_constant_tensor(oracle_mod):
    w = np.full((5, 40), 0x4040, dtype=np.uint16)  # 3.0
    xi = np.arange(-20, 20)
    e = oracle_mod.encode(w)
    assert e.U == 1 and e.b == 0 and e.words.size == 0
    y, _ = oracle_mod.gemv(e, _int_bf16(xi))
    assert np.array_equal(y, np.full(5, 3.0 * xi.sum()))


def test_gemv_against_float64_matmul(oracle_mod):
    w = synth.student_t_bf16((64, 515), 4.0, 0.02, seed=[4])
    x = synth.activation_bf16(515, seed=[4, 1])
    e = oracle_mod.encode(w)
    y, absb = oracle_mod.gemv(e, x)
    Wf = synth.bf16_to_f32(w).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = Wf @ xf
    assert np.all(np.abs(y - ref) <= 1e-12 * absb + 1e-300)
    assert np.allclose(absb, np.abs(Wf * xf).sum(1), rtol=1e-12, atol=0)
    # selected rows agree with the full pass
    ys, _ = oracle_mod.gemv(e, x, rows=[0, 5, 63])
    assert np.array_equal(ys, y[[0, 5, 63]])


def test_gemm_rows_match_per_column_gemv(oracle_mod):
    w = synth.gaussian_bf16((33, 96), 0.02, seed=[8])
    X = synth.activations_bf16(3, 96, 8)
    e = oracle_mod.encode(w)
    Y, _ = oracle_mod.gemm(e, X)
    Xf = synth.bf16_to_f32(X).astype(np.float64)
    Wf = synth.bf16_to_f32(w).astype(np.float64)
    assert np.allclose(Y, Xf @ Wf.T, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------- planted mistakes (CPU)
def _mutant_encode(w, mutation):
    """oracle_ref.encode with one deliberate mistake, to show the pins above would catch it."""
    w = [int(v) for v in w]
    if mutation == "float_order":
        def key(v):
            f = float(synth.bf16_to_f32(np.array([v], dtype=np.uint16))[0])
            return (f, v)
        codebook = sorted(set(w), key=key)
    else:
        codebook = sorted(set(w))
    U = len(codebook)
    b = oracle_ref.bits_for(U)
    if mutation == "floor_log2_plus_one":
        b = int(math.floor(math.log2(U))) + 1 if U > 1 else 0
    pos = {v: i for i, v in enumerate(codebook)}
    digits = []
    for v in w:
        d = format(pos[v], f"0{b}b") if b else ""
        digits.append(d if mutation == "msb_first" else d[::-1])
    s = "".join(digits)
    if mutation == "drop_straddle":
        s = "".join(d if (i * b) // 32 == (i * b + b - 1) // 32 else "0" * b
                    for i, d in enumerate(digits))
    nwords = (len(s) + 31) // 32
    s = s.ljust(nwords * 32, "0")
    return codebook, U, b, [int(s[32 * k:32 * k + 32][::-1], 2) for k in range(nwords)]


@pytest.mark.parametrize("mutation", ["msb_first", "float_order", "floor_log2_plus_one",
                                      "drop_straddle"])
def test_pins_catch_planted_mistakes(mutation):
    caught = False
    for ex in _golden():
        w = _hex(ex["w"])
        cb, U, b, words = _mutant_encode(w, mutation)
        if (cb, b, words) != (_hex(ex["codebook"]), ex["b"], _hex(ex["words"])):
            caught = True
    w = synth.with_distinct_count(300, 4, seed=[1])  # U = 4, a power of two
    ncb, _, nb, nwords, _ = numpy_encode(w)
    cb, _, b, words = _mutant_encode(w.tolist(), mutation)
    if (cb, b, words) != (ncb.tolist(), nb, nwords.tolist()):
        caught = True
    assert caught, mutation
