"""Pins for the entropy-coded format's oracle (oracle/entropy.py).

Sources of truth used here (none is the oracle's own code path being pinned):
  * a hand-worked stream in tests/golden/entropy_worked_example.json;
  * brute force over every length vector with Kraft sum <= 1 on small alphabets (optimality under
    the length cap, including cases where the cap binds);
  * the cost of an unconstrained Huffman code built with a heap, where the cap cannot bind, and a
    textbook example (frequencies 45, 13, 12, 16, 9, 5: cost 224);
  * Kraft equality and prefix-freeness of the canonical codes;
  * round trips through the bit-by-bit decoder, and span-by-span table decoding against it;
  * for the GEMV: exact integer results computed with Python integers from the known weights,
    one-hot x returning a column exactly, and the codebook oracle's float64 GEMV of the same
    weights (a different format, decoder and summation);
  * the DFloat11 article's observation (section "Przełom: DFloat11") that the BF16 exponent of
    LLM weights carries about 2.6 bits: the coded exponent of Gaussian weights costs between its
    Shannon entropy and one bit more.
"""
import json
import os
import random

import numpy as np
import pytest

import synth
from oracle import entropy as ec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "entropy_worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _cost(freq, lengths):
    return sum(int(f) * int(l) for f, l in zip(freq, lengths))


def test_worked_example_bytes():
    g = _golden()
    w = np.array([int(v, 16) for v in g["w"]], dtype=np.uint16)
    e, sm = ec.split(w)
    assert e.tolist() == g["exponents"]
    assert sm.tolist() == [int(v, 16) for v in g["sm"]]
    enc = ec.encode(w)
    want_len = {int(k): v for k, v in g["lengths"].items()}
    assert {s: l for s, l in enumerate(enc.lengths) if l} == want_len
    codes = ec.canonical_codes(enc.lengths)
    assert {s: format(c, f"0{enc.lengths[s]}b") for s, c in codes.items()} == {int(k): v for k, v in g["codes"].items()}
    assert enc.total_bits == g["total_bits"]
    assert enc.stream.tolist() == [int(v, 16) for v in g["stream"]]
    assert enc.gaps.tolist() == [int(v, 16) for v in g["gaps"]]
    assert enc.bases.tolist() == g["bases"]
    for k, v in g["lut_samples"].items():
        assert int(enc.lut[int(k)]) == int(v, 16), k
    assert np.array_equal(ec.decode(enc), w)


@pytest.mark.parametrize("seed", range(40))
def test_lengths_optimal_under_the_cap_by_brute_force(seed):
    rng = random.Random(seed)
    n = rng.randint(2, 6)
    lmax = rng.randint(max(2, (n - 1).bit_length()), 5)
    freq = [0] * 16
    for s in rng.sample(range(16), n):
        freq[s] = rng.choice([1, 1, 2, 3, 5, 8, 13, 40, 100, 1000])
    lengths = ec.optimal_lengths(freq, lmax)
    assert max(lengths) <= lmax
    assert all((l > 0) == (f > 0) for l, f in zip(lengths, freq))
    assert sum(2.0 ** -l for l in lengths if l) <= 1.0
    assert _cost(freq, lengths) == ec.brute_force_cost(freq, lmax)


@pytest.mark.parametrize("seed", range(10))
def test_lengths_equal_huffman_cost_when_the_cap_cannot_bind(seed):
    rng = np.random.default_rng(seed)
    n = 20
    freq = np.zeros(256, dtype=np.int64)
    freq[rng.choice(256, n, replace=False)] = rng.integers(1, 10 ** 6, n)
    # a code over n symbols never needs more than n - 1 bits
    lengths = ec.optimal_lengths(freq, n - 1)
    assert _cost(freq, lengths) == ec.huffman_cost(freq)


def test_textbook_huffman_example():
    freq = [45, 13, 12, 16, 9, 5]
    assert ec.huffman_cost(freq) == 224
    lengths = ec.optimal_lengths(freq, 12)
    assert _cost(freq, lengths) == 224
    assert lengths[0] == 1 and sorted(lengths[1:4]) == [3, 3, 3] and sorted(lengths[4:]) == [4, 4]


def test_cap_binds_on_fibonacci_frequencies():
    fib = [1, 1]
    while len(fib) < 20:
        fib.append(fib[-1] + fib[-2])
    freq = fib + [0] * (256 - 20)
    assert ec.optimal_lengths(freq, 19)[0] == 19   # unconstrained: a 19-bit code
    lengths = ec.optimal_lengths(freq, 12)
    assert max(lengths) == 12
    assert sum(2.0 ** -l for l in lengths if l) == 1.0
    assert _cost(freq, lengths) >= ec.huffman_cost(freq)


@pytest.mark.parametrize("seed", range(8))
def test_codes_complete_and_prefix_free(seed):
    rng = np.random.default_rng(100 + seed)
    freq = np.zeros(256, dtype=np.int64)
    k = int(rng.integers(2, 200))
    freq[rng.choice(256, k, replace=False)] = rng.geometric(0.01, k)
    lengths = ec.optimal_lengths(freq)
    assert sum(2.0 ** -l for l in lengths if l) == 1.0
    codes = ec.canonical_codes(lengths)
    words = [format(c, f"0{lengths[s]}b") for s, c in codes.items()]
    for a in words:
        for b in words:
            assert a == b or not b.startswith(a)


def _roundtrip(w):
    enc = ec.encode(w)
    assert np.array_equal(ec.decode(enc), np.asarray(w, dtype=np.uint16).reshape(-1))
    return enc


def test_roundtrip_gaussian_weights():
    w = synth.gaussian_bf16((50000,), 0.02, seed=[7, 1])
    _roundtrip(w)


@pytest.mark.parametrize("case", ["one", "constant", "two_values", "all_exponents", "specials"])
def test_roundtrip_edge_cases(case):
    rng = np.random.default_rng(5)
    if case == "one":
        w = np.array([0x3F80], dtype=np.uint16)
    elif case == "constant":
        w = np.full(1000, 0xC2F7, dtype=np.uint16)
    elif case == "two_values":
        w = rng.choice(np.array([0x3F80, 0x4000], dtype=np.uint16), 777)
    elif case == "all_exponents":
        w = rng.permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16)
    else:
        w = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16), 3000)
    enc = _roundtrip(w)
    if case in ("one", "constant"):
        assert enc.total_bits == w.size     # one exponent value: a 1-bit code
    if case == "all_exponents":
        assert sum(1 for l in enc.lengths if l) == 256 and max(enc.lengths) <= ec.L_MAX


def test_empty():
    enc = ec.encode(np.zeros(0, dtype=np.uint16))
    assert enc.total_bits == 0 and enc.stream.size == 0 and enc.gaps.size == 0 and enc.bases.size == 0
    assert ec.decode(enc).size == 0


@pytest.mark.parametrize("seed", range(3))
def test_spans_decode_on_their_own(seed):
    """Each span decoded from its gap with the table gives exactly the codes that start in it,
    and every block base counts the codes before the block."""
    rng = np.random.default_rng(seed)
    # a heavier tail than the workloads (long codes, spans that start mid-code)
    w = synth.student_t_bf16((40000,), 2.0, 0.02, seed=[8, seed])
    enc = ec.encode(w)
    e, _ = ec.split(w)
    lens = np.array(enc.lengths)[e]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    got = []
    counts = []
    for j in range(enc.spans):
        s = ec.decode_span(enc, j)
        lo, hi = j * ec.SPAN_BITS, (j + 1) * ec.SPAN_BITS
        want = e[(starts >= lo) & (starts < hi)]
        assert s == want.tolist(), j
        got += s
        counts.append(len(s))
    assert got == e.tolist()
    cum = np.concatenate([[0], np.cumsum(counts)])
    assert enc.bases.tolist() == [int(cum[k * ec.BLOCK_SPANS]) for k in range(enc.blocks)]
    assert max(enc.lengths) > 8   # the tail reached long codes


def test_table_agrees_with_bit_by_bit_codes():
    w = synth.gaussian_bf16((20000,), 0.02, seed=[9])
    enc = ec.encode(w)
    codes = ec.canonical_codes(enc.lengths)
    for s, c in codes.items():
        l = enc.lengths[s]
        bits = [(c >> (l - 1 - k)) & 1 for k in range(l)]   # first bit first
        field = sum(b << k for k, b in enumerate(bits))
        for hi in {0, min(1, (1 << (12 - l)) - 1), (1 << (12 - l)) - 1}:
            assert int(enc.lut[field | (hi << l)]) == s | (l << 8)


def test_exponent_cost_between_entropy_and_one_more_bit():
    w = synth.gaussian_bf16((1 << 20,), 0.02, seed=[10])
    e, _ = ec.split(w)
    p = np.bincount(e, minlength=256) / e.size
    h = float(-(p[p > 0] * np.log2(p[p > 0])).sum())
    enc = ec.encode(w)
    avg = enc.total_bits / e.size
    assert h <= avg < h + 1
    # the DFloat11 article's ~2.6 bits for LLM exponents; Gaussian synthetic weights land nearby
    assert 2.0 < avg < 3.2


def _int_patterns(values):
    """BF16 bit patterns of small integers (exact in BF16)."""
    return synth.f32_to_bf16(np.asarray(values, dtype=np.float32))


@pytest.mark.parametrize("rows,cols", [(7, 40), (33, 9), (1, 128)])
def test_gemv_integer_data_exact(rows, cols):
    """Integer weights in [-8, 7] and x in [-4, 4]: every product and partial sum is an integer far
    below 2^53, so the float64 result equals the Python-integer dot product exactly."""
    rng = np.random.default_rng(rows * 1000 + cols)
    wi = rng.integers(-8, 8, size=(rows, cols))
    xi = rng.integers(-4, 5, size=cols)
    y, absb = ec.gemv(ec.encode(_int_patterns(wi)), rows, cols, _int_patterns(xi))
    for r in range(rows):
        assert y[r] == sum(int(a) * int(b) for a, b in zip(wi[r], xi))
        assert absb[r] == sum(abs(int(a)) * abs(int(b)) for a, b in zip(wi[r], xi))


def test_gemv_one_hot_returns_a_column():
    rows, cols = 12, 50
    w = synth.gaussian_bf16((rows, cols), 0.02, seed=[91])
    for k in (0, 17, cols - 1):
        x = np.zeros(cols, dtype=np.uint16)
        x[k] = 0x3F80  # 1.0
        y, _ = ec.gemv(ec.encode(w), rows, cols, x)
        assert np.array_equal(y, synth.bf16_to_f32(w[:, k]).astype(np.float64))


def test_gemv_agrees_with_the_codebook_oracle(oracle_mod):
    """The same Gaussian weights through the codebook format's C oracle: both are float64 sums of
    exact products, so they agree to rounding (1e-12 of sum|W x|)."""
    rows, cols = 64, 300
    w = synth.gaussian_bf16((rows, cols), 0.02, seed=[92])
    x = synth.activation_bf16(cols, seed=[93])
    y, absb = ec.gemv(ec.encode(w), rows, cols, x)
    ref, ref_abs = oracle_mod.gemv(oracle_mod.encode(w), x)
    assert np.all(np.abs(y - ref) <= 1e-12 * ref_abs)
    assert np.allclose(absb, ref_abs, rtol=1e-12, atol=0)


def test_gemv_pin_catches_a_transposed_reshape():
    """A planted mistake (the decoded weights read as [cols][rows] and transposed) fails the
    integer pin."""
    rows, cols = 5, 8
    rng = np.random.default_rng(94)
    wi = rng.integers(-8, 8, size=(rows, cols))
    xi = rng.integers(-4, 5, size=cols)
    enc = ec.encode(_int_patterns(wi))

    def wrong(enc, rows, cols, x):
        w = ec.decode(enc).reshape(cols, rows).T
        wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xf = (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return wf @ xf
    y = wrong(enc, rows, cols, _int_patterns(xi))
    exact = np.array([sum(int(a) * int(b) for a, b in zip(wi[r], xi)) for r in range(rows)])
    assert not np.array_equal(y, exact)
