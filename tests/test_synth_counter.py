"""CPU tests of the counter-based BF16 Gaussian generator (synth/counter.py) that the 7B- and
70B-shaped step workloads use: the host (numpy) and torch implementations agree bit for bit, the
uniform stage is SplitMix64 as published, and the BF16 values follow N(0, sigma)."""
import json
import os

import numpy as np
import pytest
from scipy.special import ndtr, ndtri

import synth
from synth import counter

HERE = os.path.dirname(os.path.abspath(__file__))


def test_splitmix64_reference_outputs():
    g = json.load(open(os.path.join(HERE, "golden", "splitmix64.json")))
    x, got = g["state"], []
    for _ in g["outputs_hex"]:
        x = (x + counter.GAMMA) & counter.M64
        got.append(f"{counter._mix_int(x):016x}")
    assert got == g["outputs_hex"]


def _uniform_np(key, start, count):
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    z = np.uint64(key) + n * np.uint64(counter.GAMMA)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(counter.MIX1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(counter.MIX2)
    return z ^ (z >> np.uint64(31))


def test_vectorised_stream_equals_the_scalar_definition():
    key = counter.key_of([5, 3, 6])
    vec = _uniform_np(key, 1000, 50)
    for i, v in enumerate(vec):
        assert int(v) == counter._mix_int(key + (1000 + i + 1) * counter.GAMMA)


@pytest.mark.parametrize("seed,sigma", [([4, 0, 0], 0.02), ([5, 79, 6], 0.015), ([5, 2, 4], 1.0)])
def test_numpy_and_torch_cpu_agree_bit_for_bit(seed, sigma):
    key = counter.key_of(seed)
    for start, count in [(0, 70001), (123456789, 4097), (2**35 + 3, 1000)]:
        a = counter.gaussian_bf16_np(key, start, count, sigma)
        b = counter.gaussian_bf16_torch(key, start, count, sigma, "cpu", chunk=30000).numpy().view(np.uint16)
        assert np.array_equal(a, b)


def test_host_threads_and_rows_are_slices_of_one_stream():
    t = synth.WORKLOADS[5][0][1]  # k: 1024 x 8192
    key = counter.key_of([5, 1, t.tensor_id])
    whole = counter.gaussian_bf16_host(key, 0, 64 * t.cols, t.scale, threads=4, chunk=10007)
    assert np.array_equal(whole, counter.gaussian_bf16_np(key, 0, 64 * t.cols, t.scale))
    rows = synth.workload_rows(5, 1, t, [0, 7, 63])
    assert np.array_equal(rows, whole.reshape(64, t.cols)[[0, 7, 63]])


def test_table_interpolation_tracks_the_normal_quantile():
    """For random 52-bit m, the generator's magnitude (before scaling) is -PhiInv((2m+1)/2^54)
    to within 1e-6: the cell index and position are exact and the cells are narrow."""
    z0, dz = counter.table()
    rng = np.random.default_rng(5)
    m = rng.integers(0, 2**52, size=20000, dtype=np.uint64)
    m[:4] = [0, 1, 2**51, 2**52 - 1]
    v = (m * np.uint64(2) + np.uint64(1)).astype(np.float64)
    mant, ex = np.frexp(v)
    g = (mant * 2.0 - 1.0) * 256
    j = np.floor(g)
    cell = (ex.astype(np.int64) - 1) * 256 + j.astype(np.int64)
    mag = z0[cell] + dz[cell] * (g - j)
    exact = -ndtri(v * 2.0**-54)
    assert np.max(np.abs(mag - exact)) < 1e-6
    assert mag.min() > 0 and abs(mag.max() - (-ndtri(2.0**-54))) < 1e-9


def test_bf16_values_follow_the_normal_distribution():
    """Frequencies of the BF16 values of 4M draws against the probability mass of each value's
    rounding interval under N(0, sigma) (a chi-square over bins with enough expected mass), plus
    the sign balance and the tail beyond 4 sigma."""
    sigma = 0.015
    w = counter.gaussian_bf16_host(counter.key_of([9, 9, 9]), 0, 1 << 22, sigma)
    vals, counts = np.unique(w, return_counts=True)
    f = synth.bf16_to_f32(vals).astype(np.float64)
    order = np.argsort(f)
    f, counts = f[order], counts[order]
    # rounding interval of each BF16 value: halfway to its neighbours (RNE ties do not matter
    # here); the neighbours come from the bit patterns, one unit in the last place either side
    pat = synth.f32_to_bf16(f.astype(np.float32)).astype(np.int32)
    nxt = synth.bf16_to_f32(np.where(f >= 0, pat + 1, pat - 1).astype(np.uint16)).astype(np.float64)
    prv = synth.bf16_to_f32(np.where(f > 0, pat - 1, pat + 1).astype(np.uint16)).astype(np.float64)
    prv = np.where(vals[order] == 0x8000, 0.0, prv)
    prv = np.where(vals[order] == 0x0000, 0.0, prv)
    a = np.minimum(prv, nxt)
    b = np.maximum(prv, nxt)
    left = (f + a) / 2
    right = (f + b) / 2
    p = ndtr(right / sigma) - ndtr(left / sigma)
    n = w.size
    expected = p * n
    keep = expected > 50
    chi2 = np.sum((counts[keep] - expected[keep]) ** 2 / expected[keep])
    dof = int(keep.sum()) - 1
    assert chi2 < dof + 6 * np.sqrt(2 * dof), (chi2, dof)
    neg = np.count_nonzero(w & 0x8000)
    assert abs(neg - n / 2) < 5 * np.sqrt(n / 4)
    tail = np.count_nonzero(np.abs(synth.bf16_to_f32(w)) > 4 * sigma)
    pt = 2 * ndtr(-4.0)
    assert abs(tail - pt * n) < 6 * np.sqrt(pt * n) + 2
