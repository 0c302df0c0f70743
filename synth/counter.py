"""A counter-based N(0, sigma) BF16 generator that gives the same bits on the host (numpy) and on
a GPU (torch), for workloads too large to draw on the host in a benchmark run (a 70B-shaped decode
step is 68 billion weights).

Weight i of a tensor is a pure function of the tensor's key and i, so any row of any tensor can be
regenerated on the host, alone, to check a GPU result.  Every step is exact integer arithmetic,
an exact float64 operation, a table lookup, or one IEEE-rounded float64 multiply or add, so numpy
and torch (CPU or GPU) produce identical bits:

1. Uniform bits: the SplitMix64 generator (Steele, Lea and Flood, "Fast splittable pseudorandom
   number generators", OOPSLA 2014).  Its n-th output (n = 1, 2, ...) for state s is
   mix(s + n * 0x9E3779B97F4A7C15 mod 2^64) with mix(z) = z ^ (z >> 30); z *= 0xBF58476D1CE4E5B9;
   z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.  Weight i takes output n = i + 1.  A seed
   sequence (s_1, s_2, ...) becomes the state by folding: k <- mix(k + 0x9E3779B97F4A7C15 + s_j),
   starting from k = 0.
2. Sign and tail probability: the top bit of the output is the sign; its low 52 bits m give
   p = (2m + 1) / 2^54, a value in (0, 1/2) that float64 holds exactly.
3. Magnitude |z| = -PhiInv(p) (PhiInv = the standard normal quantile): p's binade 2^(e-55) (e from
   frexp of 2m + 1) is cut into 256 equal cells; within a cell |z| is interpolated linearly between
   the quantiles at the cell's ends, which are tabulated once in float64 (scipy's ndtri).  The cell
   index and the position t in [0, 1) inside it are exact; |z| = z0 + dz * t (a rounded multiply,
   then a rounded add).  The interpolation error is below 3e-7 standard deviations, far under the
   BF16 resolution, and |z| reaches 8.3 (p = 2^-54).
4. Weight: float64 |z| * sigma (rounded), the sign applied, converted to float32 (round to
   nearest even), then to BF16 by round-to-nearest-even on the float32 bits.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
M64 = (1 << 64) - 1
CELLS_PER_BINADE = 256
BINADES = 53  # frexp exponents 1..53 of the odd integers 2m + 1 < 2^53

_TABLE = None


def _mix_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def key_of(seed) -> int:
    """The 64-bit SplitMix64 state for a seed sequence (a sequence of non-negative ints)."""
    k = 0
    for s in (seed if hasattr(seed, "__iter__") else [seed]):
        k = _mix_int(k + GAMMA + int(s))
    return k


def table():
    """(z0, dz) float64 arrays over the BINADES * 256 cells: the magnitude -PhiInv(p) at each cell's
    left end and its change to the right end."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        e = np.arange(1, BINADES + 1, dtype=np.float64)[:, None]
        j = np.arange(CELLS_PER_BINADE + 1, dtype=np.float64)[None, :]
        p = np.ldexp(1.0 + j / CELLS_PER_BINADE, (e - 55).astype(np.int64))
        zq = -ndtri(p)                                   # [BINADES, 257] magnitudes, decreasing in p
        z0 = np.ascontiguousarray(zq[:, :-1]).reshape(-1)
        dz = np.ascontiguousarray(zq[:, 1:] - zq[:, :-1]).reshape(-1)
        _TABLE = (z0, dz)
    return _TABLE


def _f32_bits_to_bf16_np(f32: np.ndarray) -> np.ndarray:
    u = f32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def gaussian_bf16_np(key: int, start: int, count: int, sigma: float) -> np.ndarray:
    """Weights start .. start + count - 1 of the stream with SplitMix64 state `key`, as BF16 bit
    patterns (numpy uint16)."""
    z0t, dzt = table()
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + n * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    z ^= z >> np.uint64(31)
    neg = (z >> np.uint64(63)).astype(bool)
    v = ((z & np.uint64((1 << 52) - 1)) * np.uint64(2) + np.uint64(1)).astype(np.float64)  # exact
    mant, ex = np.frexp(v)                       # v = mant * 2^ex, mant in [0.5, 1), ex in 1..53
    g = (mant * 2.0 - 1.0) * CELLS_PER_BINADE    # exact: fraction bits of v scaled to the cells
    j = np.floor(g)
    t = g - j                                    # exact
    cell = (ex.astype(np.int64) - 1) * CELLS_PER_BINADE + j.astype(np.int64)
    mag = z0t[cell] + dzt[cell] * t              # one rounded multiply, one rounded add
    val = mag * np.float64(sigma)
    val = np.where(neg, -val, val).astype(np.float32)
    return _f32_bits_to_bf16_np(val)


def gaussian_bf16_torch(key: int, start: int, count: int, sigma: float, device, out=None, chunk=1 << 25):
    """The same weights as ``gaussian_bf16_np`` computed with torch on `device`, as an int16 tensor
    of BF16 bit patterns (written into `out` when given).  Works in chunks of `chunk` weights."""
    import torch

    def s64(c):  # a uint64 constant as the int64 with the same bits
        return c - (1 << 64) if c >= (1 << 63) else c

    def lsr(x, k):  # logical shift right of int64 bit patterns
        return torch.bitwise_and(torch.bitwise_right_shift(x, k), (1 << (64 - k)) - 1)

    z0t, dzt = table()
    z0d = torch.from_numpy(z0t).to(device)
    dzd = torch.from_numpy(dzt).to(device)
    if out is None:
        out = torch.empty(count, dtype=torch.int16, device=device)
    keyd = s64(key)
    for c0 in range(0, count, chunk):
        c1 = min(count, c0 + chunk)
        n = torch.arange(start + c0 + 1, start + c1 + 1, dtype=torch.int64, device=device)
        z = n * s64(GAMMA) + keyd                 # wraps mod 2^64 like the uint64 arithmetic
        del n
        z = torch.bitwise_xor(z, lsr(z, 30)) * s64(MIX1)
        z = torch.bitwise_xor(z, lsr(z, 27)) * s64(MIX2)
        z = torch.bitwise_xor(z, lsr(z, 31))
        neg = z < 0
        v = (torch.bitwise_and(z, (1 << 52) - 1) * 2 + 1).to(torch.float64)
        del z
        mant, ex = torch.frexp(v)
        del v
        g = (mant * 2.0 - 1.0) * float(CELLS_PER_BINADE)
        del mant
        j = torch.floor(g)
        t = g - j
        del g
        cell = (ex.to(torch.int64) - 1) * CELLS_PER_BINADE + j.to(torch.int64)
        del ex, j
        mag = torch.add(z0d[cell], torch.mul(dzd[cell], t))
        del cell, t
        val = torch.mul(mag, float(sigma))
        del mag
        val = torch.where(neg, -val, val).to(torch.float32)
        del neg
        u = torch.bitwise_and(val.view(torch.int32).to(torch.int64), 0xFFFFFFFF)
        del val
        h = torch.bitwise_right_shift(u + 0x7FFF + torch.bitwise_and(torch.bitwise_right_shift(u, 16), 1), 16)
        out[c0:c1] = h.to(torch.int32).to(torch.int16)
        del u, h
    return out


def gaussian_bf16_host(key: int, start: int, count: int, sigma: float, threads: int = 0,
                       chunk: int = 1 << 20) -> np.ndarray:
    """``gaussian_bf16_np`` over a long range, in chunks spread over host threads (numpy releases
    the interpreter lock inside its array operations)."""
    import concurrent.futures as cf
    import os
    out = np.empty(count, dtype=np.uint16)
    spans = [(c0, min(count, c0 + chunk)) for c0 in range(0, count, chunk)]

    def run(span):
        c0, c1 = span
        out[c0:c1] = gaussian_bf16_np(key, start + c0, c1 - c0, sigma)

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(spans) <= 1:
        for s in spans:
            run(s)
    else:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, spans))
    return out
