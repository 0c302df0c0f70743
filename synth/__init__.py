"""Seeded synthetic BF16 weight tensors and activation vectors.

This module is the only code shared by the CPU oracle's tests and the HIP path's tests and
benchmark.  It holds none of the codebook method's arithmetic: it draws random numbers,
rounds them to BF16 bit patterns, and names the workload shapes.  Everything it returns is a
plain ``numpy.uint16`` array of BF16 bit patterns (or float32 for convenience views).

Workloads (stand-ins for the real checkpoints the pages measure on, which are not available):
a Llama-7B-shaped attention projection, a Llama-7B-shaped MLP pair with heavy-tailed values,
a full 7B-shaped decode step and a 70B-shaped decode step, plus a small 1024x1024 case.
Gaussian weights are N(0, sigma) drawn in float32 and rounded to BF16 by round-to-nearest-even;
heavy-tailed weights are Student-t with nu = 4, scaled by 0.02.  Activations are N(0, 1) BF16.

Seeds: ``numpy.random.default_rng([cfg_id, layer, tensor_id])`` for weights and
``default_rng([cfg_id, 1000 + length, column])`` for activation vectors.  The two decode-step
workloads (the 7B- and 70B-shaped steps, 6.5 and 68 billion weights) are too large to draw on the
host in a benchmark run: their N(0, sigma) weights come from the counter-based generator in
``synth.counter`` with state ``counter.key_of([cfg_id, layer, tensor_id])``, which gives the same
bits from numpy on the host (any single row on its own) and from torch on a GPU.
"""
from __future__ import annotations

import numpy as np

from . import counter

__all__ = [
    "f32_to_bf16", "bf16_to_f32", "gaussian_bf16", "student_t_bf16", "activation_bf16",
    "activations_bf16", "from_alphabet", "with_distinct_count", "finite_exponents", "WORKLOADS", "Workload",
    "workload_tensor", "workload_x", "workload_rows", "workload_tensor_device", "counter",
]


def f32_to_bf16(a) -> np.ndarray:
    """Round float32 values to BF16 bit patterns, round-to-nearest-even; NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_to_f32(h) -> np.ndarray:
    """The float32 value of BF16 bit patterns (exact: BF16 is the top half of float32)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(shape, sigma: float, seed) -> np.ndarray:
    """N(0, sigma) drawn in float32 (PCG64 ``standard_normal``), scaled in float32, rounded to BF16."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(sigma)
    return f32_to_bf16(v)


def student_t_bf16(shape, nu: float, scale: float, seed) -> np.ndarray:
    """Student-t(nu) drawn in float64, scaled, cast to float32, rounded to BF16."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_t(nu, size=shape) * scale).astype(np.float32)
    return f32_to_bf16(v)


def activation_bf16(length: int, seed) -> np.ndarray:
    """One activation vector x ~ N(0, 1) in BF16."""
    return gaussian_bf16((length,), 1.0, seed)


def activations_bf16(batch: int, length: int, cfg_id: int) -> np.ndarray:
    """A [batch][length] activation matrix; row j uses seed [cfg_id, 1000 + length, j]."""
    return np.stack([activation_bf16(length, [cfg_id, 1000 + length, j]) for j in range(batch)])


def from_alphabet(n: int, alphabet, seed) -> np.ndarray:
    """n draws (uniform, with replacement) from a list of 16-bit patterns."""
    rng = np.random.default_rng(seed)
    alphabet = np.asarray(alphabet, dtype=np.uint16)
    return alphabet[rng.integers(0, len(alphabet), size=n)]


def with_distinct_count(n: int, distinct: int, seed, exponents=None) -> np.ndarray:
    """n patterns holding exactly ``distinct`` different 16-bit values (needs n >= distinct).

    The distinct values are a random subset of all 65,536 patterns, or, with
    ``exponents=(lo, hi)``, of the finite normal BF16 patterns whose biased exponent lies in
    [lo, hi) (2 * (hi - lo) * 128 candidates, both signs).  Every value appears at least once and
    the order is shuffled.
    """
    if distinct > n or distinct > 65536:
        raise ValueError("need n >= distinct and distinct <= 65536")
    rng = np.random.default_rng(seed)
    if exponents is not None:
        lo, hi = exponents
        if not 1 <= lo < hi <= 255:
            raise ValueError("exponents must lie in [1, 255)")
        exps = np.arange(lo, hi, dtype=np.uint32)
        mags = (exps[:, None] << 7 | np.arange(128, dtype=np.uint32)[None, :]).ravel()
        pool = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        if distinct > len(pool):
            raise ValueError(f"the exponent range holds only {len(pool)} patterns")
    else:
        pool = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    values = rng.choice(pool, size=distinct, replace=False)
    picks = np.concatenate([np.arange(distinct), rng.integers(0, distinct, size=n - distinct)])
    rng.shuffle(picks)
    return values[picks].astype(np.uint16)


def finite_exponents(distinct: int):
    """An exponent range around 1.0 wide enough for ``distinct`` finite normal BF16 values."""
    half = max(8, -(-distinct // 512))  # 256 patterns per exponent (two signs x 128 mantissas)
    return (127 - half, 127 + half)


class Workload:
    """One weight tensor shape of a workload: name, rows (out features), cols (in features);
    dist is "normal" (PCG64 draws), "t4" (PCG64 Student-t) or "normal_ctr" (the counter-based
    generator)."""

    def __init__(self, name: str, rows: int, cols: int, dist: str, scale: float, tensor_id: int):
        self.name, self.rows, self.cols = name, rows, cols
        self.dist, self.scale, self.tensor_id = dist, scale, tensor_id

    def __repr__(self):
        return f"Workload({self.name}, {self.rows}x{self.cols}, {self.dist}({self.scale}))"


def _layer(shapes, dist, scale):
    return [Workload(n, r, c, dist, scale, i) for i, (n, r, c) in enumerate(shapes)]


# cfg_id -> (per-layer tensor list, layer count)
WORKLOADS = {
    1: (_layer([("w", 1024, 1024)], "normal", 0.02), 1),
    2: (_layer([("attn", 4096, 4096)], "normal", 0.02), 1),
    3: (_layer([("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)], "t4", 0.02), 1),
    4: (_layer([("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)], "normal_ctr", 0.02), 32),
    5: (_layer([("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
                ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)], "normal_ctr", 0.015), 80),
}


def workload_tensor(cfg_id: int, layer: int, tensor: Workload) -> np.ndarray:
    """The seeded [rows][cols] BF16 weight tensor of one workload entry."""
    seed = [cfg_id, layer, tensor.tensor_id]
    shape = (tensor.rows, tensor.cols)
    if tensor.dist == "normal":
        return gaussian_bf16(shape, tensor.scale, seed)
    if tensor.dist == "t4":
        return student_t_bf16(shape, 4.0, tensor.scale, seed)
    if tensor.dist == "normal_ctr":
        return counter.gaussian_bf16_host(counter.key_of(seed), 0, tensor.rows * tensor.cols,
                                          tensor.scale).reshape(shape)
    raise ValueError(tensor.dist)


def workload_rows(cfg_id: int, layer: int, tensor: Workload, rows) -> np.ndarray:
    """The listed rows of a workload tensor, [len(rows)][cols] BF16, generated on their own when
    the tensor comes from the counter-based generator (else sliced from the whole tensor)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    if tensor.dist != "normal_ctr":
        return np.ascontiguousarray(workload_tensor(cfg_id, layer, tensor)[rows])
    key = counter.key_of([cfg_id, layer, tensor.tensor_id])
    out = np.empty((rows.size, tensor.cols), dtype=np.uint16)
    for i, r in enumerate(rows):
        out[i] = counter.gaussian_bf16_np(key, int(r) * tensor.cols, tensor.cols, tensor.scale)
    return out


def workload_tensor_device(cfg_id: int, layer: int, tensor: Workload, device, out=None):
    """A workload tensor as a flat int16 torch tensor of BF16 patterns on `device`: computed there
    by the counter-based generator, or drawn on the host and copied for the PCG64 workloads."""
    import torch
    n = tensor.rows * tensor.cols
    if tensor.dist == "normal_ctr":
        return counter.gaussian_bf16_torch(counter.key_of([cfg_id, layer, tensor.tensor_id]), 0, n,
                                           tensor.scale, device, out=out)
    w = torch.from_numpy(workload_tensor(cfg_id, layer, tensor).reshape(-1).view(np.int16))
    if out is None:
        return w.to(device)
    out.copy_(w)
    return out


def workload_x(cfg_id: int, length: int, batch: int = 1) -> np.ndarray:
    """Seeded activations for a workload: shape [batch][length] BF16."""
    return activations_bf16(batch, length, cfg_id)
