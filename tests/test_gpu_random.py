"""Seeded random sweep of the GPU calls against the oracle, through the C ABI.

48 cases, each drawn from its own fixed seed:
* an index width b from 1 to 16, with a distinct count U of that width;
* rows from 1 to 300 (more when the tensor needs them to hold U distinct values);
* cols from 1 to 2199, every third case a multiple of 64 (the fast kernels), the rest ragged (the
  generic kernels);
* a batch from 1 to 16.

For each case:
* the standalone decode gives back every weight exactly;
* the GEMV and the GEMM at the drawn batch are within 1e-3 * sum|W x| of the oracle on every
  element;
* a grouped GEMV and GEMM of the tensor with a second one of other rows and the same cols (every
  fourth case of another width, so the group splits into runs of equal b) give each tensor's
  single-call result bit for bit.

Weights are drawn over an exponent range around 1.0 (finite, no overflow in fp32 sums); x and X are
N(0, 1) in BF16.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 1e-3
CASES = 48


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


def _distinct_for(rng, b):
    if b == 16:
        return int(rng.integers(32769, 40001))  # keeps the exponent range inside fp32 sums
    return int(rng.integers(2 ** (b - 1) + 1, 2 ** b + 1))


def _case(i):
    rng = np.random.default_rng([61, i])
    b = int(rng.integers(1, 17))
    U = _distinct_for(rng, b)
    cols = 64 * int(rng.integers(1, 35)) if i % 3 == 0 else int(rng.integers(1, 2200))
    rows = max(int(rng.integers(1, 301)), -(-U // cols))
    batch = int(rng.integers(1, 17))
    rows2 = max(int(rng.integers(1, 301)), -(-U // cols))
    b2 = b if i % 4 else int(rng.integers(1, 17))
    U2 = U if b2 == b else _distinct_for(rng, b2)
    rows2 = max(rows2, -(-U2 // cols))
    return b, U, rows, cols, batch, U2, rows2


def _weights(U, rows, cols, seed):
    return synth.with_distinct_count(rows * cols, U, seed=seed,
                                     exponents=synth.finite_exponents(U)).reshape(rows, cols)


def _up(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


def _within(got, ref, absb, what):
    err = np.abs(got - ref)
    assert np.all(err <= TOL * absb), f"{what}: max err/bound {np.max(err / np.maximum(TOL * absb, 1e-300))}"


@pytest.mark.parametrize("i", range(CASES))
def test_random_case(env, oracle_mod, i):
    torch, cbk = env
    b, U, rows, cols, batch, U2, rows2 = _case(i)
    print(f"case {i}: b {b} U {U} {rows}x{cols} batch {batch}; second tensor {rows2} rows, U {U2}", flush=True)
    w = _weights(U, rows, cols, [62, i])
    c = cbk.encode(w)
    assert (c.U, c.b) == (U, b)
    d = c.to("cuda")
    e = oracle_mod.encode(w)

    out = cbk.decode_bf16(d)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), w)

    x = synth.activation_bf16(cols, [63, i])
    y = cbk.gemv(d, _up(torch, x)).cpu().numpy().astype(np.float64)
    ref, absb = oracle_mod.gemv(e, x)
    _within(y, ref, absb, "gemv")

    X = synth.activations_bf16(batch, cols, 64 + i)
    Y = cbk.gemm_small(d, _up(torch, X)).cpu().numpy().astype(np.float64)
    refm, absm = oracle_mod.gemm(e, X)
    _within(Y, refm, absm, f"gemm batch {batch}")

    # grouped calls: each tensor's result equals its single call
    d2 = cbk.encode(_weights(U2, rows2, cols, [65, i])).to("cuda")
    xd, Xd = _up(torch, x), _up(torch, X)
    ys = cbk.gemv_group([d, d2], xd)
    Ys = cbk.gemm_group([d, d2], Xd)
    singles = [cbk.gemv(t, xd) for t in (d, d2)]
    singles_m = [cbk.gemm_small(t, Xd) for t in (d, d2)]
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(ys[k], singles[k]), f"grouped gemv, tensor {k}"
        assert torch.equal(Ys[k], singles_m[k]), f"grouped gemm, tensor {k}"
