"""GPU parity of the GEMV chain (cbk_gemv_chain_*): dependent grouped GEMV phases run by one
persistent cooperative launch, through the C ABI.

* A chain that takes every row-loop shape of the kernel (one, two and three wave steps per row, a
  one-unit row, rows claimed dynamically, groups of one to three tensors, tensors with fewer rows
  than the grid has waves): every output equals the single-launch cbk_gemv_group result bit for
  bit, and sampled rows (first and last included) are within 1e-3 * sum|W x| of the oracle.
* Runs repeat: three runs with the outputs clobbered in between give the same bits.
* The bounded barrier wait: a run whose waits may not last at all (timeout 0) ends, reports
  CBK_E_TIMEOUT, and the next run with a normal limit completes with the full results.
* One layer of the 7B- and 70B-shaped steps as bench.py builds them: the chain equals the
  per-phase launches bit for bit.
* Other index widths (b = 1, 4, 8, 15) on a three-phase chain: bit-equal to the single launches,
  within tolerance of the oracle.

The oracle's inputs are the same host patterns, encoded by the oracle itself.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 1e-3
CBK_E_TIMEOUT = 6


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


# (tensor shapes of the phase, seed): K = 4096 (one step per row), 8192 (two), 11008 (three, the
# general loop), 1024 with 16,500 rows (rows claimed dynamically), 64 (a one-unit row)
PHASES = [
    ([(300, 4096), (1024, 4096), (77, 4096)], 1),
    ([(513, 8192)], 2),
    ([(700, 11008)], 3),
    ([(16500, 1024)], 4),
    ([(2, 4096), (6000, 4096)], 5),
    ([(6000, 64)], 6),
]
DISTINCT = 5000  # every tensor b = 13


@pytest.fixture(scope="module")
def chain_case(env):
    torch, cbk = env
    phases, host = [], []
    for shapes, seed in PHASES:
        ws = [synth.with_distinct_count(r * c, DISTINCT, [41, seed, i],
                                        exponents=synth.finite_exponents(DISTINCT)).reshape(r, c)
              for i, (r, c) in enumerate(shapes)]
        x = synth.activation_bf16(shapes[0][1], [42, seed])
        ds = [cbk.encode(w).to("cuda") for w in ws]
        assert all(d.b == 13 for d in ds)
        xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        ys = [torch.full((d.rows,), float("nan"), dtype=torch.float32, device="cuda") for d in ds]
        phases.append((ds, xd, ys))
        host.append((ws, x))
    print(f"chain of {len(phases)} phases", flush=True)
    chain = cbk.GemvChain(phases)
    return chain, phases, host


def _outputs(torch, phases):
    torch.cuda.synchronize()
    return [[y.cpu().numpy().copy() for y in ys] for _, _, ys in phases]


def test_chain_equals_single_launches_and_oracle(env, oracle_mod, chain_case):
    torch, cbk = env
    chain, phases, host = chain_case
    chain.run()
    got = _outputs(torch, phases)
    assert chain.check() == 0
    for p, ((ds, xd, _), (ws, x)) in enumerate(zip(phases, host)):
        single = cbk.gemv_group(ds, xd)
        torch.cuda.synchronize()
        for i, (d, s, w) in enumerate(zip(ds, single, ws)):
            assert np.array_equal(got[p][i], s.cpu().numpy()), f"phase {p} tensor {i}: differs from cbk_gemv_group"
            rng = np.random.default_rng([p, i])
            rows = np.unique(np.concatenate([[0, d.rows - 1], rng.choice(d.rows, min(d.rows, 40), replace=False)]))
            ref, absb = oracle_mod.gemv(oracle_mod.encode(w[rows]), x)
            err = np.abs(got[p][i][rows] - ref)
            assert np.all(err <= TOL * absb), f"phase {p} tensor {i}: max err/bound {np.max(err / (TOL * absb))}"


def test_chain_runs_repeat(env, chain_case):
    torch, cbk = env
    chain, phases, _ = chain_case
    chain.run()
    first = _outputs(torch, phases)
    for rep in range(3):
        for _, _, ys in phases:
            for y in ys:
                y.fill_(float("nan"))
        chain.run()
        again = _outputs(torch, phases)
        assert chain.check() == 0
        for p in range(len(phases)):
            for i in range(len(first[p])):
                assert np.array_equal(first[p][i], again[p][i]), f"run {rep}: phase {p} tensor {i} changed"


def test_chain_wait_limit_reports_and_recovers(env, chain_case):
    """A zero limit makes every workgroup that has to wait at a barrier give up at once: the run
    still ends, the failure is reported, and the next run (which clears the barrier state) is
    complete."""
    torch, cbk = env
    chain, phases, _ = chain_case
    chain.run()
    want = _outputs(torch, phases)
    for _, _, ys in phases:
        for y in ys:
            y.fill_(float("nan"))
    chain.run(timeout_us=0)
    torch.cuda.synchronize()
    assert chain.check() == CBK_E_TIMEOUT
    chain.run()
    got = _outputs(torch, phases)
    assert chain.check() == 0
    for p in range(len(phases)):
        for i in range(len(want[p])):
            assert np.array_equal(want[p][i], got[p][i])


@pytest.mark.parametrize("workload", ["llama7b", "l70b_b1"])
def test_chain_step_layer_equals_phase_launches(env, workload):
    """One layer of the step workload: the chain (as bench.py --launch chain runs it) gives the
    per-phase launches' outputs bit for bit."""
    torch, cbk = env
    import bench
    print(f"chain of one layer of {workload}", flush=True)
    work = bench.Workload(workload, layers=1)
    work.step()
    want = [y.cpu().numpy().copy() for y in work.ys]
    for y in work.ys:
        y.fill_(float("nan"))
    work.make_chain()
    work.run_chain()
    torch.cuda.synchronize()
    assert work.chain.check() == 0
    for i, y in enumerate(work.ys):
        assert np.array_equal(y.cpu().numpy(), want[i]), f"{work.specs[i][2].name}: chain differs"


@pytest.mark.parametrize("distinct", [2, 9, 200, 20000])  # b = 1, 4, 8, 15
def test_chain_other_widths(env, oracle_mod, distinct):
    """A three-phase chain (K = 1024, 4096 and 5120: one, one and two wave steps per row) at other
    index widths: equal to cbk_gemv_group bit for bit and to the oracle within tolerance."""
    torch, cbk = env
    shapes = [[(700, 1024), (64, 1024)], [(300, 4096)], [(257, 5120)]]
    phases, host = [], []
    for p, group in enumerate(shapes):
        ws = [synth.with_distinct_count(r * c, distinct, [43, distinct, p, i],
                                        exponents=synth.finite_exponents(distinct)).reshape(r, c)
              for i, (r, c) in enumerate(group)]
        x = synth.activation_bf16(group[0][1], [44, p])
        ds = [cbk.encode(w).to("cuda") for w in ws]
        xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        ys = [torch.full((d.rows,), float("nan"), dtype=torch.float32, device="cuda") for d in ds]
        phases.append((ds, xd, ys))
        host.append((ws, x))
    print(f"chain at b = {phases[0][0][0].b}", flush=True)
    chain = cbk.GemvChain(phases)
    chain.run()
    got = _outputs(torch, phases)
    assert chain.check() == 0
    for p, ((ds, xd, _), (ws, x)) in enumerate(zip(phases, host)):
        single = cbk.gemv_group(ds, xd)
        torch.cuda.synchronize()
        for i, (d, s, w) in enumerate(zip(ds, single, ws)):
            assert np.array_equal(got[p][i], s.cpu().numpy()), f"phase {p} tensor {i}: differs from cbk_gemv_group"
            rows = np.unique([0, d.rows // 2, d.rows - 1])
            ref, absb = oracle_mod.gemv(oracle_mod.encode(w[rows]), x)
            assert np.all(np.abs(got[p][i][rows] - ref) <= TOL * absb)
