"""GPU parity at the decode-step workloads' full tensor sizes, through the C ABI.

* One tensor of each 70B shape (8192x8192, 1024x8192, 28672x8192, 8192x28672): the weights drawn on
  the GPU equal the host's draw bit for bit, the GPU encoder's output equals the host encoder's,
  and the standalone decode gives back every weight exactly.
* The 70B layer's grouped batch-1 launches ([q, k, v] and [gate, up], K = 8192): every row equals
  the single-tensor cbk_gemv bit for bit, and sampled rows (first and last included) are within
  1e-3 * sum|W x| of the oracle.
* One layer of each step workload captured in a HIP graph exactly as bench.py builds and times it,
  replayed twice with the outputs clobbered in between: every tensor's output, on sampled rows, is
  within tolerance of the oracle after each replay.
* The grouped calls of the 4096^2 workloads (decode, GPU encode, entropy-coded decode and fused
  GEMV) captured and replayed three times the same way: the first and last tensor of every call
  equal the host weights or the host encoder (the fused GEMV: sampled rows within tolerance of the
  oracle) after each replay.

The oracle's inputs are the host draws of the same rows (synth.workload_rows), encoded by the
oracle itself; nothing the GPU computes is used as an expected value.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


def _host(torch, t):
    return t.cpu().numpy().view(np.uint16)


def _sample(rows, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, k, replace=False)]))


def _check_rows(oracle_mod, cfg, layer, t, got_rows_fn, X, rows):
    """got_rows_fn(rows) -> GPU values for those rows ([rows] or [batch][rows]); X [batch][cols]."""
    e = oracle_mod.encode(synth.workload_rows(cfg, layer, t, rows))
    if X.shape[0] == 1:
        ref, absb = oracle_mod.gemv(e, X[0])
    else:
        ref, absb = oracle_mod.gemm(e, X)
    got = got_rows_fn(rows)
    err = np.abs(got - ref)
    assert np.all(err <= TOL * absb), \
        f"{t.name} layer {layer}: max err/bound {np.max(err / np.maximum(TOL * absb, 1e-300))}"


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_70b_shapes_generate_encode_decode_full_size(env, name):
    torch, cbk = env
    t = next(t for t in synth.WORKLOADS[5][0] if t.name == name)
    print(f"70b shape {name} {t.rows}x{t.cols}", flush=True)
    w = synth.workload_tensor(5, 0, t)                       # host draw
    raw = synth.workload_tensor_device(5, 0, t, "cuda")       # GPU draw of the same tensor
    torch.cuda.synchronize()
    assert np.array_equal(_host(torch, raw), w.reshape(-1)), "GPU draw differs from the host draw"
    host = cbk.encode(w)
    dev = cbk.encode_gpu(raw, rows=t.rows, cols=t.cols)
    assert (dev.U, dev.b) == (host.U, host.b) and host.b == 13
    assert np.array_equal(_host(torch, dev.codebook), host.codebook)
    assert np.array_equal(dev.words.cpu().numpy().view(np.uint32), host.words)
    del raw, dev
    d = host.to("cuda")
    out = cbk.decode_bf16(d)
    torch.cuda.synchronize()
    assert np.array_equal(_host(torch, out.view(torch.int16)).reshape(t.rows, t.cols), w)


@pytest.mark.parametrize("names", [("q", "k", "v"), ("gate", "up")])
def test_70b_grouped_gemv_k8192(env, oracle_mod, names):
    torch, cbk = env
    group = [t for t in synth.WORKLOADS[5][0] if t.name in names]
    print(f"70b grouped gemv {names}", flush=True)
    ds = [cbk.encode_gpu(synth.workload_tensor_device(5, 0, t, "cuda"), rows=t.rows, cols=t.cols) for t in group]
    x = synth.workload_x(5, 8192)
    xd = torch.from_numpy(x[0].view(np.int16)).to("cuda").view(torch.bfloat16)
    ys = cbk.gemv_group(ds, xd)
    singles = [cbk.gemv(d, xd) for d in ds]
    torch.cuda.synchronize()
    for t, d, y, s in zip(group, ds, ys, singles):
        assert torch.equal(y, s), f"{t.name}: grouped launch differs from the single-tensor call"
        yh = y.cpu().numpy().astype(np.float64)
        _check_rows(oracle_mod, 5, 0, t, lambda r: yh[r], x, _sample(t.rows, 62, [5, t.tensor_id, 31]))


@pytest.mark.parametrize("workload", ["l70b_b1", "l70b_b16", "llama7b"])
def test_layer_step_graph_replay(env, oracle_mod, workload):
    """One layer of the step workload, captured and replayed as bench.py times it."""
    torch, cbk = env
    import bench
    print(f"graph replay of one layer of {workload}", flush=True)
    work = bench.Workload(workload, layers=1)
    graph = work.capture()
    X = {c: synth.workload_x(work.specs[0][0], c, max(1, work.batch)) for c in {d.cols for d in work.tensors}}
    for rep in range(2):
        for y in work.ys:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (cfg, layer, t) in enumerate(work.specs):
            yh = work.ys[i].cpu().numpy().astype(np.float64)
            rows = _sample(t.rows, 30, [cfg, t.tensor_id, rep])
            pick = (lambda r: yh[r]) if work.batch == 1 else (lambda r: yh[:, r])
            _check_rows(oracle_mod, cfg, layer, t, pick, X[t.cols], rows)
            assert not np.isnan(yh).any(), f"{t.name}: replay {rep} left outputs unwritten"


@pytest.mark.parametrize("workload,ec_index", [("decode4096", False), ("encode4096", False), ("ecdecode4096", False),
                                               ("ecdecode4096", True), ("ecgemv4096", True)])
def test_grouped_calls_graph_replay(env, workload, ec_index):
    """The grouped calls of the 4096^2 workloads (cbk_decode_group, cbk_encode_gpu_group,
    cbk_ec_decode_group, cbk_ec_gemv_group; four or three tensors per call, the last call ragged)
    captured in a HIP graph as bench.py builds it and replayed three times, every output clobbered
    before each replay: the first and last tensor of every call are checked after each replay
    (bit-exact, or within the tolerance for the fused GEMV)."""
    torch, cbk = env
    import bench
    print(f"graph replay of {workload} (index {ec_index})", flush=True)
    work = bench.Workload(workload, count=10, ec_index=ec_index)
    graph = work.capture()
    which = sorted({i for ph in work.phases for i in (ph[0], ph[-1])})
    for rep in range(3):
        if work.encode:
            for t in work.enc_words + work.enc_meta + work.enc_cb:
                t.fill_(-1)
        else:
            for y in work.ys:
                y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        if work.encode:
            bench.check_encoded(work, which)
        elif work.ecfmt:
            bench.check_ec(work, which)
        else:
            bench.check_decoded(work, which)
