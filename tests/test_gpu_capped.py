"""GPU parity for capped (lossy) codebooks: the tensor after cbk_cap_patterns is encoded as usual,
so the fast kernels must decode it bit-exactly to the oracle's capped tensor (oracle/capped.py)
and compute its GEMV and skinny GEMM within the usual bound, at the narrower widths the cap gives."""
import numpy as np
import pytest

import synth
from oracle import capped

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


@pytest.mark.parametrize("K,b", [(2048, 11), (1024, 10), (256, 8), (16, 4)])
def test_capped_decode_and_gemv(env, oracle_mod, K, b):
    torch, cbk = env
    print(f"capped K={K}", flush=True)
    w = synth.gaussian_bf16((1024, 4096), 0.02, seed=[80, K])
    wc = capped.cap(w, K)
    c = cbk.encode(w, cap=K)
    assert (c.U, c.b) == (min(K, np.unique(w).size), b)
    d = c.to("cuda")
    out = cbk.decode_bf16(d)
    x = synth.workload_x(2, 4096)[0]
    y = cbk.gemv(d, torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16))
    X = synth.workload_x(2, 4096, 16)
    Y = cbk.gemm_small(d, torch.from_numpy(X.view(np.int16)).to("cuda").view(torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), wc)
    e = oracle_mod.encode(wc)
    ref, absb = oracle_mod.gemv(e, x)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref) <= TOL * absb)
    Yg = Y.cpu().numpy().astype(np.float64)
    for j in (0, 7, 15):
        ref, absb = oracle_mod.gemv(e, X[j])
        assert np.all(np.abs(Yg[j] - ref) <= TOL * absb), j
