"""GPU test of cbk_encode_gpu_noalloc, the encoder entry point that allocates nothing (its
presence bitmaps live in the library's static device scratch): its output must equal that of
cbk_encode_gpu (caller-owned workspace) exactly, on two calls in a row, the second with a smaller
input, so that whatever the first call left in the shared scratch cannot leak into the second."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


def _outputs(torch, cbk, n):
    cb = torch.full((65536,), -1, dtype=torch.int16, device="cuda")
    words = torch.full((max(cbk.words_for(n, 16), 4),), -1, dtype=torch.int32, device="cuda")
    meta = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    return cb, words, meta


def _encode_both(env, w):
    torch, cbk = env
    flat = np.ascontiguousarray(w).reshape(-1)
    d = torch.from_numpy(flat.view(np.int16)).to("cuda")
    n = flat.size
    ws = torch.empty(cbk.encode_gpu_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ref = _outputs(torch, cbk, n)
    got = _outputs(torch, cbk, n)
    cbk.encode_gpu_launch(d, ws, *ref)
    cbk.encode_gpu_noalloc_launch(d, *got)
    torch.cuda.synchronize()
    U, b = (int(v) for v in ref[2].cpu().tolist())
    assert [int(v) for v in got[2].cpu().tolist()] == [U, b]
    nw = cbk.words_for(n, b)
    assert np.array_equal(got[0][:U].cpu().numpy(), ref[0][:U].cpu().numpy())
    assert np.array_equal(got[1][:nw].cpu().numpy(), ref[1][:nw].cpu().numpy())
    # nothing past the stream is written, as for the workspace call
    assert bool((got[1][nw:] == -1).all())
    return U, b


def test_noalloc_encode_equals_workspace_encode_twice_second_smaller(env):
    print("noalloc: 2048x4096 N(0,0.02), then 1000x257 with 300 distinct patterns", flush=True)
    big = synth.gaussian_bf16((2048, 4096), 0.02, seed=[7, 0, 0])
    U1, b1 = _encode_both(env, big)
    small = synth.with_distinct_count(1000 * 257, 300, seed=[7, 0, 1])
    U2, b2 = _encode_both(env, small)
    assert (U2, b2) == (300, 9) and b1 >= 12


def test_noalloc_encode_matches_host_encoder(env):
    torch, cbk = env
    w = synth.gaussian_bf16((513, 1000), 0.02, seed=[7, 0, 2])
    U, b = _encode_both(env, w)
    h = cbk.encode(w)
    assert (U, b) == (h.U, h.b)
