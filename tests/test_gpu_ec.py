"""GPU parity for the exponent entropy-coded format: cbk_ec_decode_bf16 (through the C ABI) must
give back the exact input patterns, which the oracle's decoder also reproduces (the oracle's own
pins are in test_oracle_entropy.py; the host encoder's bytes equal the oracle's in
test_abi_ec.py)."""
import numpy as np
import pytest

import synth
from oracle import entropy as ec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import fly_decode_amd as cbk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cbk.load_library()
    return torch, cbk


def _check(env, w, oracle_too=False):
    torch, cbk = env
    print(f"ec decode shape={w.shape}", flush=True)
    t = cbk.ec_encode(w)
    d = t.to("cuda")
    out = cbk.ec_decode_bf16(d)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape)
    assert np.array_equal(got, w), f"mismatch at {np.flatnonzero(got.reshape(-1) != w.reshape(-1))[:10]}"
    if oracle_too:
        o = ec.encode_with_lengths(w, t.lengths)
        assert np.array_equal(ec.decode(o), got.reshape(-1))
    return t


def _mixed_short_codes(shape, seed):
    """A leading run of 60 % of the weights shares one exponent (random mantissas), so that exponent
    gets a one-bit code: the blocks of the run hold more codes than the decoder's exponent array
    and are placed and joined in two halves, the blocks after it in one pass."""
    w = synth.gaussian_bf16(shape, 0.02, seed=seed).reshape(-1).copy()
    k = int(0.6 * w.size)
    w[:k] = (0x3C00 | np.random.default_rng(seed).integers(0, 128, k)).astype(np.uint16)
    return w.reshape(shape)


def _cases():
    rng = np.random.default_rng(21)
    return {
        "gaussian_300x777": synth.gaussian_bf16((300, 777), 0.02, seed=[41]),
        "t2_heavy_tail": synth.student_t_bf16((200, 1000), 2.0, 0.02, seed=[42]),
        "t4_64x4096": synth.student_t_bf16((64, 4096), 4.0, 0.02, seed=[43]),
        "constant": np.full((10, 1000), 0x3F80, dtype=np.uint16),
        "two_exponents": rng.choice(np.array([0x3F80, 0x4012], dtype=np.uint16), (70, 130)),
        "every_pattern": rng.permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16).reshape(256, 256),
        "specials": rng.choice(np.array([0x7F80, 0xFF80, 0x7FC1, 0x0000, 0x8000, 0x0001, 0x807F], dtype=np.uint16), (9, 111)),
        "one": np.array([[0xC2F7]], dtype=np.uint16),
        # one-bit codes over several blocks and a ragged end: every block in two halves
        "one_bit_codes_multi_block": rng.choice(np.array([0x3F80, 0x4012], dtype=np.uint16), (1, 64 * 256 * 3 + 11)),
        "mixed_short_codes": _mixed_short_codes((200, 1000), [45]),
    }


@pytest.mark.parametrize("name", list(_cases()))
def test_ec_decode_bit_exact(env, name):
    w = _cases()[name]
    t = _check(env, w, oracle_too=w.size <= 70000)
    if name == "constant":
        assert t.total_bits == w.size   # 64 one-bit codes in every span
    if name == "t2_heavy_tail":
        assert max(t.lengths) >= 10     # long codes, spans that start inside a code
    if name == "mixed_short_codes":
        # blocks of both kinds: more codes than the decoder places at once (8,192) and fewer
        per_block = np.diff(np.append(t.bases.astype(np.int64), w.size))
        assert per_block.max() > 8192 and per_block[:-1].min() < 8185, per_block


@pytest.mark.parametrize("n", [7, 8, 9, 63, 64, 65, 1000, 16383, 16384, 16385, 64 * 256 * 3 + 11])
def test_ec_decode_ragged_lengths(env, n):
    """Lengths around the 8-weight output segment, the 64-bit span and the 256-span block."""
    w = synth.gaussian_bf16((1, n), 0.02, seed=[44, n])
    _check(env, w)


def test_ec_decode_workload_tensor(env):
    """A 4096^2 tensor of the attention workload: every weight exact; the format stores about
    10.6 bits per weight."""
    w = synth.workload_tensor(2, 0, synth.WORKLOADS[2][0][0])
    t = _check(env, w)
    bits = 8.0 * t.stored_bytes / w.size
    assert 10.0 < bits < 11.5, bits


def test_ec_decode_writes_nothing_past_the_end(env):
    torch, cbk = env
    for n in (64 * 256 * 2 + 5, 8 * 700 + 1, 4096 + 8, 7, 3 * 4096):
        print(f"ec guard n={n}", flush=True)
        w = synth.gaussian_bf16((1, n), 0.02, seed=[45, n])
        d = cbk.ec_encode(w).to("cuda")
        buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
        assert buf.data_ptr() % 16 == 0
        cbk.ec_decode_bf16(d, out=buf[:n].view(torch.bfloat16).view(1, n))
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        assert np.array_equal(got[:n].view(np.uint16), w.reshape(-1)), n
        assert bool((got[n:] == -7).all()), n


def test_ec_decode_repeated_launches_identical(env):
    torch, cbk = env
    w = synth.gaussian_bf16((512, 1024), 0.02, seed=[46])
    d = cbk.ec_encode(w).to("cuda")
    a = cbk.ec_decode_bf16(d).clone()
    for _ in range(3):
        b = cbk.ec_decode_bf16(d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_ec_decode_corrupt_stream_stays_in_bounds(env):
    """Random stream words and gaps (the table, bases and sizes valid): the values are undefined,
    but nothing is written outside the output."""
    torch, cbk = env
    n = 64 * 256 * 2 + 100
    w = synth.gaussian_bf16((1, n), 0.02, seed=[47])
    t = cbk.ec_encode(w)
    rng = np.random.default_rng(48)
    bad = cbk.ECTensor(t.rows, t.cols, t.total_bits, t.lengths, t.sm,
                       rng.integers(0, 2 ** 32, t.stream.size, dtype=np.uint64).astype(np.uint32),
                       rng.integers(0, 2 ** 32, t.gaps.size, dtype=np.uint64).astype(np.uint32),
                       t.bases, t.lut).to("cuda")
    buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
    cbk.ec_decode_bf16(bad, out=buf[:n].view(torch.bfloat16).view(1, n))
    torch.cuda.synchronize()
    assert bool((buf[n:].cpu() == -7).all())


# ---------------------------------------------------------------- fused GEMV on the same format
TOL = 1e-3


def _gemv_check(env, w, x, rows=None):
    """cbk_ec_gemv against the oracle: the oracle decodes (bit by bit) the rows it checks, from its
    own encoding of them, and forms y = W x in float64."""
    torch, cbk = env
    R, C = w.shape
    print(f"ec gemv shape={w.shape}", flush=True)
    d = cbk.ec_encode(w).to("cuda")
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    y = cbk.ec_gemv(d, xd)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    sub = w if rows is None else np.ascontiguousarray(w[np.asarray(rows)])
    ref, absb = ec.gemv(ec.encode(sub), sub.shape[0], C, x)
    if rows is not None:
        got = got[np.asarray(rows)]
    err = np.abs(got - ref)
    assert np.all(err <= TOL * absb), f"max err/bound {np.max(err / np.maximum(absb, 1e-300))}"
    return y


def _gemv_cases():
    rng = np.random.default_rng(31)
    return {
        "gaussian_300x776": synth.gaussian_bf16((300, 776), 0.02, seed=[51]),
        "t2_200x1000": synth.student_t_bf16((200, 1000), 2.0, 0.02, seed=[52]),
        "t4_64x4096": synth.student_t_bf16((64, 4096), 4.0, 0.02, seed=[53]),
        "one_bit_codes_10x1000": np.full((10, 1000), 0x3F80, dtype=np.uint16),
        "narrow_rows_300x64": synth.gaussian_bf16((300, 64), 0.02, seed=[54]),
        # row lengths whose segment count (cols / 8) is odd or prime: the row index of a segment
        # comes from a multiply-and-shift division by cols
        "cols_8x1049_40x8392": synth.gaussian_bf16((40, 8392), 0.02, seed=[59]),
        "cols_11008_24x11008": synth.gaussian_bf16((24, 11008), 0.02, seed=[60]),
        "cols_72_500x72": synth.gaussian_bf16((500, 72), 0.02, seed=[61]),
        "specials_free_mix_37x128": rng.choice(np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4000, 0x3C00],
                                                        dtype=np.uint16), (37, 128)),
        # blocks placed in two halves (one-bit codes), rows crossing the halves and the blocks
        "one_bit_codes_60x1000": rng.choice(np.array([0x3F80, 0xBF80], dtype=np.uint16), (60, 1000)),
        "mixed_short_codes_200x1024": _mixed_short_codes((200, 1024), [62]),
    }


@pytest.mark.parametrize("name", list(_gemv_cases()))
def test_ec_gemv_matches_oracle(env, name):
    w = _gemv_cases()[name]
    x = synth.activation_bf16(w.shape[1], seed=[55, w.shape[1]])
    _gemv_check(env, w, x)


def test_ec_gemv_workload_tensor_sampled_rows(env):
    """A 4096^2 attention-workload tensor; 64 sampled rows, the first and last included."""
    w = synth.workload_tensor(2, 0, synth.WORKLOADS[2][0][0])
    x = synth.workload_x(2, 4096)[0]
    rows = np.concatenate([[0, 4095], np.random.default_rng(56).choice(np.arange(1, 4095), 62, replace=False)])
    _gemv_check(env, w, x, rows=rows)


def test_ec_gemv_overwrites_y_and_repeats_within_tolerance(env):
    """y is overwritten (not accumulated into) and repeated calls agree to the tolerance (the
    atomic adds may sum a row's block partials in any order)."""
    torch, cbk = env
    w = synth.gaussian_bf16((512, 1024), 0.02, seed=[57])
    x = synth.activation_bf16(1024, seed=[58])
    d = cbk.ec_encode(w).to("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    y = torch.full((512,), 1e30, dtype=torch.float32, device="cuda")
    cbk.ec_gemv(d, xd, y=y)
    y0 = y.clone()
    for _ in range(3):
        cbk.ec_gemv(d, xd, y=y)
    torch.cuda.synchronize()
    ref, absb = ec.gemv(ec.encode(w), 512, 1024, x)
    for v in (y0, y):
        assert np.all(np.abs(v.cpu().numpy().astype(np.float64) - ref) <= TOL * absb)


def test_ec_gemv_zero_cols_gives_zeros(env):
    """rows x 0 weights: y = W x is all zeros, x (empty) is not read and may be NULL."""
    torch, cbk = env
    d = cbk.ec_encode(np.zeros((8, 0), dtype=np.uint16)).to("cuda")
    y = torch.full((8,), 5.0, dtype=torch.float32, device="cuda")
    x = torch.zeros(8, dtype=torch.bfloat16, device="cuda")[:0]
    cbk.ec_gemv(d, x, y=y)
    torch.cuda.synchronize()
    assert not y.any()


def test_ec_decode_empty_tensor(env):
    torch, cbk = env
    d = cbk.ec_encode(np.zeros((0, 64), dtype=np.uint16)).to("cuda")
    out = cbk.ec_decode_bf16(d)
    torch.cuda.synchronize()
    assert out.numel() == 0


# ---------------------------------------------------------------- span index (one walk per span)
def _oracle_span_counts(t_host, w):
    """Codes that start in each span, from the oracle's span decoder on its own encoding."""
    o = ec.encode_with_lengths(w, t_host.lengths)
    return np.array([len(ec.decode_span(o, j)) for j in range(o.spans)], dtype=np.int64)


@pytest.mark.parametrize("name", ["gaussian_300x777", "t2_heavy_tail", "constant", "two_exponents", "specials", "one",
                                  "mixed_short_codes"])
def test_ec_index_counts_equal_the_oracle(env, name):
    torch, cbk = env
    w = _cases()[name]
    t = cbk.ec_encode(w)
    d = t.to("cuda")
    index = cbk.ec_build_index(d)
    torch.cuda.synchronize()
    want = _oracle_span_counts(t, w)
    got = index.cpu().numpy()[: want.size].astype(np.int64)
    assert np.array_equal(got, want)
    assert int(got.sum()) == w.size  # every code starts in exactly one span


@pytest.mark.parametrize("name", list(_cases()))
def test_ec_indexed_decode_bit_exact(env, name):
    torch, cbk = env
    w = _cases()[name]
    print(f"ec indexed decode {name}", flush=True)
    d = cbk.ec_encode(w).to("cuda")
    out = cbk.ec_decode_bf16(d, index=cbk.ec_build_index(d))
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape), w)


@pytest.mark.parametrize("n", [7, 64, 65, 16384, 16385, 64 * 256 * 3 + 11])
def test_ec_indexed_decode_ragged_lengths_and_guard(env, n):
    torch, cbk = env
    w = synth.gaussian_bf16((1, n), 0.02, seed=[57, n])
    d = cbk.ec_encode(w).to("cuda")
    index = cbk.ec_build_index(d)
    buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
    cbk.ec_decode_bf16(d, out=buf[:n].view(torch.bfloat16).view(1, n), index=index)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:n].view(np.uint16), w.reshape(-1))
    assert bool((got[n:] == -7).all())


def test_ec_indexed_decode_workload_tensor(env):
    torch, cbk = env
    w = synth.workload_tensor(2, 0, synth.WORKLOADS[2][0][0])
    d = cbk.ec_encode(w).to("cuda")
    out = cbk.ec_decode_bf16(d, index=cbk.ec_build_index(d))
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape), w)


@pytest.mark.parametrize("name", list(_gemv_cases()))
def test_ec_indexed_gemv_matches_oracle(env, name):
    torch, cbk = env
    w = _gemv_cases()[name]
    x = synth.activation_bf16(w.shape[1], seed=[55, w.shape[1]])
    d = cbk.ec_encode(w).to("cuda")
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    y = cbk.ec_gemv(d, xd, index=cbk.ec_build_index(d))
    torch.cuda.synchronize()
    ref, absb = ec.gemv(ec.encode(w), w.shape[0], w.shape[1], x)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= TOL * absb), f"max err/bound {np.max(err / np.maximum(absb, 1e-300))}"


def test_ec_wrong_index_stays_in_bounds(env):
    """An index whose counts do not match the stream (every count 255, read as 64): the values are
    undefined, but nothing is written outside the output."""
    torch, cbk = env
    n = 64 * 256 * 2 + 100
    w = synth.gaussian_bf16((1, n), 0.02, seed=[58])
    d = cbk.ec_encode(w).to("cuda")
    index = torch.full_like(cbk.ec_build_index(d), 255)
    buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
    cbk.ec_decode_bf16(d, out=buf[:n].view(torch.bfloat16).view(1, n), index=index)
    torch.cuda.synchronize()
    assert bool((buf[n:].cpu() == -7).all())


# ------------------------------------------------- grouped calls (a block's matrices together)
def _group_weights():
    """Eleven tensors (two launches: a run of eight, then three): shapes from one weight to several
    blocks, heavy tails, one-bit codes, a ragged length and an empty tensor in the middle."""
    cases = _cases()
    ws = [synth.gaussian_bf16((257, 1000), 0.02, seed=[70]), cases["t2_heavy_tail"], cases["constant"],
          np.zeros((0, 64), dtype=np.uint16), cases["one"], synth.gaussian_bf16((1, 64 * 256 * 3 + 11), 0.02, seed=[71]),
          cases["specials"], cases["two_exponents"], synth.student_t_bf16((64, 4096), 4.0, 0.02, seed=[72]),
          cases["every_pattern"], synth.gaussian_bf16((3, 7), 0.02, seed=[73])]
    return ws


@pytest.mark.parametrize("indexed", [False, True])
def test_ec_decode_group_bit_exact(env, indexed):
    """cbk_ec_decode_group: every output equals the input patterns (and so the single call), with
    and without the span indexes."""
    torch, cbk = env
    ws = _group_weights()
    print(f"ec decode group of {len(ws)} tensors, indexed={indexed}", flush=True)
    ds = [cbk.ec_encode(w).to("cuda") for w in ws]
    ix = [cbk.ec_build_index(d) for d in ds] if indexed else None
    outs = [torch.full((d.rows, d.cols), float("nan"), dtype=torch.bfloat16, device="cuda") for d in ds]
    cbk.ec_decode_group(ds, outs=outs, indexes=ix)
    torch.cuda.synchronize()
    for i, (w, o) in enumerate(zip(ws, outs)):
        got = o.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape)
        assert np.array_equal(got, w), f"tensor {i} {w.shape}"


def test_ec_decode_group_workload_layer(env):
    """Four 4096^2 attention-workload tensors, the bench's grouped launch: every weight exact."""
    torch, cbk = env
    t = synth.WORKLOADS[2][0][0]
    ws = [synth.workload_tensor(2, layer, t) for layer in range(4)]
    ds = [cbk.ec_encode(w).to("cuda") for w in ws]
    ix = [cbk.ec_build_index(d) for d in ds]
    outs = cbk.ec_decode_group(ds, indexes=ix)
    torch.cuda.synchronize()
    for i, (w, o) in enumerate(zip(ws, outs)):
        assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), w), f"tensor {i}"


@pytest.mark.parametrize("indexed", [False, True])
def test_ec_gemv_group_matches_oracle(env, indexed):
    """cbk_ec_gemv_group over nine tensors of 1,000 columns and different rows (a run of eight,
    then one; one tensor has no rows): every y within the tolerance of the oracle's decode and
    float64 product, and every y overwritten."""
    torch, cbk = env
    cols = 1000
    shapes = [(300, cols), (1, cols), (0, cols), (77, cols), (1100, cols), (17, cols), (64, cols), (5, cols), (129, cols)]
    ws = [synth.student_t_bf16(s, 4.0, 0.02, seed=[74, i]) if i % 2 else synth.gaussian_bf16(s, 0.02, seed=[74, i])
          for i, s in enumerate(shapes)]
    x = synth.activation_bf16(cols, seed=[75])
    print(f"ec gemv group of {len(ws)} tensors, indexed={indexed}", flush=True)
    ds = [cbk.ec_encode(w).to("cuda") for w in ws]
    ix = [cbk.ec_build_index(d) for d in ds] if indexed else None
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    ys = [torch.full((d.rows,), 1e30, dtype=torch.float32, device="cuda") for d in ds]
    cbk.ec_gemv_group(ds, xd, ys=ys, indexes=ix)
    torch.cuda.synchronize()
    for i, (w, y) in enumerate(zip(ws, ys)):
        if w.shape[0] == 0:
            continue
        ref, absb = ec.gemv(ec.encode(w), w.shape[0], cols, x)
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= TOL * absb), f"tensor {i}: max err/bound {np.max(err / np.maximum(absb, 1e-300))}"


def test_ec_gemv_group_workload_rows(env):
    """Three 4096^2 attention-workload tensors sharing x, as the bench groups them: sampled rows
    (first and last included) within the tolerance of the oracle."""
    torch, cbk = env
    t = synth.WORKLOADS[2][0][0]
    ws = [synth.workload_tensor(2, layer, t) for layer in range(3)]
    x = synth.workload_x(2, 4096)[0]
    ds = [cbk.ec_encode(w).to("cuda") for w in ws]
    ix = [cbk.ec_build_index(d) for d in ds]
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    ys = cbk.ec_gemv_group(ds, xd, indexes=ix)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 4095], np.random.default_rng(76).choice(np.arange(1, 4095), 30, replace=False)])
    for i, (w, y) in enumerate(zip(ws, ys)):
        sub = np.ascontiguousarray(w[rows])
        ref, absb = ec.gemv(ec.encode(sub), len(rows), 4096, x)
        err = np.abs(y.cpu().numpy().astype(np.float64)[rows] - ref)
        assert np.all(err <= TOL * absb), f"tensor {i}"


def test_ec_decode_fitted_kernel_and_a_wrong_bound(env):
    """Blocks of at most 8,185 codes take the decode that holds half a block's exponents; a tensor
    whose stated bound is below its true block counts (one-bit codes: 16,384 per block) gets
    unspecified values for those blocks but no write outside the output, with and without the
    index; with its true bound it decodes exactly."""
    torch, cbk = env
    n = 64 * 256 * 3 + 11
    w = np.random.default_rng(77).choice(np.array([0x3F80, 0x4012], dtype=np.uint16), (1, n))
    d = cbk.ec_encode(w).to("cuda")
    assert d.max_block_codes == 16384
    ix = cbk.ec_build_index(d)
    for index in (None, ix):
        d.max_block_codes = 8000   # wrong: the fitted kernel runs and skips the full blocks
        buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
        cbk.ec_decode_bf16(d, out=buf[:n].view(torch.bfloat16).view(1, n), index=index)
        torch.cuda.synchronize()
        assert bool((buf[n:].cpu() == -7).all())
        d.max_block_codes = 16384  # true bound: the general kernel, exact
        out = cbk.ec_decode_bf16(d, index=index)
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), w)
    g = synth.gaussian_bf16((300, 1000), 0.02, seed=[78])
    dg = cbk.ec_encode(g).to("cuda")
    assert 0 < dg.max_block_codes <= 8185   # the fitted kernel
    out = cbk.ec_decode_bf16(dg)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), g)
