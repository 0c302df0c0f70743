"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar: standalone decode bit-exact; fused GEMV / GEMM within |y - y_ref| <= 1e-3 * sum_k |W x| per
element (y_ref and the bound from the oracle, float64); exact equality where the result is exact
whatever the summation order (integer-valued data, one-hot x, constant tensors).
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


def _up(torch, a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(dtype)


def _decode_check(env, w, oracle_mod=None):
    torch, cbk = env
    c = cbk.encode(w)
    d = c.to("cuda")
    out = cbk.decode_bf16(d)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape)
    assert np.array_equal(got, w), f"decode mismatch U={c.U} b={c.b} shape={w.shape}"
    return c, d


def _oracle_rows(oracle_mod, w, rows, product):
    """The oracle's product over all rows of w, or over the listed rows only: the oracle then
    encodes just those rows (its own codebook of them), which decodes to the same weights, so the
    reference for those rows is unchanged and a 235M-weight tensor needs no full oracle encode."""
    if rows is None:
        return product(oracle_mod.encode(w))
    return product(oracle_mod.encode(np.ascontiguousarray(w[np.asarray(rows)])))


def _gemv_check(env, oracle_mod, w, x, rows=None, exact=False):
    torch, cbk = env
    c = cbk.encode(w)
    d = c.to("cuda")
    y = cbk.gemv(d, _up(torch, x, torch.bfloat16))
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref, absb = _oracle_rows(oracle_mod, w, rows, lambda e: oracle_mod.gemv(e, x))
    got = y if rows is None else y[np.asarray(rows)]
    if exact:
        assert np.array_equal(got, ref)
    else:
        err = np.abs(got - ref)
        assert np.all(err <= TOL * absb), f"max err/bound {np.max(err / np.maximum(absb, 1e-300))}"
    return got, ref


def _gemm_check(env, oracle_mod, w, X, rows=None, exact=False, ldx=None):
    torch, cbk = env
    c = cbk.encode(w)
    d = c.to("cuda")
    batch, K = X.shape
    if ldx is None:
        Xd = _up(torch, X, torch.bfloat16)
    else:
        buf = torch.zeros((batch, ldx), dtype=torch.bfloat16, device="cuda")
        buf[:, :K] = _up(torch, X, torch.bfloat16)
        Xd = buf[:, :K]
    Y = cbk.gemm_small(d, Xd)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy().astype(np.float64)
    ref, absb = _oracle_rows(oracle_mod, w, rows, lambda e: oracle_mod.gemm(e, X))
    got = Y if rows is None else Y[:, np.asarray(rows)]
    if exact:
        assert np.array_equal(got, ref)
    else:
        err = np.abs(got - ref)
        assert np.all(err <= TOL * absb), f"max err/bound {np.max(err / np.maximum(absb, 1e-300))}"
    return got


# --------------------------------------------------------------------------------- decode
@pytest.mark.parametrize("b", list(range(0, 17)))
def test_decode_every_width(env, b):
    """Every width b = 0..16, U at both ends of the width, ragged and unit-aligned lengths."""
    for U in sorted({max(1, 2 ** (b - 1) + 1) if b else 1, 2 ** b}):
        for rows, cols in [(37, 111), (3, 2 * 128 * 7 + 5), (64, 256)]:
            n = rows * cols
            if n < U:
                rows = (U + cols - 1) // cols
                n = rows * cols
            w = synth.with_distinct_count(n, U, seed=[31, b, U, cols]).reshape(rows, cols)
            c, _ = _decode_check(env, w)
            assert c.U == U and c.b == b


def test_decode_tail_and_misaligned_output(env):
    torch, cbk = env
    w = synth.with_distinct_count(12345, 6000, seed=[32]).reshape(1, -1)
    c = cbk.encode(w)
    d = c.to("cuda")
    buf = torch.zeros(12345 + 8, dtype=torch.bfloat16, device="cuda")
    out = buf[1:1 + 12345].view(1, -1)  # 2-byte aligned only: generic path
    cbk.decode_bf16(d, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), w)
    assert int(buf[0].view(torch.int16)) == 0 and not buf[1 + 12345:].view(torch.int16).any()



def test_decode_fast_path_writes_nothing_past_the_end(env):
    """16-byte-aligned output (fast kernel) followed by a guard region: lengths ending inside a
    16-byte chunk, just past a wave step of 4096 weights, and shorter than one chunk."""
    torch, cbk = env
    for n in (4096 * 3 + 5, 8 * 700 + 1, 4096 + 8, 7, 3 * 4096):
        w = synth.with_distinct_count(n, min(n, 3000), seed=[34, n]).reshape(1, n)
        d = cbk.encode(w).to("cuda")
        buf = torch.full((n + 64,), -7, dtype=torch.int16, device="cuda")
        assert buf.data_ptr() % 16 == 0
        cbk.decode_bf16(d, out=buf[:n].view(torch.bfloat16).view(1, n))
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        assert np.array_equal(got[:n].view(np.uint16), w.reshape(-1)), n
        assert bool((got[n:] == -7).all()), n

def test_decode_corrupt_index_is_memory_safe(env, oracle_mod):
    torch, cbk = env
    w = synth.with_distinct_count(4096, 5000 // 2, seed=[33]).reshape(32, 128)
    c = cbk.encode(w)
    assert c.b == 12 and c.U < 4096
    words = c.words.copy()
    bad_fields = [0, 77, 1000, 4095]
    for f in bad_fields:  # force index 4095 >= U into these fields
        for j in range(12):
            p = f * 12 + j
            words[p >> 5] |= np.uint32(1 << (p & 31))
    bad = c.__class__(c.rows, c.cols, c.U, c.b, c.codebook, words).to("cuda")
    out = cbk.decode_bf16(bad)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    e = oracle_mod.Encoded(c.codebook, c.U, c.b, words[:oracle_mod.stream_words(4096, 12)], 4096, (32, 128))
    assert np.array_equal(got, oracle_mod.decode(e))
    assert all(got[f] == 0x7FC0 for f in bad_fields)


@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_workload_full_size(env, cfg):
    w = synth.workload_tensor(cfg, 0, synth.WORKLOADS[cfg][0][0])
    c, _ = _decode_check(env, w)
    assert c.b in (12, 13)


def test_decode_heavy_tailed_mlp_full_size(env):
    for t in synth.WORKLOADS[3][0]:
        if t.name in ("gate", "down"):
            _decode_check(env, synth.workload_tensor(3, 0, t))


# ----------------------------------------------------------------------------------- GEMV
def _int_bf16(vals):
    return synth.f32_to_bf16(np.asarray(vals, dtype=np.float32))


# GEMV shapes: cols/64 = 3 (one partial wave step per row), 130 (three steps, the last partial),
# 67 (odd: rows start half-way into a 16-byte chunk for odd b), and a ragged K (generic kernel).
GEMV_SHAPES = [(67, 192), (5, 64 * 130), (9, 64 * 67), (33, 129)]


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16])
def test_gemv_every_width(env, oracle_mod, b):
    U = 2 ** b if b <= 12 else 2 ** (b - 1) + 3
    for rows, cols in GEMV_SHAPES:
        n = rows * cols
        if n < U:
            rows = (U + cols - 1) // cols
        w = synth.with_distinct_count(rows * cols, U, seed=[41, b, cols],
                                      exponents=synth.finite_exponents(U)).reshape(rows, cols)
        x = synth.activation_bf16(cols, seed=[42, cols])
        _gemv_check(env, oracle_mod, w, x)


def test_gemv_integer_exact(env, oracle_mod):
    rng = np.random.default_rng(43)
    for rows, cols in [(129, 4096), (70, 1000), (1024, 1024)]:
        Wi = rng.integers(-8, 8, size=(rows, cols))
        xi = rng.integers(-4, 5, size=cols)
        _gemv_check(env, oracle_mod, _int_bf16(Wi), _int_bf16(xi), exact=True)


def test_gemv_one_hot_returns_column(env, oracle_mod):
    w = synth.gaussian_bf16((300, 4096), 0.02, seed=[44])
    for k in (0, 129, 4095):
        x = np.zeros(4096, dtype=np.float32)
        x[k] = 1.0
        got, _ = _gemv_check(env, oracle_mod, w, _int_bf16(x), exact=True)
        assert np.array_equal(got, synth.bf16_to_f32(w[:, k]).astype(np.float64))


def test_gemv_constant_tensor(env, oracle_mod):
    w = np.full((50, 640), 0x4040, dtype=np.uint16)
    xi = np.random.default_rng(45).integers(-3, 4, size=640)
    _gemv_check(env, oracle_mod, w, _int_bf16(xi), exact=True)


def test_gemv_zero_cols(env):
    torch, cbk = env
    c = cbk.encode(np.zeros((8, 0), dtype=np.uint16), rows=8, cols=0).to("cuda")
    y = torch.full((8,), 5.0, device="cuda")
    x = torch.zeros(8, dtype=torch.bfloat16, device="cuda")[:0]
    cbk.gemv(c, x, y=y)
    torch.cuda.synchronize()
    assert not y.any()


@pytest.mark.parametrize("cfg", [1, 2])
def test_gemv_workload_full_size(env, oracle_mod, cfg):
    t = synth.WORKLOADS[cfg][0][0]
    w = synth.workload_tensor(cfg, 0, t)
    x = synth.workload_x(cfg, t.cols)[0]
    _gemv_check(env, oracle_mod, w, x)


def test_gemv_mlp_full_size(env, oracle_mod):
    for t in synth.WORKLOADS[3][0]:
        if t.name in ("gate", "down"):
            w = synth.workload_tensor(3, 0, t)
            x = synth.workload_x(3, t.cols)[0]
            rows = np.random.default_rng(46).choice(t.rows, 512, replace=False)
            _gemv_check(env, oracle_mod, w, x, rows=rows)



@pytest.mark.parametrize("rows,cols", [(16421, 1024), (17000, 640), (20000, 8192 + 64)])
def test_gemv_dynamic_rows_every_row(env, oracle_mod, rows, cols):
    """Enough rows per wave (at least 8 on a 256-CU device) for the waves of a workgroup to claim
    rows dynamically: every row is produced exactly once, checked against the oracle in full."""
    w = synth.gaussian_bf16((rows, cols), 0.02, seed=[81, rows, cols])
    x = synth.activation_bf16(cols, seed=[82, cols])
    _gemv_check(env, oracle_mod, w, x)


def test_gemv_70b_shapes_sampled(env, oracle_mod):
    """70B-shaped tensors at full size (one of each shape), 128 sampled rows each."""
    for t in synth.WORKLOADS[5][0]:
        if t.name in ("q", "k", "gate", "down"):
            w = synth.workload_tensor(5, 0, t)
            x = synth.workload_x(5, t.cols)[0]
            rows = np.random.default_rng(47).choice(t.rows, 128, replace=False)
            _gemv_check(env, oracle_mod, w, x, rows=rows)


# ----------------------------------------------------------------------------------- GEMM
# GEMM shapes: cols/64 = 10 (steps of 4, 4, 2 units), 32, 13 (odd, M < 16: one partial row tile),
# 64 with 40 rows (few tiles: K is split over workgroups and Y is accumulated with atomics), and a
# ragged K (generic kernel).
GEMM_SHAPES = [(50, 640), (16, 2048), (7, 832), (40, 4096), (23, 393)]


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 8, 9, 12, 16])
def test_gemm_batches(env, oracle_mod, batch):
    for b, U in [(13, 5000), (12, 3000), (8, 200), (3, 7), (16, 40000)]:
        for rows, cols in GEMM_SHAPES:
            n = rows * cols
            if n < U:
                rows = (U + cols - 1) // cols
            w = synth.with_distinct_count(rows * cols, U, seed=[51, b, cols],
                                          exponents=synth.finite_exponents(U)).reshape(rows, cols)
            X = synth.activations_bf16(batch, cols, 52)
            _gemm_check(env, oracle_mod, w, X)


@pytest.mark.parametrize("batch", [2, 5, 8, 12, 16])
@pytest.mark.parametrize("cols", [320, 640])
def test_gemm_partial_step_ignores_next_row_nonfinite(env, oracle_mod, batch, cols):
    """K / 64 is not a multiple of 4 here, so a wave's last step runs past its part of K and its
    unused units hold the next row's first fields.  Every odd row starts with 192 infinite
    weights: the even rows' outputs must still match the oracle (the fast kernels drop those
    units' products instead of multiplying them by zero), and the odd rows are non-finite."""
    torch, cbk = env
    rows = 48
    w = synth.gaussian_bf16((rows, cols), 0.02, seed=[57, batch, cols]).copy()
    w[1::2, :192] = 0x7F80  # +inf
    X = synth.activations_bf16(batch, cols, 58)
    d = cbk.encode(w).to("cuda")
    Y = cbk.gemm_small(d, _up(torch, X, torch.bfloat16))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy().astype(np.float64)
    even = list(range(0, rows, 2))
    ref, absb = _oracle_rows(oracle_mod, w, even, lambda e: oracle_mod.gemm(e, X))
    got = Y[:, even]
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= TOL * absb)
    assert not np.any(np.isfinite(Y[:, 1::2]))


def test_gemm_integer_exact_and_column_equals_gemv(env, oracle_mod):
    torch, cbk = env
    rng = np.random.default_rng(53)
    for batch in (4, 8, 16):
        Wi = rng.integers(-8, 8, size=(200, 2048))
        Xi = rng.integers(-4, 5, size=(batch, 2048))
        w, X = _int_bf16(Wi), _int_bf16(Xi)
        Y = _gemm_check(env, oracle_mod, w, X, exact=True)
        d = cbk.encode(w).to("cuda")
        for j in range(batch):
            y = cbk.gemv(d, _up(torch, X[j], torch.bfloat16)).cpu().numpy()
            assert np.array_equal(y.astype(np.float64), Y[j])


def test_gemm_padded_leading_dimension(env, oracle_mod):
    w = synth.gaussian_bf16((96, 1024), 0.02, seed=[54])
    X = synth.activations_bf16(10, 1024, 54)
    _gemm_check(env, oracle_mod, w, X, ldx=1024 + 24)
    _gemm_check(env, oracle_mod, w, X[:4], ldx=1024 + 3)  # ldx % 8 != 0: generic kernel


def test_gemv_misaligned_x_takes_generic_path(env, oracle_mod):
    torch, cbk = env
    w = synth.gaussian_bf16((64, 512), 0.02, seed=[59])
    x = synth.activation_bf16(512, seed=[60])
    d = cbk.encode(w).to("cuda")
    buf = torch.zeros(520, dtype=torch.bfloat16, device="cuda")
    buf[1:513] = _up(torch, x, torch.bfloat16)
    y = cbk.gemv(d, buf[1:513]).cpu().numpy()
    ref, absb = oracle_mod.gemv(oracle_mod.encode(w), x)
    assert np.all(np.abs(y - ref) <= TOL * absb)


def test_gemm_mlp_batch8_sampled(env, oracle_mod):
    for t in synth.WORKLOADS[3][0]:
        if t.name in ("up", "down"):
            w = synth.workload_tensor(3, 0, t)
            X = synth.workload_x(3, t.cols, batch=8)
            rows = np.random.default_rng(55).choice(t.rows, 96, replace=False)
            _gemm_check(env, oracle_mod, w, X, rows=rows)


def test_gemm_70b_batch16_sampled(env, oracle_mod):
    for t in synth.WORKLOADS[5][0]:
        if t.name in ("v", "o", "up", "down"):
            w = synth.workload_tensor(5, 0, t)
            X = synth.workload_x(5, t.cols, batch=16)
            rows = np.random.default_rng(56).choice(t.rows, 32, replace=False)
            _gemm_check(env, oracle_mod, w, X, rows=rows)



@pytest.mark.parametrize("batch", [8, 16])
def test_gemm_many_tiles_sampled(env, oracle_mod, batch):
    """16384- and 32768-row tensors (1024 and 2048 row tiles), where a 256-CU device gives each
    workgroup 4 and 8 tiles; at 4 tiles K = 768 splits into a 512- and a 256-column part.  Sampled
    rows, the first and the last included, against the oracle."""
    for rows in (16384, 32768):
        w = synth.gaussian_bf16((rows, 768), 0.02, seed=[73, rows])
        X = synth.activations_bf16(batch, 768, 74)
        sample = np.concatenate([[0, rows - 1], np.random.default_rng(75).choice(rows, 254, replace=False)])
        _gemm_check(env, oracle_mod, w, X, rows=sample)

def test_repeated_launches_are_identical(env):
    torch, cbk = env
    w = synth.gaussian_bf16((4096, 4096), 0.02, seed=[57])
    d = cbk.encode(w).to("cuda")
    x = _up(torch, synth.activation_bf16(4096, seed=[58]), torch.bfloat16)
    y0 = cbk.gemv(d, x).clone()
    for _ in range(5):
        assert torch.equal(cbk.gemv(d, x), y0)


# ----------------------------------------------------------------------------- grouped GEMV
def test_gemv_group_matches_oracle_and_single_calls(env, oracle_mod):
    """Tensors sharing x: different row counts and codebooks, a width change mid-list (two
    launches), more than eight tensors (several launches) and one generic-path (b = 0) tensor."""
    torch, cbk = env
    K = 1024
    ws = [synth.gaussian_bf16((r, K), 0.02, seed=[61, i]) for i, r in enumerate([300, 64, 1000, 7, 513])]
    ws.append(synth.with_distinct_count(200 * K, 200, seed=[62], exponents=(120, 130)).reshape(200, K))
    ws += [synth.gaussian_bf16((96, K), 0.02, seed=[63, i]) for i in range(5)]
    ws.append(np.full((33, K), 0x3F80, dtype=np.uint16))
    x = synth.activation_bf16(K, seed=[64])
    xd = _up(torch, x, torch.bfloat16)
    ds = [cbk.encode(w).to("cuda") for w in ws]
    assert len({d.b for d in ds}) >= 3
    ys = cbk.gemv_group(ds, xd)
    torch.cuda.synchronize()
    for w, d, y in zip(ws, ds, ys):
        ref, absb = oracle_mod.gemv(oracle_mod.encode(w), x)
        got = y.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= TOL * absb)
        assert torch.equal(cbk.gemv(d, xd), y)


def test_gemv_group_7b_layer_phases(env, oracle_mod):
    """The q/k/v and gate/up phases of a 7B-shaped layer as grouped launches, sampled rows."""
    torch, cbk = env
    tensors, _ = synth.WORKLOADS[4]
    for names in (("q", "k", "v"), ("gate", "up")):
        group = [t for t in tensors if t.name in names]
        ws = [synth.workload_tensor(4, 0, t) for t in group]
        x = synth.workload_x(4, group[0].cols)[0]
        ds = [cbk.encode(w).to("cuda") for w in ws]
        ys = cbk.gemv_group(ds, _up(torch, x, torch.bfloat16))
        torch.cuda.synchronize()
        rows = np.random.default_rng(65).choice(group[0].rows, 256, replace=False)
        for w, y in zip(ws, ys):
            ref, absb = _oracle_rows(oracle_mod, w, rows, lambda e: oracle_mod.gemv(e, x))
            got = y.cpu().numpy().astype(np.float64)[rows]
            assert np.all(np.abs(got - ref) <= TOL * absb)


@pytest.mark.parametrize("batch", [3, 8, 16])
def test_gemm_group_matches_oracle_and_single_calls(env, oracle_mod, batch):
    """Tensors sharing X: different row counts (a partial tile, a 1024-row tensor next to larger
    ones), padded Y leading dimensions, a width change mid-list (two launches) and more than
    eight tensors (several launches).  Each Y matches the oracle within tolerance (the tile split,
    and with it the summation order, depends on the whole group, so no bitwise match with the
    single call is expected), and the padding columns of Y are left alone."""
    torch, cbk = env
    K = 1024
    rows = [300, 64, 1024, 7, 513]
    ws = [synth.gaussian_bf16((r, K), 0.02, seed=[66, i]) for i, r in enumerate(rows)]
    ws.append(synth.with_distinct_count(200 * K, 200, seed=[67], exponents=(120, 130)).reshape(200, K))
    ws += [synth.gaussian_bf16((96, K), 0.02, seed=[68, i]) for i in range(4)]
    X = synth.activations_bf16(batch, K, 69)
    Xd = _up(torch, X, torch.bfloat16)
    ds = [cbk.encode(w).to("cuda") for w in ws]
    assert len({d.b for d in ds}) >= 2 and len(ds) > 8
    bufs = [torch.full((batch, d.rows + 5), -1.0, dtype=torch.float32, device="cuda") for d in ds]
    Ys = cbk.gemm_group(ds, Xd, Ys=[b[:, :d.rows] for b, d in zip(bufs, ds)])
    torch.cuda.synchronize()
    for w, d, Y, buf in zip(ws, ds, Ys, bufs):
        ref, absb = oracle_mod.gemm(oracle_mod.encode(w), X)
        got = Y.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= TOL * absb)
        single = cbk.gemm_small(d, Xd).cpu().numpy().astype(np.float64)
        assert np.all(np.abs(single - ref) <= TOL * absb)
        assert bool((buf[:, d.rows:] == -1.0).all())  # padding columns untouched


def test_gemm_group_70b_qkv_batch16(env, oracle_mod):
    """The q/k/v phase of a 70B-shaped layer at batch 16 as one grouped launch, sampled rows."""
    torch, cbk = env
    group = [t for t in synth.WORKLOADS[5][0] if t.name in ("q", "k", "v")]
    ws = [synth.workload_tensor(5, 0, t) for t in group]
    X = synth.workload_x(5, group[0].cols, batch=16)
    ds = [cbk.encode(w).to("cuda") for w in ws]
    Ys = cbk.gemm_group(ds, _up(torch, X, torch.bfloat16))
    torch.cuda.synchronize()
    for w, t, Y in zip(ws, group, Ys):
        rows = np.random.default_rng(70).choice(t.rows, 32, replace=False)
        ref, absb = _oracle_rows(oracle_mod, w, rows, lambda e: oracle_mod.gemm(e, X))
        got = Y.cpu().numpy().astype(np.float64)[:, rows]
        assert np.all(np.abs(got - ref) <= TOL * absb)


@pytest.mark.parametrize("b", [14, 15])
def test_gemm_wide_codebooks_fast_path(env, oracle_mod, b):
    """b = 14 and 15: the largest widths whose table still fits the fast kernels' LDS budget
    (a 32 or 64 KB table next to the stages), at batch 5 (VALU) and 16 (MFMA)."""
    U = 2 ** (b - 1) + 11
    for batch in (5, 16):
        for rows, cols in [(40, 1024), (9, 640)]:
            n = max(rows * cols, U)
            rows = (n + cols - 1) // cols
            w = synth.with_distinct_count(rows * cols, U, seed=[71, b, cols],
                                          exponents=synth.finite_exponents(U)).reshape(rows, cols)
            X = synth.activations_bf16(batch, cols, 72)
            _gemm_check(env, oracle_mod, w, X)



# ------------------------------------------------------------------------------- GPU encoder
def _encode_gpu_check(env, w):
    torch, cbk = env
    host = cbk.encode(w.reshape(1, -1))
    dev = torch.from_numpy(np.ascontiguousarray(w.reshape(-1)).view(np.int16)).to("cuda")
    got = cbk.encode_gpu(dev, rows=1, cols=w.size)
    torch.cuda.synchronize()
    assert (got.U, got.b) == (host.U, host.b), (w.size, got.U, host.U)
    assert np.array_equal(got.codebook.cpu().numpy().view(np.uint16), host.codebook)
    assert np.array_equal(got.words.cpu().numpy().view(np.uint32), host.words), (w.size, host.U)
    return got


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 31, 32, 33, 2047, 2048, 2049, 2048 * 64 + 5, 100003])
def test_encode_gpu_matches_host_ragged_lengths(env, n):
    """Empty input and ragged lengths around the 8-pattern load chunk and the 32-field and 2048-field pack blocks."""
    w = synth.gaussian_bf16((n,), 0.02, seed=[91, n])
    _encode_gpu_check(env, w)


@pytest.mark.parametrize("U", [1, 2, 3, 255, 256, 257, 4097, 32768, 32769, 65536])
def test_encode_gpu_matches_host_every_width(env, U):
    """Distinct counts at both ends of the widths, up to every 16-bit pattern (+0/-0, NaNs)."""
    n = max(U, 50000)
    w = synth.with_distinct_count(n, U, seed=[92, U])
    got = _encode_gpu_check(env, w)
    assert got.U == U


def test_encode_gpu_workload_tensor_and_oracle(env, oracle_mod):
    """A 4096^2 tensor of the attention workload: equal to the host encoder and to the oracle, and
    the device result decodes back to the input."""
    torch, cbk = env
    w = synth.workload_tensor(1, 0, synth.WORKLOADS[1][0][0])
    got = _encode_gpu_check(env, w)
    e = oracle_mod.encode(w)
    assert got.U == e.U and got.b == e.b
    n = w.size
    assert np.array_equal(got.words.cpu().numpy().view(np.uint32)[:oracle_mod.stream_words(n, e.b)], e.words)
    out = cbk.decode_bf16(got)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.shape), w)


def test_decode_group_bit_exact(env):
    """cbk_decode_group over sixteen tensors: runs of one width split by a width change, a run of
    nine (eight, then one), an empty tensor, b = 0, a misaligned output (the generic kernel) and
    ragged lengths; every output equals the input patterns, as the single-tensor call's does."""
    torch, cbk = env
    shapes = [(300, 1000, 5000), (1, 7, 3), (4096, 64, 5000), (0, 64, 1), (17, 333, 1), (9, 1000, 5000),
              (70, 130, 2), (257, 512, 2), (100, 100, 2), (33, 65, 2), (64, 64, 2), (5, 999, 2),
              (3, 64, 2), (40, 72, 2), (2, 8, 2), (11, 1024, 2)]
    ws, ds = [], []
    for i, (r, c, U) in enumerate(shapes):
        n = r * c
        w = (synth.with_distinct_count(n, min(U, n), seed=[110, i]) if n else np.zeros(0, np.uint16)).reshape(r, c)
        ws.append(w)
        ds.append(cbk.encode(w).to("cuda"))
    print(f"decode group of {len(ws)} tensors, widths {[d.b for d in ds]}", flush=True)
    outs = [torch.full((d.rows, d.cols), float("nan"), dtype=torch.bfloat16, device="cuda") for d in ds]
    # tensor 6's output starts 2 bytes into its buffer: not 16-byte aligned
    spare = torch.full((ds[6].rows * ds[6].cols + 8,), -1, dtype=torch.int16, device="cuda")
    outs[6] = spare[1:1 + ds[6].rows * ds[6].cols].view(torch.bfloat16).view(ds[6].rows, ds[6].cols)
    cbk.decode_group(ds, outs=outs)
    torch.cuda.synchronize()
    for i, (w, o) in enumerate(zip(ws, outs)):
        assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), w), (i, w.shape)
    assert int(spare[0]) == -1 and bool((spare[1 + ws[6].size:].cpu() == -1).all())


def test_encode_gpu_group_matches_host(env):
    """cbk_encode_gpu_group over eleven tensors (a run of eight, then three reusing the first
    workspaces): empty and ragged lengths, widths from 0 to 16 (every 16-bit pattern) and a
    workload tensor; each job's codebook, U, b and words equal the host encoder's."""
    torch, cbk = env
    ws = [synth.gaussian_bf16((n,), 0.02, seed=[97, n]) for n in (0, 1, 7, 2049, 100003)]
    ws += [synth.with_distinct_count(max(U, 50000), U, seed=[98, U]) for U in (1, 2, 257, 32769, 65536)]
    ws.append(synth.workload_tensor(1, 0, synth.WORKLOADS[1][0][0]).reshape(-1))
    print(f"encode group of {len(ws)} tensors", flush=True)
    devs = [torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to("cuda") for w in ws]
    cbs = [torch.empty(65536, dtype=torch.int16, device="cuda") for _ in ws]
    words = [torch.full((max(cbk.words_for(w.size, 16), 4),), -1, dtype=torch.int32, device="cuda") for w in ws]
    metas = [torch.full((2,), -1, dtype=torch.int32, device="cuda") for _ in ws]
    space = torch.empty(8 * cbk.encode_gpu_workspace_bytes(), dtype=torch.uint8, device="cuda")
    cbk.encode_gpu_group_launch(devs, space, cbs, words, metas)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        host = cbk.encode(w.reshape(1, -1))
        U, b = (int(v) for v in metas[i].cpu().tolist())
        assert (U, b) == (host.U, host.b), (i, w.size)
        assert np.array_equal(cbs[i][:U].cpu().numpy().view(np.uint16), host.codebook), i
        assert np.array_equal(words[i][:cbk.words_for(w.size, b)].cpu().numpy().view(np.uint32), host.words), i


@pytest.mark.parametrize("rows,K,U", [([1, 4097, 33], 1024, 600), ([8193, 1, 2, 1023], 640, 600),
                                      ([300, 7], 4160, 4500), ([2049, 1025, 513, 3], 8192, 4500),
                                      ([100, 31, 7, 1], 12288, 4500)])
def test_gemv_group_ragged_rows_every_row(env, oracle_mod, rows, K, U):
    """Groups of 2-4 tensors of one width: row counts that do not divide over the waves or the
    workgroups, tensors of one row, rows of one, two and three wave steps.  Every row of every
    tensor against the oracle, and bit for bit against the single-tensor call."""
    torch, cbk = env
    ws = [synth.with_distinct_count(r * K, U, seed=[95, i, r], exponents=synth.finite_exponents(U)).reshape(r, K)
          for i, r in enumerate(rows)]
    x = synth.activation_bf16(K, seed=[96, K])
    xd = _up(torch, x, torch.bfloat16)
    ds = [cbk.encode(w).to("cuda") for w in ws]
    assert len({d.b for d in ds}) == 1
    ys = cbk.gemv_group(ds, xd)
    torch.cuda.synchronize()
    for w, d, y in zip(ws, ds, ys):
        ref, absb = oracle_mod.gemv(oracle_mod.encode(w), x)
        got = y.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= TOL * absb)
        assert torch.equal(cbk.gemv(d, xd), y)
