"""Parity of the HIP path (through the C-ABI) with the fp64 CPU oracle.

Bars (tests/bars.py): indices / budgets / permutations bit-exact; fp32
outputs (dW, c, dc, and y / dx with fp32 activations) within 1e-5 of the
largest reference entry; bf16 outputs element by element within
2^-8 |b| + 1e-5 max|b| (one bf16 rounding of an fp32 sum). Every output is
compared whole, at the small shapes and at the full layer configurations
(the same launch configuration bench.py times).
"""

import numpy as np
import pytest

import oracle as O
import synth
from tests.bars import assert_act_close, assert_f32_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def q():
    _need_gpu()
    import quantization_aware_sparse_amd as qq
    return qq


def say(*a):
    print(*a, flush=True)


DEV = "cuda:0"


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_np(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def init_both(q, dwq, p, m=3, t=1.0):
    ref = O.init_select(dwq, p, m=m, t=t, with_diagnostics=True)
    got = q.qwha_init_select(to_dev(dwq), p, m, t)
    torch.cuda.synchronize()
    return ref, got


def assert_init_equal(ref, got):
    for key in ("row_ptr", "E", "col_ptr", "csc_perm"):
        a = got[key].cpu().numpy()
        assert a.shape == ref[key].shape, key
        if not np.array_equal(a, ref[key]):
            bad = np.nonzero((a != ref[key]).reshape(len(a), -1).any(1))[0][:5]
            raise AssertionError(f"{key} differs at {bad}")
    assert O.rel_err(got["c"].cpu().numpy(), ref["c"]) <= 1e-6


# ------------------------------------------------------------------ FWHT
@pytest.mark.parametrize("log_n", list(range(1, 15)))
@pytest.mark.parametrize("dts", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"),
                                 ("bf16", "bf16")])
def test_fwht_parity(q, log_n, dts):
    n = 1 << log_n
    rows = 37 if n <= 4096 else 5
    say("fwht", n, dts, rows)
    rng = np.random.default_rng(log_n)
    a = rng.standard_normal((rows, n)).astype(np.float32)
    if dts[0] == "bf16":
        a = synth.f32_to_bf16_bits(a)
    x = to_dev(a)
    out_dt = torch.float32 if dts[1] == "f32" else torch.bfloat16
    scale = 1.0 / n
    y = q.qwha_fwht(x, scale, out_dtype=out_dt)
    torch.cuda.synchronize()
    ref = synth.act_to_f64(a) @ O.sylvester(n) * scale
    assert_act_close(to_np(y), ref, dts[1], "fwht")


# ------------------------------------------------------------------ init
def _edge_dwq(d_out, d_in, seed):
    rng = np.random.default_rng(seed)
    a = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    return a


@pytest.mark.parametrize("d_out,d_in,p,m", [
    (37, 2, 40, 1), (5, 4, 12, 2), (64, 16, 300, 3), (300, 64, 2500, 3),
    (129, 128, 9000, 3), (17, 1024, 2000, 3), (3, 8192, 900, 3), (2, 16384, 1000, 3),
    (64, 256, 64 * 256, 3), (50, 512, 150, 3),
    # more rows than the allocator's threads: several rows (and budget
    # values) per thread, the last threads with none
    (1025, 128, 20000, 3), (2500, 64, 30000, 3), (4100, 32, 50000, 3),
    # more than 64 rows per CSC chunk: the row-at-a-time placement
    (20000, 8, 80000, 3)])
def test_init_select_edges(q, d_out, d_in, p, m):
    say("init edge", d_out, d_in, p, m)
    dwq = _edge_dwq(d_out, d_in, d_out + d_in)
    ref, got = init_both(q, dwq, p, m)
    assert_init_equal(ref, got)


def test_init_select_ties_zero_rows_and_bounds(q):
    # spike rows (every |C| equal: ties to the lower column), all-zero rows
    # (w = 0: the floor binds), one dominant row (the cap binds)
    d_out, d_in = 40, 64
    dwq = _edge_dwq(d_out, d_in, 7) * 0.01
    dwq[3] = 0.0
    dwq[3, 9] = 0.5
    dwq[11] = 0.0
    dwq[12] = 0.0
    dwq[20] = 50.0 * np.sign(dwq[20] + 1e-9)
    dwq[30] = 0.0
    dwq[30, 0] = -0.25
    say("init ties/zero/cap")
    ref, got = init_both(q, dwq, 1500, 3)
    assert ref["budgets"][20] == d_in
    assert abs(int(ref["budgets"][11]) - int(ref["budgets"][12])) <= 1
    assert_init_equal(ref, got)


@pytest.mark.parametrize("d_in", [64, 1024, 3072])
def test_init_select_wide_range_ties_and_cap(q, d_in):
    """Selection edge rows in both selection orders (rows below 1024 columns
    go back to natural order; from 1024 columns, and for the three blocks of
    1024 of a 3072-wide row, the selection runs on the transform's order):
    rows 5 and 6 have three large |C| and the rest about 20 octaves below, so
    the k-th key lies past the radix select's first-level bins and the
    bisection decides; row 3 is a spike (|C| flat: the boundary inside a run
    of ties, lowest columns first); rows 11 and 12 are zero (the floor); row
    20 dominates (the cap: every column taken)."""
    d_out = 40
    N = O.block_size(d_in)
    dwq = _edge_dwq(d_out, d_in, 7 + d_in) * 0.01
    n0 = float(np.median(np.linalg.norm(dwq, axis=1)))
    for i in (5, 6):
        L = 4 * n0 * np.sqrt(N / 3) * (1 + 0.1 * i)
        C = L * 1e-6 * (1.0 + np.arange(d_in) / d_in)
        C[[3, d_in // 2, d_in - 1]] = L
        dwq[i] = (O.wht(C[None, :], d_in)[0] / N).astype(np.float32)
    dwq[3] = 0.0
    dwq[3, 9] = 4 * n0
    dwq[11] = 0.0
    dwq[12] = 0.0
    dwq[20] = 50.0 * np.sign(dwq[20] + 1e-9)
    p = d_in + d_out * d_in // 8
    say("init wide/ties/cap", d_in, p)
    ref, got = init_both(q, dwq, p, 3)
    b = ref["budgets"]
    assert b[20] == d_in and b[11] >= 3 and b[12] >= 3
    for i in (5, 6):   # the k-th key sits more than 16 octaves below the largest
        a = np.sort(np.abs(ref["C"][i]))[::-1]
        assert 3 < b[i] < d_in and np.log2(a[0] / a[b[i] - 1]) > 16
    assert np.min(ref["budget_margin"]) > 1e-9
    gap = ref["boundary_gap"]
    assert not np.any((gap > 0) & (gap < 1e-9))
    assert_init_equal(ref, got)


def test_init_select_temperature_two(q):
    dwq = _edge_dwq(100, 128, 3)
    say("init t=2")
    ref, got = init_both(q, dwq, 3000, 3, t=2.0)
    # the seed is chosen so that no share sits within fp64 rounding of an
    # integer (where a different summation order could move a budget)
    assert np.min(ref["budget_margin"]) > 1e-9, "ambiguous budget at this seed"
    gap = ref["boundary_gap"]
    assert not np.any((gap > 0) & (gap < 1e-9)), "ambiguous selection at this seed"
    assert_init_equal(ref, got)


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
def test_init_select_configs(q, cfg):
    for spec in synth.config_specs(cfg):
        say("init config", spec.name)
        layer = synth.make_layer(spec, seed=0)
        ref, got = init_both(q, layer.dwq, spec.p, 3)
        amb_gap = np.sum((ref["boundary_gap"] > 0) & (ref["boundary_gap"] < 1e-9))
        amb_budget = np.sum(ref["budget_margin"] < 1e-9)
        assert amb_gap == 0 and amb_budget == 0, "ambiguous rows at this seed"
        assert_init_equal(ref, got)


# ------------------------------------------------------------------ global selection
def global_both(q, dwq, p, strategy, seed=0):
    ref = O.init_select_global(dwq, p, strategy, seed)
    got = q.qwha_init_select_global(to_dev(dwq), p, strategy, seed)
    torch.cuda.synchronize()
    return ref, got


def magnitude_boundary_ambiguous(ref, p):
    """True when the p-th and (p+1)-th largest |C| differ by less than the
    rounding of an fp64 transform (different summation orders could swap
    them); exact ties (gap 0) are decided by position on both sides."""
    a = np.sort(np.abs(ref["C"]).ravel())[::-1]
    if p == 0 or p >= a.size:
        return False
    gap = a[p - 1] - a[p]
    return 0 < gap <= 1e-12 * max(a[0], 1e-300)


@pytest.mark.parametrize("strategy", ["magnitude", "random"])
@pytest.mark.parametrize("d_out,d_in,p", [
    (37, 2, 40), (5, 4, 0), (5, 4, 20), (5, 4, 1), (64, 16, 300), (300, 64, 2500),
    (129, 128, 9000), (17, 1024, 2000), (3, 8192, 900), (2, 16384, 1000), (1, 16384, 16383),
    (64, 256, 64 * 256), (50, 512, 150), (1000, 32, 7)])
def test_init_global_edges(q, strategy, d_out, d_in, p):
    say("init global", strategy, d_out, d_in, p)
    dwq = _edge_dwq(d_out, d_in, 5 * d_out + d_in)
    ref, got = global_both(q, dwq, p, strategy, seed=d_out * 31 + p)
    if strategy == "magnitude":
        assert not magnitude_boundary_ambiguous(ref, p)
    assert_init_equal(ref, got)


def test_init_global_magnitude_ties_across_rows(q):
    # rows that are one spike each have |C| equal to the spike everywhere:
    # the boundary falls inside a run of equal keys spanning several rows,
    # which go in row-major order; an all-zero matrix is one tie of all keys
    d_out, d_in = 24, 64
    dwq = _edge_dwq(d_out, d_in, 11) * 1e-3
    for i, col in ((2, 5), (3, 0), (7, 63), (8, 9), (15, 1)):
        dwq[i] = 0.0
        dwq[i, col] = 0.125 if i % 2 else -0.125
    for p in (40, 64 + 10, 5 * 64 - 1, 5 * 64 + 3):
        say("init global ties", p)
        ref, got = global_both(q, dwq, p, "magnitude")
        assert_init_equal(ref, got)
    zero = np.zeros((9, 32), dtype=np.float32)
    for p in (0, 1, 33, 9 * 32 - 1, 9 * 32):
        say("init global zeros", p)
        ref, got = global_both(q, zero, p, "magnitude")
        assert_init_equal(ref, got)
        assert np.array_equal(got["E"].cpu().numpy()[:, 0] * 32 + got["E"].cpu().numpy()[:, 1],
                              np.arange(p))


@pytest.mark.parametrize("seed", [0, 1, 0x9E3779B97F4A7C15, (1 << 64) - 1])
def test_init_global_random_seeds(q, seed):
    dwq = _edge_dwq(200, 128, 3)
    say("init global random seed", seed)
    ref, got = global_both(q, dwq, 3000, "random", seed)
    assert_init_equal(ref, got)
    # the draw ignores the data: another matrix, same positions
    got2 = q.qwha_init_select_global(to_dev(_edge_dwq(200, 128, 4)), 3000, "random", seed)
    assert torch.equal(got2["E"], got["E"])


@pytest.mark.parametrize("strategy", ["magnitude", "random"])
def test_init_global_workspace_reuse(q, strategy):
    # one workspace for two calls, the second smaller: nothing carries over
    big = _edge_dwq(300, 256, 1)
    small = _edge_dwq(40, 64, 2)
    ws = q.workspace(q.lib.qwha_init_global_workspace_bytes(300, 256, 1 if strategy ==
                                                            "magnitude" else 2), DEV)
    for dwq, p in ((big, 9000), (small, 500), (big, 1)):
        say("init global reuse", strategy, dwq.shape, p)
        ref = O.init_select_global(dwq, p, strategy, 9)
        got = q.qwha_init_select_global(to_dev(dwq), p, strategy, 9, ws=ws)
        torch.cuda.synchronize()
        assert_init_equal(ref, got)


@pytest.mark.parametrize("strategy", ["magnitude", "random"])
@pytest.mark.parametrize("cfg", ["c2", "c4"])
def test_init_global_configs(q, strategy, cfg):
    for spec in synth.config_specs(cfg):
        say("init global config", strategy, spec.name)
        layer = synth.make_layer(spec, seed=0)
        ref, got = global_both(q, layer.dwq, spec.p, strategy, seed=17)
        if strategy == "magnitude":
            assert not magnitude_boundary_ambiguous(ref, spec.p), "ambiguous at this seed"
        assert_init_equal(ref, got)


# ------------------------------------------------------------------ materialize
@pytest.mark.parametrize("d_out,d_in,p", [(37, 2, 40), (300, 64, 2500), (17, 1024, 2000),
                                          (3, 8192, 900), (2, 16384, 1000), (256, 256, 2048),
                                          # more nonzeros per row than the row kernel holds
                                          # in registers (128 at 1024 columns)
                                          (8, 1024, 4000),
                                          # more rows than workgroups (1024 at 4096
                                          # columns, 512 at 8192)
                                          (1500, 4096, 60000), (600, 8192, 30000)])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_materialize(q, d_out, d_in, p, out_dt):
    say("materialize", d_out, d_in, p, out_dt)
    dwq = _edge_dwq(d_out, d_in, 11)
    r = O.init_select(dwq, p, m=1)
    dt = torch.float32 if out_dt == "f32" else torch.bfloat16
    alpha = 0.75
    got = q.qwha_materialize(to_dev(r["row_ptr"]), to_dev(r["E"]), to_dev(r["c"]), d_out, d_in,
                             alpha, out_dtype=dt)
    torch.cuda.synchronize()
    ref = O.materialize(r["E"], r["c"], d_out, d_in, alpha)
    assert_act_close(to_np(got), ref, out_dt, "dW")
    # accumulate mode: dW += alpha F H^-1
    base = np.random.default_rng(1).standard_normal((d_out, d_in)).astype(np.float32)
    acc = to_dev(base)
    q.qwha_materialize(to_dev(r["row_ptr"]), to_dev(r["E"]), to_dev(r["c"]), d_out, d_in,
                       alpha, out=acc, accumulate=True)
    torch.cuda.synchronize()
    assert_f32_close(to_np(acc), base + ref, "dW accumulated")


def test_materialize_full_budget_reconstructs(q):
    d_out, d_in = 16, 128
    dwq = _edge_dwq(d_out, d_in, 5)
    r = O.init_select(dwq, d_out * d_in, m=3)
    got = q.qwha_materialize(to_dev(r["row_ptr"]), to_dev(r["E"]), to_dev(r["c"]), d_out, d_in)
    torch.cuda.synchronize()
    assert_f32_close(to_np(got), dwq.astype(np.float64), "dW")


# ------------------------------------------------------------------ fwd / bwd small
def _small_case(d_out, d_in, p, T, act, seed):
    dwq = _edge_dwq(d_out, d_in, seed)
    r = O.init_select(dwq, p, m=min(3, d_in))
    rng = np.random.default_rng(seed + 1)
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    dy = rng.standard_normal((T, d_out)).astype(np.float32)
    if act == "bf16":
        x, dy = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(dy)
    return r, x, dy


def _dev_adapter(r):
    return {k: to_dev(r[k]) for k in ("row_ptr", "E", "c", "col_ptr", "csc_perm")}


@pytest.mark.parametrize("d_out,d_in,p,T", [
    (256, 256, 2048, 64), (300, 64, 2500, 77), (37, 2, 74, 130), (513, 128, 4000, 129),
    (64, 1024, 6000, 200), (40, 8192, 2000, 9), (3, 16384, 300, 5), (1100, 32, 3300, 1),
    # one block of 64 rows of F holding more nonzeros than a workgroup stages at once
    (64, 128, 1920, 40),
    # more than 256 blocks of 64 rows of F (the backward's per-workgroup run table)
    (16500, 4, 49500, 70)])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fwd_bwd_small(q, d_out, d_in, p, T, act):
    say("fwd/bwd small", d_out, d_in, p, T, act)
    r, x, dy = _small_case(d_out, d_in, p, T, act, d_out + T)
    a = _dev_adapter(r)
    alpha = 1.25
    xt, dyt = to_dev(x), to_dev(dy)
    y = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], alpha)
    dx, dc = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                        alpha)
    torch.cuda.synchronize()
    x64, dy64 = synth.act_to_f64(x), synth.act_to_f64(dy)
    dW = O.materialize(r["E"], r["c"], d_out, d_in, alpha)
    y_ref = O.forward(x64, dW)
    dx_ref, dc_ref = O.backward(x64, dy64, r["E"], r["c"], d_out, d_in, alpha, dW=dW)
    assert_act_close(to_np(y), y_ref, act, "y")
    assert_act_close(to_np(dx), dx_ref, act, "dx")
    assert_f32_close(to_np(dc), dc_ref, "dc")


@pytest.mark.parametrize("d_out,d_in,p,T,act", [(300, 64, 2500, 77, "f32"),
                                                 (513, 128, 4000, 129, "bf16"),
                                                 (37, 192, 600, 33, "bf16")])
def test_saved_activation_path_matches(q, d_out, d_in, p, T, act):
    # qwha_fwd_save / qwha_bwd_saved: the same kernels on the kept z, so the
    # outputs equal the plain calls bit for bit; z is the forward transform
    say("saved activation", d_out, d_in, p, T, act)
    r, x, dy = _small_case(d_out, d_in, p, T, act, d_out + T)
    a = _dev_adapter(r)
    xt, dyt = to_dev(x), to_dev(dy)
    y0 = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 0.9)
    dx0, dc0 = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                          0.9)
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    y1 = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 0.9, z_out=z)
    dx1, dc1 = q.qwha_bwd(None, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                          0.9, z=z)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(dx0, dx1) and torch.equal(dc0, dc1)
    b = O.block_size(d_in)
    z_ref = O.wht(synth.act_to_f64(x), d_in) / b
    assert O.rel_err(to_np(z), z_ref) <= 1e-6


def test_fwd_bwd_accumulate_and_partial_outputs(q):
    say("accumulate")
    r, x, dy = _small_case(300, 64, 2500, 77, "f32", 3)
    a = _dev_adapter(r)
    xt, dyt = to_dev(x), to_dev(dy)
    base_y = np.random.default_rng(2).standard_normal((77, 300)).astype(np.float32)
    base_dx = np.random.default_rng(3).standard_normal((77, 64)).astype(np.float32)
    yt, dxt = to_dev(base_y), to_dev(base_dx)
    q.qwha_fwd(xt, 300, a["row_ptr"], a["E"], a["c"], 1.0, y=yt, accumulate=True)
    q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.0,
               need_dc=False, dx=dxt, accumulate_dx=True)
    _, dc_only = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"],
                            a["csc_perm"], 1.0, need_dx=False)
    torch.cuda.synchronize()
    dW = O.materialize(r["E"], r["c"], 300, 64, 1.0)
    dx_ref, dc_ref = O.backward(x, dy, r["E"], r["c"], 300, 64, 1.0, dW=dW)
    assert_f32_close(to_np(yt), base_y + O.forward(x, dW), "y accumulated")
    assert_f32_close(to_np(dxt), base_dx + dx_ref, "dx accumulated")
    assert_f32_close(to_np(dc_only), dc_ref, "dc")


def test_zero_tokens(q):
    r, x, dy = _small_case(64, 32, 500, 4, "f32", 9)
    a = _dev_adapter(r)
    xt = torch.empty((0, 32), device=DEV)
    dyt = torch.empty((0, 64), device=DEV)
    y = q.qwha_fwd(xt, 64, a["row_ptr"], a["E"], a["c"], 1.0)
    dc = torch.full((500,), 7.0, device=DEV)
    q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.0,
               need_dx=False, dc=dc)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert torch.count_nonzero(dc).item() == 0


def test_backward_deterministic(q):
    say("determinism")
    r, x, dy = _small_case(513, 128, 4000, 300, "bf16", 4)
    a = _dev_adapter(r)
    xt, dyt = to_dev(x), to_dev(dy)
    outs = []
    for _ in range(2):
        dx, dc = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"],
                            a["csc_perm"], 1.0)
        y = q.qwha_fwd(xt, 513, a["row_ptr"], a["E"], a["c"], 1.0)
        torch.cuda.synchronize()
        outs.append((dx.clone(), dc.clone(), y.clone()))
    for u, v in zip(outs[0], outs[1]):
        assert torch.equal(u, v)


def test_autograd_function(q):
    say("autograd")
    r, x, dy = _small_case(256, 256, 2048, 64, "f32", 6)
    a = _dev_adapter(r)
    xt = to_dev(x).requires_grad_(True)
    ct = a["c"].clone().requires_grad_(True)
    y = q.WHAFunction.apply(xt, ct, a["row_ptr"], a["E"], a["col_ptr"], a["csc_perm"], 256, 1.0)
    y.backward(to_dev(dy))
    torch.cuda.synchronize()
    dW = O.materialize(r["E"], r["c"], 256, 256, 1.0)
    dx_ref, dc_ref = O.backward(x, dy, r["E"], r["c"], 256, 256, 1.0, dW=dW)
    assert_f32_close(to_np(y), O.forward(x, dW), "y")
    assert_f32_close(to_np(xt.grad), dx_ref, "dx")
    assert_f32_close(to_np(ct.grad), dc_ref, "dc")


# ------------------------------------------------------------------ full configs
def _check_layer_full(q, spec, layer, x, dy, got_init=None):
    """Init (bit-exact), materialize, fwd and bwd at full size, every output
    compared whole with the oracle. Returns the GPU adapter, the GPU dc and
    the oracle's dc."""
    d_out, d_in, T = spec.d_out, spec.d_in, x.shape[0]
    ref = O.init_select(layer.dwq, spec.p, m=3)
    if got_init is None:
        got_init = q.qwha_init_select(to_dev(layer.dwq), spec.p, 3, 1.0)
    torch.cuda.synchronize()
    assert_init_equal(ref, got_init)
    a = got_init
    xt, dyt = to_dev(x), to_dev(dy)
    dW = q.qwha_materialize(a["row_ptr"], a["E"], a["c"], d_out, d_in, 1.0)
    y = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.0)
    dx, dc = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.0)
    torch.cuda.synchronize()
    del xt, dyt
    dW_ref = O.materialize(ref["E"], ref["c"], d_out, d_in, 1.0)
    assert_f32_close(to_np(dW), dW_ref, f"{spec.name} dW")
    del dW
    x64 = synth.act_to_f64(x)
    dy64 = synth.act_to_f64(dy)
    assert_act_close(to_np(y), O.forward(x64, dW_ref), spec.act, f"{spec.name} y")
    del y
    dx_ref, dc_ref = O.backward(x64, dy64, ref["E"], ref["c"], d_out, d_in, 1.0, dW=dW_ref)
    del x64, dy64
    assert_act_close(to_np(dx), dx_ref, spec.act, f"{spec.name} dx")
    del dx, dx_ref
    assert_f32_close(to_np(dc), dc_ref, f"{spec.name} dc")
    return a, dc, dc_ref


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4"])
def test_full_config_layer(q, cfg):
    spec = synth.config_specs(cfg)[0]
    say("full config", cfg)
    layer = synth.make_layer(spec, seed=0)
    x, dy = synth.make_activations(spec, seed=0)
    _check_layer_full(q, spec, layer, x, dy)


def test_full_config_attention_block_step(q):
    """Training step of the GQA block: four adapters fwd+bwd, c += 1e-3 sign(dc),
    dW re-materialised. The update is checked bitwise against the GPU's own dc
    (an exactly-zero or near-zero dc would make the sign ambiguous); signs must
    agree with the oracle wherever |dc_ref| exceeds the observed error; the
    whole re-materialised dW is checked against the oracle fed the GPU's c'."""
    specs = synth.config_specs("c5")
    for spec in specs:
        say("c5", spec.name)
        layer = synth.make_layer(spec, seed=0)
        x, dy = synth.make_activations(spec, seed=0, x_stream=synth.C5_X_STREAM[spec.name])
        a, dc, dc_ref = _check_layer_full(q, spec, layer, x, dy)
        del x, dy
        dc_np = dc.cpu().numpy()
        err = float(np.max(np.abs(dc_np.astype(np.float64) - dc_ref)))
        sure = np.abs(dc_ref) > err
        assert sure.mean() > 0.99, "too few dc entries with a certain sign"
        assert np.array_equal(np.sign(dc_np[sure]), np.sign(dc_ref[sure])), "dc sign"
        c_old = a["c"].clone()
        q.qwha_sign_update(a["c"], dc, 1e-3)
        torch.cuda.synchronize()
        c_new = a["c"].cpu().numpy()
        assert np.array_equal(c_new, O.sign_update(c_old.cpu().numpy(), dc_np))
        dW2 = q.qwha_materialize(a["row_ptr"], a["E"], a["c"], spec.d_out, spec.d_in, 1.0)
        torch.cuda.synchronize()
        E_np = a["E"].cpu().numpy()
        ref2 = O.materialize(E_np, c_new, spec.d_out, spec.d_in, 1.0)
        assert_f32_close(to_np(dW2), ref2, f"{spec.name} dW after the update")
