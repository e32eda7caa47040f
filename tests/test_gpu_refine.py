"""Parity of the calibrated init and Value Refinement (HIP path, through the
C-ABI) with the fp64 CPU oracle.

Bars: indices, budgets and permutations bit-exact; the Hessian, the
refinement system G and its right-hand side within a normwise relative error
of 1e-12 (fp64 throughout, only the summation order differs); dense and
refined values c within 1e-6 (fp32 rounding of fp64 solutions of systems
whose condition stays far below 1e6 at these inputs).
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantization_aware_sparse_amd as qq
    return qq


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def _dwq(d_out, d_in, seed):
    rng = np.random.default_rng(seed)
    return (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)


def oracle_calibrated(dwq, X, p, m=3, t=1.0, damp=0.0, rows=None):
    """The oracle's calibrated init; refined values only for `rows` (all by
    default), by solving those rows' systems."""
    Hs = O.damped(O.hessian(synth.act_to_f64(X)), damp)
    d_out, d_in = dwq.shape
    C = O.transform(dwq)
    w = O.activation_error_norms(dwq, Hs)
    budgets = O.adaalloc(w, p, d_in, m, t)
    margin = O.adaalloc_margins(w, p, d_in, m, t)
    row_ptr, E = O.select(C, budgets)
    c0 = O.values(C, E)
    G, Q = O.refine_system(dwq, Hs)
    rows = np.arange(d_out) if rows is None else np.asarray(rows)
    sub_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    sub_ptr[1:] = np.cumsum(budgets[rows])
    sub_E = np.concatenate([E[row_ptr[i]:row_ptr[i + 1]] for i in rows]) if len(E) else E
    x, ok = O.refine_values(G, Q[rows], sub_ptr, sub_E)     # sub-row n is row rows[n]
    return dict(Hs=Hs, w=w, budgets=budgets, margin=margin, row_ptr=row_ptr, E=E, c0=c0, G=G,
                rhs=Q[E[:, 0], E[:, 1]] if len(E) else np.zeros(0), rows=rows,
                sub_ptr=sub_ptr, x=x, ok=ok, C=C)


def check_init(ref, got):
    for key in ("row_ptr", "E"):
        assert np.array_equal(host(got[key]), ref[key]), key
    col_ptr, perm = O.csc(ref["E"], ref["G"].shape[0])
    assert np.array_equal(host(got["col_ptr"]), col_ptr)
    assert np.array_equal(host(got["csc_perm"]), perm)
    assert O.rel_err(host(got["c"]), ref["c0"]) <= 1e-6
    assert O.rel_err(host(got["G"]), ref["G"]) <= 1e-12
    if len(ref["rhs"]):
        assert O.rel_err(host(got["rhs"]), ref["rhs"]) <= 1e-12


def check_refined(ref, c_got):
    """Refined rows against the oracle's solves; rows it finds not definite
    keep the dense values."""
    for n, i in enumerate(ref["rows"]):
        a, b = ref["row_ptr"][i], ref["row_ptr"][i + 1]
        got = c_got[a:b]
        if ref["ok"][n]:
            want = ref["x"][ref["sub_ptr"][n]:ref["sub_ptr"][n + 1]]
            assert O.rel_err(got, want) <= 1e-6, (i, O.rel_err(got, want))
        else:
            assert np.array_equal(got, ref["c0"][a:b]), i


# ------------------------------------------------------------------ Hessian
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("N,d_in", [(1, 2), (5, 4), (37, 16), (300, 128), (1000, 256),
                                    (129, 1024), (17, 8192)])
def test_hessian_parity(q, act, N, d_in):
    say("hessian", act, N, d_in)
    X = synth.make_calibration(d_in, N, seed=N + d_in, act=act)
    got = q.qwha_hessian(to_dev(X))
    torch.cuda.synchronize()
    ref = O.hessian(synth.act_to_f64(X))
    assert O.rel_err(host(got), ref) <= 1e-13
    assert np.array_equal(host(got), host(got).T)     # mirrored tiles: exactly symmetric


def test_hessian_accumulates_batches_and_empty_batch(q):
    X = synth.make_calibration(256, 700, seed=3, act="bf16")
    Hs = q.qwha_hessian(to_dev(X[:300]))
    q.qwha_hessian(to_dev(X[300:]), Hs, accumulate=True)
    q.qwha_hessian(to_dev(X[:0]), Hs, accumulate=True)      # N = 0 leaves it
    torch.cuda.synchronize()
    assert O.rel_err(host(Hs), O.hessian(synth.act_to_f64(X))) <= 1e-13
    Z = q.qwha_hessian(to_dev(X[:0]))                        # N = 0, fresh: zeros
    torch.cuda.synchronize()
    assert not host(Z).any()


# ------------------------------------------------------------------ init + refine
@pytest.mark.parametrize("d_out,d_in,p,m,N", [
    (37, 2, 40, 1, 8), (5, 4, 12, 2, 16), (64, 16, 300, 3, 64), (300, 64, 2500, 3, 200),
    (129, 128, 9000, 3, 400), (17, 1024, 2000, 3, 2048), (40, 256, 40 * 256, 3, 600),
    (7, 4096, 1500, 3, 4500)])
def test_calibrated_init_and_refine(q, d_out, d_in, p, m, N):
    say("calibrated", d_out, d_in, p, m, N)
    dwq = _dwq(d_out, d_in, d_out + 7 * d_in)
    X = synth.make_calibration(d_in, N, seed=d_in + N, act="f32")
    ref = oracle_calibrated(dwq, X, p, m)
    if p < d_out * d_in:     # the full budget fixes every row at d_in
        assert np.min(ref["margin"]) > 1e-9, "ambiguous budget at this seed"
    Hs = q.qwha_hessian(to_dev(X))
    got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, p, m)
    torch.cuda.synchronize()
    check_init(ref, got)
    c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                     got["c"].clone())
    torch.cuda.synchronize()
    assert host(status).tolist() == [int(np.sum(~ref["ok"])), 0]
    check_refined(ref, host(c))


def test_refine_not_definite_rows_and_damping(q):
    # 6 calibration tokens: rows with more than 6 positions have a singular
    # G[S,S]; they keep their dense values. Damping makes them solvable.
    d_out, d_in = 24, 64
    dwq = _dwq(d_out, d_in, 5)
    X = synth.make_calibration(d_in, 6, seed=9, act="f32")
    Hs = q.qwha_hessian(to_dev(X))
    for damp in (0.0, 0.01):
        say("singular, damp", damp)
        ref = oracle_calibrated(dwq, X, 200, 3, damp=damp)
        assert np.min(ref["margin"]) > 1e-9
        got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, 200, 3, damp=damp)
        torch.cuda.synchronize()
        check_init(ref, got)
        c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                         got["c"].clone())
        torch.cuda.synchronize()
        if damp == 0.0:
            assert (~ref["ok"]).sum() > 0
        else:
            assert ref["ok"].all()
        assert host(status).tolist() == [int(np.sum(~ref["ok"])), 0]
        check_refined(ref, host(c))


def test_refine_skips_rows_that_do_not_fit_the_workspace(q):
    d_out, d_in = 30, 128
    dwq = _dwq(d_out, d_in, 12)
    X = synth.make_calibration(d_in, 500, seed=13, act="f32")
    ref = oracle_calibrated(dwq, X, 1500, 3)
    Hs = q.qwha_hessian(to_dev(X))
    got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, 1500, 3)
    torch.cuda.synchronize()
    check_init(ref, got)
    rp = ref["row_ptr"].astype(np.int64)
    tri = (np.diff(rp) + 1) * (np.diff(rp) + 2) // 2
    header = ((8 * (d_out + 1) + 255) // 256) * 256
    full = q.refine_workspace_bytes(got["row_ptr"])
    assert full == header + 8 * int(tri.sum())
    cap = int(tri[:d_out // 2].sum()) + 5               # room for the first half only
    ws = q.workspace(header + 8 * cap, DEV)
    c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                     got["c"].clone(), ws=ws)
    torch.cuda.synchronize()
    ends = np.cumsum(tri)
    fits = ends <= cap
    assert host(status).tolist() == [0, int(np.sum(~fits))]
    c = host(c)
    for i in range(d_out):
        a, b = rp[i], rp[i + 1]
        if fits[i]:
            want = ref["x"][ref["sub_ptr"][i]:ref["sub_ptr"][i + 1]]
            assert O.rel_err(c[a:b], want) <= 1e-6
        else:
            assert np.array_equal(c[a:b], ref["c0"][a:b])


def test_refine_twice_in_a_row_reuses_the_workspace(q):
    # a larger then a smaller problem through one workspace
    big = (_dwq(80, 256, 1), synth.make_calibration(256, 700, seed=2, act="bf16"), 2500)
    small = (_dwq(9, 64, 3), synth.make_calibration(64, 100, seed=4, act="bf16"), 60)
    ws = q.workspace(64 << 20, DEV)
    for dwq, X, p in (big, small):
        say("reuse", dwq.shape, p)
        ref = oracle_calibrated(dwq, X, p, 3)
        Hs = q.qwha_hessian(to_dev(X))
        got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, p, 3)
        c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                         got["c"].clone(), ws=ws)
        torch.cuda.synchronize()
        assert host(status).tolist() == [0, 0]
        check_refined(ref, host(c))


def test_refined_values_lower_the_layer_output_error(q):
    d_out, d_in = 64, 256
    dwq = _dwq(d_out, d_in, 21)
    X = synth.make_calibration(d_in, 1024, seed=22, act="f32")
    Hs = q.qwha_hessian(to_dev(X))
    got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, 2000, 3)
    c_dense = got["c"].clone()
    c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                     got["c"].clone())
    torch.cuda.synchronize()
    E = host(got["E"])
    e_dense = O.layer_output_error(dwq, X, E, host(c_dense))
    e_ref = O.layer_output_error(dwq, X, E, host(c))
    say("layer output error", e_dense, e_ref)
    assert e_ref < 0.9 * e_dense


@pytest.mark.parametrize("cfg,N", [("c2", 8192)])
def test_calibrated_full_config(q, cfg, N):
    spec = synth.config_specs(cfg)[0]
    layer = synth.make_layer(spec, seed=0)
    X = synth.make_calibration(spec.d_in, N, seed=1, act="bf16")
    rows = np.random.default_rng(5).choice(spec.d_out, size=48, replace=False)
    say("calibrated full config", cfg, N)
    ref = oracle_calibrated(layer.dwq, X, spec.p, 3, rows=np.sort(rows))
    assert np.min(ref["margin"]) > 1e-9, "ambiguous budget at this seed"
    Hs = q.qwha_hessian(to_dev(X))
    got = q.qwha_init_select_calibrated(to_dev(layer.dwq), Hs, spec.p, 3)
    torch.cuda.synchronize()
    assert O.rel_err(host(Hs), ref["Hs"]) <= 1e-13
    check_init(ref, got)
    c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                     got["c"].clone())
    torch.cuda.synchronize()
    assert host(status).tolist() == [0, 0]
    check_refined(ref, host(c))
