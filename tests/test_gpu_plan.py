"""Plans: the SpMM streams built once from the frozen E, with only the
values gathered from c per call (qwha_plan_build, qwha_fwd_plan,
qwha_bwd_plan).

The planned calls run the same kernels on the same streams as the unplanned
ones, so every output is compared bit for bit with qwha_fwd / qwha_fwd_save /
qwha_bwd_saved / qwha_bwd_dz on the same inputs: once after the build, and
again after c has moved (qwha_sign_update) with the plan reused, which is
the case the gather exists for. One shape per dtype is also checked against
the fp64 oracle with the bars of tests/bars.py.
"""

import numpy as np
import pytest

import oracle as O
import synth
from tests.bars import assert_act_close, assert_f32_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantization_aware_sparse_amd as qq
    return qq


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def acts(T, d, act, seed):
    a = np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32)
    return synth.f32_to_bf16_bits(a) if act == "bf16" else a


def adapter(d_out, d_in, p, seed):
    rng = np.random.default_rng(seed)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    r = O.init_select(dwq, p, m=min(3, d_in))
    return r, {k: dev(r[k]) for k in ("row_ptr", "E", "c", "col_ptr", "csc_perm")}


def unplanned(q, a, x, dy, d_out, alpha):
    T, d_in = x.shape
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    y = q.qwha_fwd(x, d_out, a["row_ptr"], a["E"], a["c"], alpha)
    ys = q.qwha_fwd(x, d_out, a["row_ptr"], a["E"], a["c"], alpha, z_out=z)
    dx, dc = q.qwha_bwd(None, dy, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                        alpha, z=z)
    dz, dcz = q.qwha_bwd_dz(z, dy, a["E"], a["c"], a["col_ptr"], a["csc_perm"], alpha)
    return dict(y=y, ys=ys, z=z, dx=dx, dc=dc, dz=dz, dcz=dcz)


def planned(q, plan, a, x, dy, d_out, alpha):
    T, d_in = x.shape
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    y = q.qwha_fwd_plan(x, plan, a["c"], d_out, alpha)
    ys = q.qwha_fwd_plan(x, plan, a["c"], d_out, alpha, z_out=z)
    yz = q.qwha_fwd_plan(None, plan, a["c"], d_out, alpha, z_in=z, act=x.dtype)
    dx, dc = q.qwha_bwd_plan(z, dy, plan, a["c"], alpha)
    dz = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    _, dcz = q.qwha_bwd_plan(z, dy, plan, a["c"], alpha, dz=dz)
    _, dc_only = q.qwha_bwd_plan(z, dy, plan, a["c"], alpha, need_dx=False)
    return dict(y=y, ys=ys, yz=yz, z=z, dx=dx, dc=dc, dz=dz, dcz=dcz, dc_only=dc_only)


def assert_same(u, v):
    torch.cuda.synchronize()
    for k in ("y", "ys", "z", "dx", "dc", "dz", "dcz"):
        assert torch.equal(u[k], v[k]), k
    assert torch.equal(u["ys"], v["yz"]), "forward from the kept z"
    assert torch.equal(u["dc"], v["dc_only"]), "dc without dx"


@pytest.mark.parametrize("d_out,d_in,p,T,act,alpha", [
    (300, 256, 2500, 77, "f32", 1.0),          # ragged tokens and rows
    (513, 1024, 9000, 300, "bf16", 0.75),      # two token tiles, ragged
    (64, 192, 700, 33, "bf16", 2.0),           # block-diagonal transform (3 x 64)
    (1100, 128, 3300, 256, "f32", -1.5),       # one full tile, many rows
    (37, 2, 74, 5, "f32", 1.0)])               # every position of a tiny layer
def test_plan_matches_unplanned_calls(q, d_out, d_in, p, T, act, alpha):
    print("plan", d_out, d_in, p, T, act, alpha, flush=True)
    r, a = adapter(d_out, d_in, p, d_out + d_in + T)
    x, dy = dev(acts(T, d_in, act, 1)), dev(acts(T, d_out, act, 2))
    plan = q.qwha_plan_build(a["row_ptr"], a["E"], a["col_ptr"], a["csc_perm"], d_in, d_out,
                             act=x.dtype)
    assert_same(unplanned(q, a, x, dy, d_out, alpha), planned(q, plan, a, x, dy, d_out, alpha))
    # c moves, E does not: the same plan serves the next step
    for step in range(2):
        _, dc = q.qwha_bwd(x, dy, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                           alpha, need_dx=False)
        q.qwha_sign_update(a["c"], dc, 1e-3 * (step + 1))
        assert_same(unplanned(q, a, x, dy, d_out, alpha),
                    planned(q, plan, a, x, dy, d_out, alpha))


def test_plan_accumulates(q):
    """y += and dx += / dz += on a plan, bit-equal to the unplanned sums."""
    d_out, d_in, p, T = 300, 512, 4000, 140
    print("plan accumulate", flush=True)
    r, a = adapter(d_out, d_in, p, 11)
    x, dy = dev(acts(T, d_in, "bf16", 3)), dev(acts(T, d_out, "bf16", 4))
    plan = q.qwha_plan_build(a["row_ptr"], a["E"], a["col_ptr"], a["csc_perm"], d_in, d_out,
                             act=x.dtype)
    y0 = dev(acts(T, d_out, "bf16", 5))
    dx0 = dev(acts(T, d_in, "bf16", 6))
    dz0 = torch.from_numpy(np.random.default_rng(7).standard_normal((T, d_in))
                           .astype(np.float32)).to(DEV)
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    y_u = q.qwha_fwd(x, d_out, a["row_ptr"], a["E"], a["c"], 0.5, y=y0.clone(), accumulate=True,
                     z_out=z)
    y_p = q.qwha_fwd_plan(x, plan, a["c"], d_out, 0.5, y=y0.clone(), accumulate=True)
    dx_u, _ = q.qwha_bwd(None, dy, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                         0.5, z=z, dx=dx0.clone(), accumulate_dx=True)
    dx_p, _ = q.qwha_bwd_plan(z, dy, plan, a["c"], 0.5, dx=dx0.clone(), accumulate_dx=True)
    dz_u, _ = q.qwha_bwd_dz(z, dy, a["E"], a["c"], a["col_ptr"], a["csc_perm"], 0.5,
                            dz=dz0.clone(), accumulate_dz=True)
    dz_p, _ = q.qwha_bwd_plan(z, dy, plan, a["c"], 0.5, dz=dz0.clone(), accumulate_dz=True)
    torch.cuda.synchronize()
    assert torch.equal(y_u, y_p)
    assert torch.equal(dx_u, dx_p)
    assert torch.equal(dz_u, dz_p)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_plan_against_oracle(q, act):
    """Planned forward and backward after one coefficient update, against the
    fp64 oracle on the updated c."""
    d_out, d_in, p, T, alpha = 700, 512, 6000, 270, 1.25
    print("plan oracle", act, flush=True)
    r, a = adapter(d_out, d_in, p, 21)
    xa, dya = acts(T, d_in, act, 8), acts(T, d_out, act, 9)
    x, dy = dev(xa), dev(dya)
    plan = q.qwha_plan_build(a["row_ptr"], a["E"], a["col_ptr"], a["csc_perm"], d_in, d_out,
                             act=x.dtype)
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    q.qwha_fwd_plan(x, plan, a["c"], d_out, alpha, z_out=z)
    _, dc = q.qwha_bwd_plan(z, dy, plan, a["c"], alpha, need_dx=False)
    q.qwha_sign_update(a["c"], dc, 1e-2)
    y = q.qwha_fwd_plan(x, plan, a["c"], d_out, alpha, z_out=z)
    dx, dc = q.qwha_bwd_plan(z, dy, plan, a["c"], alpha)
    torch.cuda.synchronize()
    c_now = a["c"].cpu().numpy()
    x64, dy64 = synth.act_to_f64(xa), synth.act_to_f64(dya)
    dW = O.materialize(r["E"], c_now, d_out, d_in, alpha)
    dx_ref, dc_ref = O.backward(x64, dy64, r["E"], c_now, d_out, d_in, alpha, dW=dW)
    assert_act_close(host(y), O.forward(x64, dW), act, "y")
    assert_act_close(host(dx), dx_ref, act, "dx")
    assert_f32_close(host(dc), dc_ref, "dc")


@pytest.mark.parametrize("adt", ["f32", "bf16"])
def test_plan_zero_tokens(q, adt):
    """T = 0: no output rows; dc is all zeros, written through the plan's map."""
    d_out, d_in, p = 300, 256, 2500
    act = torch.bfloat16 if adt == "bf16" else torch.float32
    r, a = adapter(d_out, d_in, p, 31)
    plan = q.qwha_plan_build(a["row_ptr"], a["E"], a["col_ptr"], a["csc_perm"], d_in, d_out,
                             act=act)
    z = torch.empty((0, d_in), dtype=torch.float32, device=DEV)
    dy = torch.empty((0, d_out), dtype=act, device=DEV)
    dc = torch.full((p,), 7.0, dtype=torch.float32, device=DEV)
    q.qwha_bwd_plan(z, dy, plan, a["c"], 1.0, dc=dc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dc).item() == 0
