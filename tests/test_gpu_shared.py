"""Adapters that share their input (q, k, v of an attention block) through
one transform: qwha_fwd_z (forward from a kept z) and qwha_bwd_dz (dz and dc
without the transform, dz summed over adapters, then one qwha_fwht).

First the single-adapter identities (the same kernels on the same data, so
bit-equal to qwha_fwd_save / qwha_bwd_saved); then three adapters of
different widths and alphas on one x against the fp64 oracle, whose dx is
the sum of the three adapters' dx. Bars as in tests/bars.py.
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


def adapter(d_out, d_in, p, seed):
    rng = np.random.default_rng(seed)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    r = O.init_select(dwq, p, m=3)
    return r, {k: dev(r[k]) for k in ("row_ptr", "E", "c", "col_ptr", "csc_perm")}


def acts(T, d, act, seed):
    a = np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32)
    return synth.f32_to_bf16_bits(a) if act == "bf16" else a


@pytest.mark.parametrize("d_out,d_in,p,T,act", [(300, 256, 2500, 77, "f32"),
                                                 (513, 1024, 9000, 300, "bf16"),
                                                 (64, 192, 700, 33, "bf16")])
def test_single_adapter_identities(q, d_out, d_in, p, T, act):
    print("shared identities", d_out, d_in, p, T, act, flush=True)
    r, a = adapter(d_out, d_in, p, d_out + T)
    x, dy = dev(acts(T, d_in, act, 1)), dev(acts(T, d_out, act, 2))
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    y0 = q.qwha_fwd(x, d_out, a["row_ptr"], a["E"], a["c"], 1.0, z_out=z)
    y1 = q.qwha_fwd_z(z, d_out, a["row_ptr"], a["E"], a["c"], 1.0, act=x.dtype)
    dx0, dc0 = q.qwha_bwd(None, dy, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"],
                          1.0, z=z)
    dz, dc1 = q.qwha_bwd_dz(z, dy, a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.0)
    b = O.block_size(d_in)
    dx1 = q.qwha_fwht(dz.view(T * (d_in // b), b), 1.0 / b, out_dtype=x.dtype).view(T, d_in)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(dc0, dc1)
    assert torch.equal(dx0, dx1)
    # dz alone (no dc requested) is the same sum through the plain product
    dz2, none = q.qwha_bwd_dz(z, dy, a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.0,
                              need_dc=False)
    torch.cuda.synchronize()
    assert none is None
    dW = O.materialize(r["E"], r["c"], d_out, d_in, 1.0)
    F = O.scatter_dense(r["E"], r["c"], d_out, d_in)
    dz_ref = synth.act_to_f64(host_bits(dy, act)) @ F
    assert_f32_close(host(dz), dz_ref, "dz with dc")
    assert_f32_close(host(dz2), dz_ref, "dz without dc")
    assert_act_close(host(y1), O.forward(synth.act_to_f64(host_bits(x, act)), dW), act, "y")


def host_bits(t, act):
    """The activation as the test created it (bf16 bits or fp32)."""
    if act == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("d_in,act", [(256, "f32"), (1024, "bf16"), (320, "bf16")])
def test_three_adapters_share_one_transform(q, d_in, act):
    T = 129
    shapes = [(300, 2400, 1.25), (77, 900, 0.5), (77, 700, 2.0)]   # q, k, v
    print("shared qkv", d_in, act, flush=True)
    xa = acts(T, d_in, act, 7)
    x = dev(xa)
    x64 = synth.act_to_f64(xa)
    b = O.block_size(d_in)
    z = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    dz = torch.empty((T, d_in), dtype=torch.float32, device=DEV)
    dx_ref = np.zeros((T, d_in))
    outs = []
    for n, (d_out, p, alpha) in enumerate(shapes):
        r, a = adapter(d_out, d_in, p, 100 + n)
        dya = acts(T, d_out, act, 200 + n)
        dy = dev(dya)
        if n == 0:
            y = q.qwha_fwd(x, d_out, a["row_ptr"], a["E"], a["c"], alpha, z_out=z)
        else:
            y = q.qwha_fwd_z(z, d_out, a["row_ptr"], a["E"], a["c"], alpha, act=x.dtype)
        _, dc = q.qwha_bwd_dz(z, dy, a["E"], a["c"], a["col_ptr"], a["csc_perm"], alpha, dz=dz,
                              accumulate_dz=n > 0)
        dW = O.materialize(r["E"], r["c"], d_out, d_in, alpha)
        dy64 = synth.act_to_f64(dya)
        dxn, dcn = O.backward(x64, dy64, r["E"], r["c"], d_out, d_in, alpha, dW=dW)
        dx_ref += dxn
        outs.append((y, dc, O.forward(x64, dW), dcn))
    dx = q.qwha_fwht(dz.view(T * (d_in // b), b), 1.0 / b, out_dtype=x.dtype).view(T, d_in)
    torch.cuda.synchronize()
    for n, (y, dc, y_ref, dc_ref) in enumerate(outs):
        assert_act_close(host(y), y_ref, act, f"y[{n}]")
        assert_f32_close(host(dc), dc_ref, f"dc[{n}]")
    assert_act_close(host(dx), dx_ref, act, "summed dx")
