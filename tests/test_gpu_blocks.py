"""Parity at input widths that are not powers of two: the block-diagonal
transform (m Sylvester blocks of order b, b the largest power of two dividing
d_in, H^-1 = H/b), through every entry point that takes such widths.

Bars as for power-of-two widths (tests/bars.py): indices, budgets and
permutations bit-exact; fp32 outputs within 1e-5 of the largest reference
entry; bf16 outputs element by element within 2^-8 |b| + 1e-5 max|b|; the
calibrated system 1e-12; refined values 1e-6; the quantized layer 4e-3.
"""

import numpy as np
import pytest

import oracle as O
import synth
from tests.test_gpu_parity import (_check_layer_full, _dev_adapter, _edge_dwq, _small_case,
                                   assert_init_equal, init_both, say, to_dev, to_np)
from tests.bars import assert_act_close, assert_f32_close
from tests.test_gpu_quant import host as qhost
from tests.test_gpu_quant import quant_layer
from tests.test_gpu_refine import check_init as check_calibrated
from tests.test_gpu_refine import check_refined, oracle_calibrated

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantization_aware_sparse_amd as qq
    return qq


WIDTHS = [(37, 192, 600), (64, 320, 2000), (17, 1536, 1500), (9, 14336, 4000),
          (50, 11008, 9000), (5, 6144, 700)]


@pytest.mark.parametrize("d_out,d_in,p", WIDTHS)
def test_init_select_block_widths(q, d_out, d_in, p):
    say("init block width", d_out, d_in, p)
    dwq = _edge_dwq(d_out, d_in, d_out + d_in)
    ref, got = init_both(q, dwq, p, 3)
    assert np.min(ref["budget_margin"]) > 1e-9
    assert_init_equal(ref, got)


# (800, 6144, 60000): 2400 blocks of 2048 columns, more than the row kernel's
# 2048 workgroups, so workgroups take several blocks of different rows
@pytest.mark.parametrize("d_out,d_in,p", WIDTHS[:4] + [(800, 6144, 60000)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_materialize_block_widths(q, d_out, d_in, p, out):
    say("materialize block width", d_out, d_in, p, out)
    r = O.init_select(_edge_dwq(d_out, d_in, 3 * d_in), p, m=3)
    a = _dev_adapter(r)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    dW = q.qwha_materialize(a["row_ptr"], a["E"], a["c"], d_out, d_in, 0.75, out_dtype=dt)
    torch.cuda.synchronize()
    ref = O.materialize(r["E"], r["c"], d_out, d_in, 0.75)
    assert_act_close(to_np(dW), ref, out, "dW")


@pytest.mark.parametrize("d_out,d_in,p,T", [(37, 192, 600, 77), (130, 320, 2000, 257),
                                            (17, 1536, 1500, 64), (9, 14336, 4000, 33)])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fwd_bwd_block_widths(q, d_out, d_in, p, T, act):
    say("fwd/bwd block width", d_out, d_in, p, T, act)
    r, x, dy = _small_case(d_out, d_in, p, T, act, d_out + T)
    a = _dev_adapter(r)
    xt, dyt = to_dev(x), to_dev(dy)
    y = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25)
    dx, dc = q.qwha_bwd(xt, dyt, a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["csc_perm"], 1.25)
    torch.cuda.synchronize()
    x64, dy64 = synth.act_to_f64(x), synth.act_to_f64(dy)
    dW = O.materialize(r["E"], r["c"], d_out, d_in, 1.25)
    dx_ref, dc_ref = O.backward(x64, dy64, r["E"], r["c"], d_out, d_in, 1.25, dW=dW)
    assert_act_close(to_np(y), O.forward(x64, dW), act, "y")
    assert_act_close(to_np(dx), dx_ref, act, "dx")
    assert_f32_close(to_np(dc), dc_ref, "dc")


@pytest.mark.parametrize("strategy", ["magnitude", "random"])
@pytest.mark.parametrize("d_out,d_in,p", [(37, 192, 600), (17, 1536, 1500), (9, 14336, 4000)])
def test_global_selection_block_widths(q, strategy, d_out, d_in, p):
    say("global block width", strategy, d_out, d_in, p)
    dwq = _edge_dwq(d_out, d_in, 7 * d_in)
    ref = O.init_select_global(dwq, p, strategy, 5)
    got = q.qwha_init_select_global(to_dev(dwq), p, strategy, 5)
    torch.cuda.synchronize()
    assert_init_equal(ref, got)


@pytest.mark.parametrize("d_out,d_in,p,N", [(37, 192, 600, 400), (20, 320, 900, 700),
                                            (9, 1536, 900, 2000)])
def test_calibrated_refine_block_widths(q, d_out, d_in, p, N):
    say("calibrated block width", d_out, d_in, p, N)
    dwq = (0.01 * np.random.default_rng(d_in).standard_normal((d_out, d_in))).astype(np.float32)
    X = synth.make_calibration(d_in, N, seed=d_in, act="f32")
    ref = oracle_calibrated(dwq, X, p, 3, damp=0.001)
    assert np.min(ref["margin"]) > 1e-9
    Hs = q.qwha_hessian(to_dev(X))
    got = q.qwha_init_select_calibrated(to_dev(dwq), Hs, p, 3, damp=0.001)
    torch.cuda.synchronize()
    check_calibrated(ref, got)
    c, status = q.qwha_refine_values(got["row_ptr"], got["E"], got["G"], got["rhs"],
                                     got["c"].clone())
    torch.cuda.synchronize()
    assert qhost(status).tolist() == [int(np.sum(~ref["ok"])), 0]
    check_refined(ref, qhost(c))


@pytest.mark.parametrize("T,d_out,d_in,bits,group,p", [(77, 37, 192, 4, 64, 600),
                                                       (130, 64, 14336, 4, 128, 4000)])
def test_quantized_layer_block_widths(q, T, d_out, d_in, bits, group, p):
    say("quantized layer block width", T, d_out, d_in, bits, group, p)
    L = quant_layer(d_out, d_in, bits, group, p, seed=d_in)
    rp, E, c = to_dev(L["r"]["row_ptr"]), to_dev(L["r"]["E"]), to_dev(L["r"]["c"])
    W = q.qwha_merge(to_dev(L["words"]), to_dev(L["s"]), to_dev(L["z"]), bits, group, rp, E, c,
                     d_in, 0.8)
    x = synth.f32_to_bf16_bits(np.random.default_rng(T).standard_normal((T, d_in)).astype(np.float32))
    y = q.qwha_layer_fwd(to_dev(x), to_dev(L["words"]), to_dev(L["s"]), to_dev(L["z"]), bits,
                         group, rp, E, c, 1.0)
    torch.cuda.synchronize()
    assert O.rel_err(qhost(W), O.merge_weights(L["W_Q"], L["r"]["E"], L["r"]["c"], 0.8)) <= 1e-6
    ref = O.layer_forward(synth.act_to_f64(x), L["W_Q"], L["r"]["E"], L["r"]["c"], 1.0)
    assert O.rel_err(qhost(y), ref) <= 4e-3


def test_full_down_proj_layer(q):
    # the down_proj shape of the same models: 4096 x 14336 (7 blocks of 2048),
    # budget P(r=64), 8192 bf16 tokens; init bit-exact, sampled fwd / bwd
    spec = synth.config_specs("down")[0]
    layer = synth.make_layer(spec, seed=0)
    x, dy = synth.make_activations(spec, seed=0)
    say("full down_proj layer")
    _check_layer_full(q, spec, layer, x, dy)
