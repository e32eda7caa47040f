"""Parity of the quantized base layer with its adapter (HIP path, through the
C-ABI) with the fp64 CPU oracle.

Bars: merged weights within 1e-6 normwise in fp32; bf16 outputs (merged
weights or the layer output y) within 4e-3 normwise: each is one
round-to-nearest of an fp32 value (relative error at most 2^-9 per element)
whose own error is that of fp32 sums, and the base product's weight operand
q - z is exact in bf16.
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
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32).copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def quant_layer(d_out, d_in, bits, group, p, seed):
    """Base weights from the fixture's quantizer (RTN of fp32 N(0, 0.02^2)
    weights), their packed codes, and an adapter initialised on the error."""
    rng = np.random.default_rng(seed)
    w0 = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    qc, s, z = synth.rtn_codes(w0, bits, group)
    words = synth.pack_codes(qc, bits)
    W_Q = synth.rtn_quantize(w0, bits, group)
    r = O.init_select(w0 - W_Q, p, m=min(3, p // d_out))
    return dict(words=words, s=s, z=z, W_Q=W_Q, r=r)


def dev_adapter(r):
    return to_dev(r["row_ptr"]), to_dev(r["E"]), to_dev(r["c"])


@pytest.mark.parametrize("d_out,d_in,bits,group,p", [
    (37, 2, 4, 2, 40), (5, 16, 2, 16, 30), (64, 64, 3, 32, 300), (300, 128, 4, 64, 2500),
    (17, 1024, 8, 128, 2000), (9, 4096, 3, 128, 900), (40, 256, 4, 128, 0)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_merge(q, d_out, d_in, bits, group, p, out):
    say("merge", d_out, d_in, bits, group, p, out)
    L = quant_layer(d_out, d_in, bits, group, p, seed=d_out + d_in + bits)
    # the oracle dequantizes from the packed words itself
    W_Q = O.dequantize(O.unpack_codes(L["words"], d_in, bits), L["s"], L["z"], group)
    assert np.array_equal(W_Q, L["W_Q"])
    ref = O.merge_weights(W_Q, L["r"]["E"], L["r"]["c"], 0.8)
    rp, E, c = dev_adapter(L["r"])
    W = q.qwha_merge(to_dev(L["words"]), to_dev(L["s"]), to_dev(L["z"]), bits, group, rp, E, c,
                     d_in, 0.8, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    bound = 1e-6 if out == "f32" else 4e-3
    assert O.rel_err(host(W), ref) <= bound


@pytest.mark.parametrize("T,d_out,d_in,bits,group,p", [
    (1, 37, 64, 4, 32, 40), (5, 200, 64, 2, 64, 700), (130, 129, 256, 3, 128, 1500),
    (300, 256, 1024, 4, 128, 4000), (77, 64, 4096, 8, 128, 3000), (200, 96, 512, 4, 64, 0),
    (129, 300, 128, 4, 32, 300 * 128), (257, 130, 320, 4, 64, 2000),
    (64, 128, 2048, 4, 256, 5000), (3, 1, 128, 4, 32, 1), (150, 200, 4096, 4, 32, 9000)])
def test_layer_forward(q, T, d_out, d_in, bits, group, p):
    say("layer fwd", T, d_out, d_in, bits, group, p)
    L = quant_layer(d_out, d_in, bits, group, p, seed=T + d_out + d_in)
    x = synth.f32_to_bf16_bits(np.random.default_rng(T).standard_normal((T, d_in)).astype(np.float32))
    ref = O.layer_forward(synth.act_to_f64(x), L["W_Q"], L["r"]["E"], L["r"]["c"], 1.0)
    rp, E, c = dev_adapter(L["r"])
    y = q.qwha_layer_fwd(to_dev(x), to_dev(L["words"]), to_dev(L["s"]), to_dev(L["z"]), bits,
                         group, rp, E, c, 1.0)
    torch.cuda.synchronize()
    assert O.rel_err(host(y), ref) <= 4e-3


def test_layer_forward_zero_tokens_and_alpha(q):
    L = quant_layer(64, 256, 4, 64, 500, seed=1)
    rp, E, c = dev_adapter(L["r"])
    args = (to_dev(L["words"]), to_dev(L["s"]), to_dev(L["z"]), 4, 64, rp, E, c)
    y = q.qwha_layer_fwd(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), *args)
    assert y.shape == (0, 64)
    x = synth.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((50, 256)).astype(np.float32))
    for alpha in (0.0, -1.5):
        ref = O.layer_forward(synth.act_to_f64(x), L["W_Q"], L["r"]["E"], L["r"]["c"], alpha)
        y = q.qwha_layer_fwd(to_dev(x), *args, alpha=alpha)
        torch.cuda.synchronize()
        assert O.rel_err(host(y), ref) <= 4e-3


def test_layer_forward_full_config(q):
    # the 4096 x 4096 layer: 4-bit g128 codes, its adapter, 8192 bf16 tokens;
    # sampled tokens against the oracle one by one
    spec = synth.config_specs("c2")[0]
    layer = synth.make_layer(spec, seed=0)
    qc, s, z = synth.rtn_codes(layer.w0, spec.bits, spec.group)
    words = synth.pack_codes(qc, spec.bits)
    r = O.init_select(layer.dwq, spec.p, m=3)
    x, _ = synth.make_activations(spec, seed=0)
    say("layer fwd full config")
    rp, E, c = dev_adapter(r)
    y = q.qwha_layer_fwd(to_dev(x), to_dev(words), to_dev(s), to_dev(z), spec.bits, spec.group,
                         rp, E, c, 1.0)
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(spec.T, size=64, replace=False)
    merged = O.merge_weights(layer.wq, r["E"], r["c"], 1.0)
    ref = synth.act_to_f64(x[rows]) @ merged.T
    assert O.rel_err(host(y[torch.from_numpy(rows).to(DEV)]), ref) <= 4e-3
