"""qwha_fwd_noalloc (the forward for callers that cannot allocate) against
qwha_fwd on the GPU, through the C-ABI: the same kernels with the workspace
in the library's static device scratch, so the outputs must be equal bit
for bit. Two calls in a row, the second on a smaller input, so that the
second runs on what the first left in the scratch; then a call that adds
into y, and the plain entry point once more to show nothing leaked back."""

import numpy as np
import pytest

import oracle as O
import synth
from tests.bars import assert_act_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def _case(d_out, d_in, p, T, act, seed):
    rng = np.random.default_rng(seed)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    r = O.init_select(dwq, p, m=min(3, d_in))
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    if act == "bf16":
        x = synth.f32_to_bf16_bits(x)
        xt = torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x).to(DEV)
    a = {k: torch.from_numpy(r[k]).to(DEV) for k in ("row_ptr", "E", "c")}
    return r, x, xt, a


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_noalloc_forward_matches_the_workspace_forward(act):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantization_aware_sparse_amd as q
    shapes = [(513, 1024, 9000, 700), (300, 64, 2500, 77)]     # second call smaller
    for d_out, d_in, p, T in shapes:
        print("noalloc", act, d_out, d_in, p, T, flush=True)
        r, x, xt, a = _case(d_out, d_in, p, T, act, d_out + T)
        need = q.lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p)
        assert 0 < need <= 64 << 20
        y_ws = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25)
        y_na = q.qwha_fwd_noalloc(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws)
        dW = O.materialize(r["E"], r["c"], d_out, d_in, 1.25)
        assert_act_close(_host(y_na), O.forward(synth.act_to_f64(x), dW), act, "y")
        # accumulate into a given y
        base = torch.randn((T, d_out), device=DEV).to(xt.dtype)
        y_acc = base.clone()
        q.qwha_fwd_noalloc(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25, y=y_acc,
                           accumulate=True)
        y_acc_ws = base.clone()
        q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25, y=y_acc_ws, accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(y_acc, y_acc_ws)
    # the workspace entry point still gives the same result after the
    # static-scratch calls
    y_again = q.qwha_fwd(xt, d_out, a["row_ptr"], a["E"], a["c"], 1.25)
    torch.cuda.synchronize()
    assert torch.equal(y_again, y_ws)


def test_noalloc_forward_rejects_what_the_scratch_cannot_hold():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantization_aware_sparse_amd as q
    # refused on the host before anything runs: the pointers are real but
    # small, and no kernel is launched
    xt = torch.zeros((16, 4096), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((16, 4096), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(8, dtype=torch.int32, device=DEV)
    c = torch.zeros(8, dtype=torch.float32, device=DEV)
    st = q.lib.qwha_fwd_noalloc(xt.data_ptr(), 1, 8192, 4096, 4096, 524288, idx.data_ptr(),
                                idx.data_ptr(), c.data_ptr(), 1.0, y.data_ptr(), 0, None)
    assert st == 6     # QWHA_ERR_WORKSPACE
    assert b"static scratch" in q.lib.qwha_last_error()
