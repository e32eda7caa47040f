"""Seeded sweep of random shapes through the whole adapter path on the GPU.

Each case draws d_out, d_in (a power of two, or a block-diagonal width
m * b with b >= 64), p, T and the activation dtype from its own seed, then
checks init (E, row_ptr, col_ptr, csc_perm bit-exact, c), materialize,
forward, backward (dx, dc) and the sign update against the fp64 oracle, to
the same bars as the other parity tests. The point is the combinations the
hand-picked shapes do not reach: ragged token tiles with ragged row groups,
budgets near the floor or the cap, block widths with few tokens.
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


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_np(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


WIDTHS = [2, 4, 16, 64, 128, 256, 512, 1024, 2048,
          3 * 64, 5 * 64, 3 * 128, 7 * 128, 5 * 256, 3 * 512]


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    d_in = int(rng.choice(WIDTHS))
    d_out = int(rng.integers(1, 700))
    m = min(3, d_in)
    lo, hi = m * d_out, d_in * d_out
    # budgets: near the floor, near the cap, or in between
    kind = seed % 3
    if kind == 0:
        p = lo + int(rng.integers(0, max(1, d_out)))
    elif kind == 1:
        p = hi - int(rng.integers(0, max(1, d_out)))
    else:
        p = int(rng.integers(lo, hi + 1))
    p = int(min(max(p, lo), hi))
    T = int(rng.integers(1, 300))
    act = "f32" if rng.integers(0, 2) == 0 else "bf16"
    return d_out, d_in, p, T, act


@pytest.mark.parametrize("seed", list(range(48)))
def test_random_shapes_whole_path(q, seed):
    d_out, d_in, p, T, act = draw_case(seed)
    print("sweep", seed, d_out, d_in, p, T, act, flush=True)
    rng = np.random.default_rng(seed)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    m = min(3, d_in)
    ref = O.init_select(dwq, p, m=m)
    got = q.qwha_init_select(to_dev(dwq), p, m, 1.0)
    torch.cuda.synchronize()
    for key in ("row_ptr", "E", "col_ptr", "csc_perm"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    assert O.rel_err(got["c"].cpu().numpy(), ref["c"]) <= 1e-6

    alpha = 0.75
    dW = q.qwha_materialize(got["row_ptr"], got["E"], got["c"], d_out, d_in, alpha)
    dW_ref = O.materialize(ref["E"], ref["c"], d_out, d_in, alpha)
    assert_f32_close(to_np(dW), dW_ref, "dW")

    x = rng.standard_normal((T, d_in)).astype(np.float32)
    dy = rng.standard_normal((T, d_out)).astype(np.float32)
    if act == "bf16":
        x, dy = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(dy)
    xt, dyt = to_dev(x), to_dev(dy)
    y = q.qwha_fwd(xt, d_out, got["row_ptr"], got["E"], got["c"], alpha)
    dx, dc = q.qwha_bwd(xt, dyt, got["row_ptr"], got["E"], got["c"], got["col_ptr"],
                        got["csc_perm"], alpha)
    torch.cuda.synchronize()
    x64, dy64 = synth.act_to_f64(x), synth.act_to_f64(dy)
    assert_act_close(to_np(y), O.forward(x64, dW_ref), act, "y")
    dx_ref, dc_ref = O.backward(x64, dy64, ref["E"], ref["c"], d_out, d_in, alpha, dW=dW_ref)
    assert_act_close(to_np(dx), dx_ref, act, "dx")
    assert_f32_close(to_np(dc), dc_ref, "dc")

    # the update takes the sign of the GPU's own dc (a sign is a decision)
    c_gpu = got["c"].cpu().numpy()
    c_new = q.qwha_sign_update(got["c"].clone(), dc, 1e-3)
    torch.cuda.synchronize()
    c_ref = O.sign_update(c_gpu, dc.cpu().numpy(), 1e-3)
    assert np.array_equal(c_new.cpu().numpy(), c_ref)


@pytest.mark.parametrize("d_out,d_in,p", [
    (16384, 16, 16384 * 5 + 777),     # the most rows the register allocator holds
    (16385, 16, 16385 * 5 + 777),     # one more: the allocator that keeps rows in memory
    (20000, 8, 20000 * 7 - 3),        # near the cap of 8 per row
    (16384, 8, 16384 * 3 + 1)])       # near the floor of 3 per row
def test_allocator_row_counts(q, d_out, d_in, p):
    """Budgets and the whole index at the row counts where the allocator
    switches from rows in registers to rows in memory."""
    print("allocator", d_out, d_in, p, flush=True)
    rng = np.random.default_rng(d_out + p)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    dwq[rng.choice(d_out, size=d_out // 50, replace=False)] *= 4.0
    ref = O.init_select(dwq, p, m=3, with_diagnostics=True)
    assert np.min(ref["budget_margin"]) > 1e-9, "ambiguous budget at this seed"
    got = q.qwha_init_select(to_dev(dwq), p, 3, 1.0)
    torch.cuda.synchronize()
    for key in ("row_ptr", "E", "col_ptr", "csc_perm"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
