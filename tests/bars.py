"""Parity bars shared by the GPU tests (HIP path against the fp64 oracle).

* Indices, budgets and permutations: bit-exact (asserted where used).
* fp32 outputs computed in fp32 (dW, c, dc, and y / dx with fp32
  activations): normwise, max|a - b| <= 1e-5 max|b|. A sum of fp32 products
  has an absolute error of order eps * sum|terms|, not one relative to each
  entry, so the bound is taken against the largest entry.
* bf16 outputs (y / dx with bf16 activations): element by element,
  |a - b| <= 2^-8 |b| + 1e-5 max|b|. The kernels sum in fp32 (the second
  term, as above) and round once to bf16, which is off by at most 2^-9 of
  the value (the first term, with a factor 2 of slack). A normwise 2e-2,
  the coarsest bar the method's statement allows for bf16, would let an
  error in every small entry through.
"""

import numpy as np

F32_BAR = 1e-5
BF16_REL = 2.0 ** -8


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def assert_f32_close(got, ref, what="", bar=F32_BAR):
    got, ref = _f64(got), _f64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= bar * scale or (scale == 0.0 and err == 0.0), \
        f"{what}: normwise error {err / max(scale, 1e-300):.3e} > {bar:g}"


def assert_act_close(got, ref, act, what=""):
    """y or dx in the activation dtype `act` ('f32' or 'bf16')."""
    if act == "f32":
        assert_f32_close(got, ref, what)
        return
    got, ref = _f64(got), _f64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    lim = BF16_REL * np.abs(ref) + F32_BAR * scale
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:3].tolist()
        worst = float(np.max(err / np.maximum(lim, 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())} entries outside "
                             f"2^-8|b| + 1e-5 max|b| (first {idx}; worst at "
                             f"{worst:.2f}x the bound)")
