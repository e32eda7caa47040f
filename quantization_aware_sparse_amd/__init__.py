"""Walsh-Hadamard adapter (WHA) of QWHA on MI355X: Python binding.

Thin wrappers over the C-ABI in include/qwha.h (same names). They only
marshal arguments: device memory comes from torch tensors, the stream is
torch's current HIP stream, and every step runs in the library's HIP
kernels. There is no CPU path.

The adapter: dW = alpha * F H^-1, F = Scatter(c, E), H the Sylvester
Walsh-Hadamard matrix along d_in (QWHA notes, papernotes.org, 方法详解 ›
整体框架; gist.science summary §2.1).
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from ._lib import QwhaError, check, lib  # noqa: F401

__all__ = [
    "QWHA_F32", "QWHA_BF16", "QwhaError", "lib",
    "QWHA_SELECT_MAGNITUDE", "QWHA_SELECT_RANDOM",
    "qwha_init_select", "qwha_init_select_global", "qwha_hessian",
    "qwha_init_select_calibrated", "qwha_refine_values", "qwha_merge", "qwha_layer_fwd",
    "qwha_materialize", "qwha_fwd", "qwha_fwd_noalloc", "qwha_fwd_z", "qwha_bwd",
    "qwha_bwd_dz", "qwha_plan_build", "qwha_fwd_plan", "qwha_bwd_plan",
    "qwha_sign_update", "qwha_fwht", "workspace", "WHAFunction",
]

QWHA_F32 = 0
QWHA_BF16 = 1
QWHA_SELECT_MAGNITUDE = 1
QWHA_SELECT_RANDOM = 2
_STRATEGY = {"magnitude": QWHA_SELECT_MAGNITUDE, "random": QWHA_SELECT_RANDOM}

_DT = {torch.float32: QWHA_F32, torch.bfloat16: QWHA_BF16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace(nbytes: int, device) -> torch.Tensor:
    """Caller-owned workspace buffer (the library never allocates)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- init
def qwha_init_select(dWq: torch.Tensor, p: int, min_per_row: int = 3,
                     temperature: float = 1.0,
                     ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    d_out, d_in = dWq.shape
    dev = dWq.device
    row_ptr = torch.empty(d_out + 1, dtype=torch.int32, device=dev)
    E = torch.empty((max(p, 1), 2), dtype=torch.int32, device=dev)[:p]
    c = torch.empty(max(p, 1), dtype=torch.float32, device=dev)[:p]
    col_ptr = torch.empty(d_in + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(p, 1), dtype=torch.int32, device=dev)[:p]
    need = lib.qwha_init_workspace_bytes(d_out, d_in)
    if ws is None:
        ws = workspace(need, dev)
    check(lib.qwha_init_select(_ptr(dWq), d_out, d_in, p, min_per_row, float(temperature),
                               _ptr(row_ptr), E.data_ptr(), c.data_ptr(), _ptr(col_ptr),
                               perm.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
          "qwha_init_select")
    return dict(row_ptr=row_ptr, E=E, c=c, col_ptr=col_ptr, csc_perm=perm)


def qwha_init_select_global(dWq: torch.Tensor, p: int, strategy: str = "magnitude",
                            seed: int = 0,
                            ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Global top-p selection by |C| ("magnitude") or uniformly at random
    ("random", SplitMix64 draws seeded with `seed`); outputs as
    qwha_init_select."""
    if strategy not in _STRATEGY:
        raise ValueError(f"strategy must be one of {sorted(_STRATEGY)}")
    st = _STRATEGY[strategy]
    d_out, d_in = dWq.shape
    dev = dWq.device
    row_ptr = torch.empty(d_out + 1, dtype=torch.int32, device=dev)
    E = torch.empty((max(p, 1), 2), dtype=torch.int32, device=dev)[:p]
    c = torch.empty(max(p, 1), dtype=torch.float32, device=dev)[:p]
    col_ptr = torch.empty(d_in + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(p, 1), dtype=torch.int32, device=dev)[:p]
    need = lib.qwha_init_global_workspace_bytes(d_out, d_in, st)
    if ws is None:
        ws = workspace(need, dev)
    check(lib.qwha_init_select_global(_ptr(dWq), d_out, d_in, p, st,
                                      int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(row_ptr),
                                      E.data_ptr(), c.data_ptr(), _ptr(col_ptr),
                                      perm.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
          "qwha_init_select_global")
    return dict(row_ptr=row_ptr, E=E, c=c, col_ptr=col_ptr, csc_perm=perm)


# ---------------------------------------------------------------- calibration
def qwha_hessian(X: torch.Tensor, Hs: Optional[torch.Tensor] = None,
                 accumulate: bool = False) -> torch.Tensor:
    """Hs (+)= X^T X in fp64 for calibration tokens X [N][d_in] (fp32/bf16)."""
    N, d_in = X.shape
    if Hs is None:
        Hs = torch.empty((d_in, d_in), dtype=torch.float64, device=X.device)
        accumulate = False
    check(lib.qwha_hessian(_ptr(X) if N else None, _dt(X), N, d_in, _ptr(Hs), int(accumulate),
                           _stream()), "qwha_hessian")
    return Hs


def qwha_init_select_calibrated(dWq: torch.Tensor, Hs: torch.Tensor, p: int,
                                min_per_row: int = 3, temperature: float = 1.0,
                                damp: float = 0.0,
                                ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """The init with a calibration Hessian: positions and dense-solution
    values as qwha_init_select (allocation by activation error norms), plus
    the refinement system G [d_in][d_in] and rhs [p] (fp64)."""
    d_out, d_in = dWq.shape
    dev = dWq.device
    row_ptr = torch.empty(d_out + 1, dtype=torch.int32, device=dev)
    E = torch.empty((max(p, 1), 2), dtype=torch.int32, device=dev)[:p]
    c = torch.empty(max(p, 1), dtype=torch.float32, device=dev)[:p]
    col_ptr = torch.empty(d_in + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(p, 1), dtype=torch.int32, device=dev)[:p]
    G = torch.empty((d_in, d_in), dtype=torch.float64, device=dev)
    rhs = torch.empty(max(p, 1), dtype=torch.float64, device=dev)[:p]
    need = lib.qwha_init_calibrated_workspace_bytes(d_out, d_in)
    if ws is None:
        ws = workspace(need, dev)
    check(lib.qwha_init_select_calibrated(_ptr(dWq), d_out, d_in, _ptr(Hs), float(damp), p,
                                          min_per_row, float(temperature), _ptr(row_ptr),
                                          E.data_ptr(), c.data_ptr(), _ptr(col_ptr),
                                          perm.data_ptr(), _ptr(G), rhs.data_ptr(),
                                          ws.data_ptr(), ws.numel(), _stream()),
          "qwha_init_select_calibrated")
    return dict(row_ptr=row_ptr, E=E, c=c, col_ptr=col_ptr, csc_perm=perm, G=G, rhs=rhs)


def refine_workspace_bytes(row_ptr: torch.Tensor) -> int:
    host = row_ptr.detach().to("cpu", torch.int32).contiguous()
    return lib.qwha_refine_workspace_bytes(host.data_ptr(), host.numel() - 1)


def qwha_refine_values(row_ptr, E, G, rhs, c: torch.Tensor,
                       ws: Optional[torch.Tensor] = None):
    """Refined values in place of c (rows whose system is not definite, or
    does not fit ws, keep theirs). Returns (c, status[2]) with status =
    (rows not positive definite, rows skipped for workspace)."""
    d_out = row_ptr.numel() - 1
    d_in = G.shape[0]
    p = c.numel()
    status = torch.empty(2, dtype=torch.int32, device=c.device)
    if ws is None:
        ws = workspace(refine_workspace_bytes(row_ptr), c.device)
    check(lib.qwha_refine_values(_ptr(row_ptr), E.data_ptr(), _ptr(G), rhs.data_ptr(), d_out,
                                 d_in, p, c.data_ptr(), _ptr(status), ws.data_ptr(), ws.numel(),
                                 _stream()), "qwha_refine_values")
    return c, status


# ---------------------------------------------------------------- quantized base
def qwha_merge(codes, scales, zeros, bits: int, group: int, row_ptr, E, c, d_in: int,
               alpha: float = 1.0, out_dtype=torch.float32) -> torch.Tensor:
    """W = W_Q + alpha F H^-1 from packed codes (uint32 words as int32)."""
    d_out = row_ptr.numel() - 1
    W = torch.empty((d_out, d_in), dtype=out_dtype, device=codes.device)
    p = c.numel()
    check(lib.qwha_merge(_ptr(codes), _ptr(scales), _ptr(zeros), bits, group, d_out, d_in, p,
                         _ptr(row_ptr), E.data_ptr(), c.data_ptr(), float(alpha),
                         _DT[out_dtype], _ptr(W), _stream()), "qwha_merge")
    return W


def qwha_layer_fwd(x: torch.Tensor, codes, scales, zeros, bits: int, group: int, row_ptr, E,
                   c, alpha: float = 1.0, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W_Q^T + alpha z F^T for bf16 x [T][d_in]; y bf16 [T][d_out]."""
    T, d_in = x.shape
    d_out = row_ptr.numel() - 1
    p = c.numel()
    y = torch.empty((T, d_out), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = workspace(lib.qwha_layer_fwd_workspace_bytes(T, d_in, d_out, p), x.device)
    check(lib.qwha_layer_fwd(_ptr(x) if T else None, _dt(x), T, d_in, d_out, _ptr(codes),
                             _ptr(scales), _ptr(zeros), bits, group, p, _ptr(row_ptr),
                             E.data_ptr(), c.data_ptr(), float(alpha),
                             _ptr(y) if T else None, ws.data_ptr(), ws.numel(), _stream()),
          "qwha_layer_fwd")
    return y


# ---------------------------------------------------------------- materialize
def qwha_materialize(row_ptr, E, c, d_out: int, d_in: int, alpha: float = 1.0,
                     out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                     accumulate: bool = False) -> torch.Tensor:
    if out is None:
        out = torch.empty((d_out, d_in), dtype=out_dtype, device=c.device)
    p = int(c.numel())
    check(lib.qwha_materialize(_ptr(row_ptr), E.data_ptr(), c.data_ptr(), d_out, d_in, p,
                               float(alpha), _dt(out), _ptr(out), int(accumulate), _stream()),
          "qwha_materialize")
    return out


# ---------------------------------------------------------------- forward
def qwha_fwd(x: torch.Tensor, d_out: int, row_ptr, E, c, alpha: float = 1.0,
             y: Optional[torch.Tensor] = None, accumulate: bool = False,
             ws: Optional[torch.Tensor] = None,
             z_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = alpha z F^T; with z_out (fp32 [T][d_in]) z = FWHT(x)/n is kept
    there for qwha_bwd(..., z=z_out)."""
    T, d_in = x.shape
    p = int(c.numel())
    if y is None:
        y = torch.empty((T, d_out), dtype=x.dtype, device=x.device)
    need = lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p)
    if ws is None:
        ws = workspace(need, x.device)
    if z_out is not None:
        check(lib.qwha_fwd_save(_ptr(x), _dt(x), T, d_in, d_out, p, _ptr(row_ptr),
                                E.data_ptr(), c.data_ptr(), float(alpha), _ptr(y),
                                int(accumulate), _ptr(z_out), ws.data_ptr(), ws.numel(),
                                _stream()), "qwha_fwd_save")
        return y
    check(lib.qwha_fwd(_ptr(x), _dt(x), T, d_in, d_out, p, _ptr(row_ptr), E.data_ptr(),
                       c.data_ptr(), float(alpha), _ptr(y), int(accumulate), ws.data_ptr(),
                       ws.numel(), _stream()), "qwha_fwd")
    return y


def qwha_fwd_noalloc(x: torch.Tensor, d_out: int, row_ptr, E, c, alpha: float = 1.0,
                     y: Optional[torch.Tensor] = None,
                     accumulate: bool = False) -> torch.Tensor:
    """qwha_fwd with the library's static device scratch as its workspace
    (the call allocates nothing on the device; y is allocated here only when
    not given)."""
    T, d_in = x.shape
    p = int(c.numel())
    if y is None:
        y = torch.empty((T, d_out), dtype=x.dtype, device=x.device)
    check(lib.qwha_fwd_noalloc(_ptr(x), _dt(x), T, d_in, d_out, p, _ptr(row_ptr), E.data_ptr(),
                               c.data_ptr(), float(alpha), _ptr(y), int(accumulate), _stream()),
          "qwha_fwd_noalloc")
    return y


# ---------------------------------------------------------------- backward
def qwha_bwd(x: Optional[torch.Tensor], dy: torch.Tensor, row_ptr, E, c, col_ptr, csc_perm,
             alpha: float = 1.0, need_dx: bool = True, need_dc: bool = True,
             dx: Optional[torch.Tensor] = None, accumulate_dx: bool = False,
             dc: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
             z: Optional[torch.Tensor] = None):
    """dx and dc; with z (the forward's z_out) x is not needed (may be None)."""
    T, d_in = (z if z is not None else x).shape
    d_out = dy.shape[1]
    p = int(c.numel())
    if need_dx and dx is None:
        dx = torch.empty((T, d_in), dtype=dy.dtype, device=dy.device)
    if need_dc and dc is None:
        dc = torch.empty(max(p, 1), dtype=torch.float32, device=dy.device)[:p]
    if not need_dx:
        dx = None
    if not need_dc:
        dc = None
    need = lib.qwha_bwd_workspace_bytes(T, d_in, d_out, p)
    if ws is None:
        ws = workspace(need, dy.device)
    if z is not None:
        check(lib.qwha_bwd_saved(_ptr(z), _ptr(dy), _dt(dy), T, d_in, d_out, p, _ptr(row_ptr),
                                 E.data_ptr(), c.data_ptr(), _ptr(col_ptr), csc_perm.data_ptr(),
                                 float(alpha), _ptr(dx), int(accumulate_dx),
                                 dc.data_ptr() if dc is not None else None,
                                 ws.data_ptr(), ws.numel(), _stream()), "qwha_bwd_saved")
        return dx, dc
    check(lib.qwha_bwd(_ptr(x), _ptr(dy), _dt(dy), T, d_in, d_out, p, _ptr(row_ptr),
                       E.data_ptr(), c.data_ptr(), _ptr(col_ptr), csc_perm.data_ptr(),
                       float(alpha), _ptr(dx), int(accumulate_dx),
                       dc.data_ptr() if dc is not None else None,
                       ws.data_ptr(), ws.numel(), _stream()), "qwha_bwd")
    return dx, dc


def qwha_fwd_z(z: torch.Tensor, d_out: int, row_ptr, E, c, alpha: float = 1.0,
               act=torch.bfloat16, y: Optional[torch.Tensor] = None, accumulate: bool = False,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y (+)= alpha z F^T from a kept z = FWHT(x)/n (fp32 [T][d_in]), y in `act`."""
    T, d_in = z.shape
    p = int(c.numel())
    if y is None:
        y = torch.empty((T, d_out), dtype=act, device=z.device)
    if ws is None:
        ws = workspace(lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p), z.device)
    check(lib.qwha_fwd_z(_ptr(z), _dt(y), T, d_in, d_out, p, _ptr(row_ptr), E.data_ptr(),
                         c.data_ptr(), float(alpha), _ptr(y), int(accumulate), ws.data_ptr(),
                         ws.numel(), _stream()), "qwha_fwd_z")
    return y


def qwha_bwd_dz(z: Optional[torch.Tensor], dy: torch.Tensor, E, c, col_ptr, csc_perm,
                alpha: float = 1.0, dz: Optional[torch.Tensor] = None,
                accumulate_dz: bool = False, need_dc: bool = True,
                dc: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                d_in: Optional[int] = None):
    """dz (+)= alpha dy F (fp32 [T][d_in]) and dc from the kept z; no transform
    (dx = FWHT(dz)/n is a qwha_fwht call)."""
    T, d_out = dy.shape
    if d_in is None:
        d_in = (z if z is not None else dz).shape[1]
    p = int(c.numel())
    if dz is None:
        dz = torch.empty((T, d_in), dtype=torch.float32, device=dy.device)
    if need_dc and dc is None:
        dc = torch.empty(max(p, 1), dtype=torch.float32, device=dy.device)[:p]
    if not need_dc:
        dc = None
    if ws is None:
        ws = workspace(lib.qwha_bwd_workspace_bytes(T, d_in, d_out, p), dy.device)
    check(lib.qwha_bwd_dz(_ptr(z), _ptr(dy), _dt(dy), T, d_in, d_out, p, E.data_ptr(),
                          c.data_ptr(), _ptr(col_ptr), csc_perm.data_ptr(), float(alpha),
                          _ptr(dz), int(accumulate_dz),
                          dc.data_ptr() if dc is not None else None, ws.data_ptr(), ws.numel(),
                          _stream()), "qwha_bwd_dz")
    return dz, dc


# ---------------------------------------------------------------- plans
def qwha_plan_build(row_ptr, E, col_ptr, csc_perm, d_in: int, d_out: int,
                    act=torch.bfloat16, plan: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Both SpMM streams of the adapter, built once from its frozen E (int32
    [p][2]) with the init's row_ptr, col_ptr and csc_perm, for activations
    of dtype `act` (the planned calls must use the same); returns the plan."""
    p = int(E.shape[0])
    need = lib.qwha_plan_bytes(d_in, d_out, p)
    if plan is None:
        plan = workspace(need, E.device)
    code = 1 if act == torch.bfloat16 else 0
    check(lib.qwha_plan_build(_ptr(row_ptr), E.data_ptr(), _ptr(col_ptr), csc_perm.data_ptr(),
                              d_in, d_out, p, code, plan.data_ptr(), plan.numel(), _stream()),
          "qwha_plan_build")
    return plan


def qwha_fwd_plan(x: Optional[torch.Tensor], plan: torch.Tensor, c, d_out: int,
                  alpha: float = 1.0, y: Optional[torch.Tensor] = None,
                  accumulate: bool = False, z_in: Optional[torch.Tensor] = None,
                  z_out: Optional[torch.Tensor] = None, act=None,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y (+)= alpha z F^T on a plan; z from x, or z_in (kept); z_out keeps it."""
    src = z_in if z_in is not None else x
    T, d_in = src.shape
    p = int(c.numel())
    adt = act if act is not None else (x.dtype if x is not None else torch.bfloat16)
    if y is None:
        y = torch.empty((T, d_out), dtype=adt, device=src.device)
    if ws is None:
        ws = workspace(lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p), src.device)
    check(lib.qwha_fwd_plan(_ptr(x), _ptr(z_in), _dt(y), T, d_in, d_out, p, plan.data_ptr(),
                            c.data_ptr(), float(alpha), _ptr(y), int(accumulate), _ptr(z_out),
                            ws.data_ptr(), ws.numel(), _stream()), "qwha_fwd_plan")
    return y


def qwha_bwd_plan(z: torch.Tensor, dy: torch.Tensor, plan: torch.Tensor, c,
                  alpha: float = 1.0, need_dx: bool = True, dx: Optional[torch.Tensor] = None,
                  accumulate_dx: bool = False, dz: Optional[torch.Tensor] = None,
                  accumulate_dz: bool = False, dc: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None):
    """dc and dx (or dz with no transform) from the kept z on a plan."""
    T, d_in = z.shape
    d_out = dy.shape[1]
    p = int(c.numel())
    if dz is not None:
        need_dx = False
    if need_dx and dx is None:
        dx = torch.empty((T, d_in), dtype=dy.dtype, device=dy.device)
    if not need_dx:
        dx = None
    if dc is None:
        dc = torch.empty(max(p, 1), dtype=torch.float32, device=dy.device)[:p]
    if ws is None:
        ws = workspace(lib.qwha_bwd_workspace_bytes(T, d_in, d_out, p), dy.device)
    check(lib.qwha_bwd_plan(_ptr(z), _ptr(dy), _dt(dy), T, d_in, d_out, p, plan.data_ptr(),
                            c.data_ptr(), float(alpha), _ptr(dx), int(accumulate_dx), _ptr(dz),
                            int(accumulate_dz), dc.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream()), "qwha_bwd_plan")
    return (dz if dz is not None else dx), dc


# ---------------------------------------------------------------- update, fwht
def qwha_sign_update(c: torch.Tensor, dc: torch.Tensor, step: float = 1e-3) -> torch.Tensor:
    check(lib.qwha_sign_update(c.data_ptr(), dc.data_ptr(), int(c.numel()), float(step),
                               _stream()), "qwha_sign_update")
    return c


def qwha_fwht(x: torch.Tensor, scale: float = 1.0, out_dtype=None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    rows = x.numel() // x.shape[-1]
    n = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    check(lib.qwha_fwht(_ptr(x), _dt(x), _ptr(out), _dt(out), rows, n, float(scale),
                        _stream()), "qwha_fwht")
    return out


# ---------------------------------------------------------------- autograd
class WHAFunction(torch.autograd.Function):
    """y = x dW^T for the adapter branch; gradients flow to x and c only
    (W_Q and H frozen: papernotes.org, 损失函数 / 训练策略). When c needs a
    gradient the forward keeps z = FWHT(x)/n (fp32) for the backward's dc,
    as a saved activation, instead of transforming x again."""

    @staticmethod
    def forward(ctx, x, c, row_ptr, E, col_ptr, csc_perm, d_out, alpha):
        x = x.contiguous()
        ctx.alpha = alpha
        ctx.saved_z = bool(ctx.needs_input_grad[1])
        if ctx.saved_z:
            z = torch.empty(x.shape, dtype=torch.float32, device=x.device)
            y = qwha_fwd(x, d_out, row_ptr, E, c, alpha, z_out=z)
            ctx.save_for_backward(z, c, row_ptr, E, col_ptr, csc_perm)
            return y
        ctx.save_for_backward(x, c, row_ptr, E, col_ptr, csc_perm)
        return qwha_fwd(x, d_out, row_ptr, E, c, alpha)

    @staticmethod
    def backward(ctx, dy):
        saved, c, row_ptr, E, col_ptr, csc_perm = ctx.saved_tensors
        dy = dy.contiguous()
        if ctx.saved_z:
            dx, dc = qwha_bwd(None, dy, row_ptr, E, c, col_ptr, csc_perm, ctx.alpha,
                              need_dx=ctx.needs_input_grad[0], need_dc=True, z=saved)
            return dx, dc, None, None, None, None, None, None
        dx, _ = qwha_bwd(saved, dy, row_ptr, E, c, col_ptr, csc_perm, ctx.alpha,
                         need_dx=ctx.needs_input_grad[0], need_dc=False)
        return dx, None, None, None, None, None, None, None
