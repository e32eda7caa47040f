"""The C-ABI library on the CPU: it loads, exports every entry point that
include/qwha.h declares, and its host-side validation rejects bad arguments
with the documented status before touching the GPU. No compute call is made
(nothing here passes validation)."""

import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qwha.h")
LIB = os.path.join(ROOT, "quantization_aware_sparse_amd", "libqwha.so")

OK, INVALID, SHAPE, BUDGET, DTYPE, ALIGN, WORKSPACE, HIP = range(8)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwha_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def q():
    if not os.path.exists(LIB):
        pytest.fail("libqwha.so is not built (run __graft_entry__.build())")
    from quantization_aware_sparse_amd import _lib
    return _lib.lib


def test_exports_every_header_symbol(q):
    names = header_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    from quantization_aware_sparse_amd import _lib
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(q):
    for s in range(8):
        assert q.qwha_status_string(s)
    assert q.qwha_status_string(OK) == b"ok"
    assert q.qwha_version() >= 100


def test_workspace_queries(q):
    a = q.qwha_fwd_workspace_bytes(8192, 4096, 4096, 524288)
    assert a >= 8192 * 4096 * 4 + 524288 * 8
    b = q.qwha_bwd_workspace_bytes(8192, 4096, 4096, 524288)
    assert b >= 2 * 8192 * 4096 * 4 + 524288 * 8
    assert q.qwha_init_workspace_bytes(4096, 4096) >= 4096 * 8
    assert q.qwha_fwd_workspace_bytes(-1, 4096, 4096, 1) == 0
    # magnitude keeps one 64-bit key per position; random draws them on the fly
    mag = q.qwha_init_global_workspace_bytes(4096, 4096, 1)
    rnd = q.qwha_init_global_workspace_bytes(4096, 4096, 2)
    assert mag >= 4096 * 4096 * 8 > rnd > 0
    assert q.qwha_init_global_workspace_bytes(4096, 4096, 3) == 0
    assert q.qwha_init_global_workspace_bytes(0, 4096, 1) == 0


FAKE = 0x10000          # aligned, never dereferenced (validation fails first)


def _fwd(q, **kw):
    a = dict(x=FAKE, act=1, T=16, d_in=256, d_out=256, p=2048, row_ptr=FAKE, E=FAKE, c=FAKE,
             alpha=1.0, y=FAKE, acc=0, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return q.qwha_fwd(a["x"], a["act"], a["T"], a["d_in"], a["d_out"], a["p"], a["row_ptr"],
                      a["E"], a["c"], a["alpha"], a["y"], a["acc"], a["ws"], a["wsb"],
                      a["stream"])


def test_fwd_validation(q):
    assert _fwd(q, d_in=12) == SHAPE
    assert _fwd(q, d_in=32768) == SHAPE
    assert _fwd(q, d_in=1) == SHAPE
    assert _fwd(q, d_out=0) == SHAPE
    assert _fwd(q, act=7) == DTYPE
    assert _fwd(q, p=256 * 256 + 1) == BUDGET
    assert _fwd(q, p=-1) == BUDGET
    assert _fwd(q, x=None) == INVALID
    assert _fwd(q, x=FAKE + 4) == ALIGN
    assert _fwd(q, E=FAKE + 2) == ALIGN
    assert _fwd(q, acc=2) == INVALID
    assert _fwd(q, alpha=float("inf")) == INVALID
    assert _fwd(q, ws=None) == WORKSPACE
    assert _fwd(q, wsb=10) == WORKSPACE
    assert b"workspace" in q.qwha_last_error()
    assert _fwd(q, T=-3) == SHAPE


def _fwd_noalloc(q, **kw):
    a = dict(x=FAKE, act=1, T=16, d_in=256, d_out=256, p=2048, row_ptr=FAKE, E=FAKE, c=FAKE,
             alpha=1.0, y=FAKE, acc=0, stream=None)
    a.update(kw)
    return q.qwha_fwd_noalloc(a["x"], a["act"], a["T"], a["d_in"], a["d_out"], a["p"],
                              a["row_ptr"], a["E"], a["c"], a["alpha"], a["y"], a["acc"],
                              a["stream"])


def test_fwd_noalloc_validation(q):
    # the same argument checks as qwha_fwd, all before any HIP call
    assert _fwd_noalloc(q, d_in=12) == SHAPE
    assert _fwd_noalloc(q, act=7) == DTYPE
    assert _fwd_noalloc(q, p=256 * 256 + 1) == BUDGET
    assert _fwd_noalloc(q, x=None) == INVALID
    assert _fwd_noalloc(q, y=FAKE + 4) == ALIGN
    assert _fwd_noalloc(q, T=0) == OK                       # nothing to do, nothing touched
    # a forward whose workspace exceeds the 64 MiB static scratch is refused
    # on the host, with the sizes in the message
    need = q.qwha_fwd_workspace_bytes(8192, 4096, 4096, 524288)
    assert need > 64 << 20
    assert _fwd_noalloc(q, T=8192, d_in=4096, d_out=4096, p=524288) == WORKSPACE
    msg = q.qwha_last_error()
    assert b"static scratch" in msg and str(need).encode() in msg
    assert q.qwha_fwd_workspace_bytes(3200, 4096, 4096, 524288) <= 64 << 20


def test_shared_transform_validation(q):
    # qwha_fwd_z: the forward from a kept z
    def fz(**kw):
        a = dict(z=FAKE, act=1, T=16, d_in=256, d_out=256, p=2048, row_ptr=FAKE, E=FAKE,
                 c=FAKE, alpha=1.0, y=FAKE, acc=0, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_fwd_z(a["z"], a["act"], a["T"], a["d_in"], a["d_out"], a["p"],
                            a["row_ptr"], a["E"], a["c"], a["alpha"], a["y"], a["acc"], a["ws"],
                            a["wsb"], None)
    assert fz(z=None) == INVALID
    assert fz(z=FAKE + 4) == ALIGN
    assert fz(d_in=12) == SHAPE
    assert fz() == WORKSPACE
    assert fz(T=0, z=None) == OK
    # only the prepared stream is needed: less than qwha_fwd's workspace
    need_fwd = q.qwha_fwd_workspace_bytes(16, 256, 256, 2048)
    assert fz(wsb=need_fwd - 16 * 256 * 4, ws=FAKE, y=FAKE + 8) == ALIGN  # passes the size check

    # qwha_bwd_dz: dz (+)= alpha dy F and dc, no transform
    def bd(**kw):
        a = dict(z=FAKE, dy=FAKE, act=1, T=16, d_in=256, d_out=256, p=2048, E=FAKE, c=FAKE,
                 col_ptr=FAKE, perm=FAKE, alpha=1.0, dz=FAKE, acc=0, dc=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_bwd_dz(a["z"], a["dy"], a["act"], a["T"], a["d_in"], a["d_out"], a["p"],
                             a["E"], a["c"], a["col_ptr"], a["perm"], a["alpha"], a["dz"],
                             a["acc"], a["dc"], a["ws"], a["wsb"], None)
    assert bd(dz=None) == INVALID
    assert bd(acc=2) == INVALID
    assert bd(dz=FAKE + 4) == ALIGN
    assert bd(z=None) == INVALID            # dc needs the kept z
    assert bd(z=None, dc=None) == WORKSPACE  # dz alone does not
    assert bd() == WORKSPACE
    assert bd(alpha=float("nan")) == INVALID


def test_plan_validation(q):
    # the plan holds both prepared streams: the forward's (padded pairs) and
    # the backward's, each with its index map, sized independently of T
    pb = q.qwha_plan_bytes(4096, 4096, 524288)
    assert pb >= 524288 * (8 + 4) * 2
    assert q.qwha_plan_bytes(0, 4096, 100) == 0
    assert q.qwha_plan_bytes(4096, 4096, -1) == 0
    assert q.qwha_plan_bytes(16384, 65536, 2**31) == 0

    def build(**kw):
        a = dict(row_ptr=FAKE, E=FAKE, col_ptr=FAKE, perm=FAKE, d_in=256, d_out=256, p=2048,
                 act=1, plan=FAKE, nb=0)
        a.update(kw)
        return q.qwha_plan_build(a["row_ptr"], a["E"], a["col_ptr"], a["perm"], a["d_in"],
                                 a["d_out"], a["p"], a["act"], a["plan"], a["nb"], None)
    assert build(d_in=12) == SHAPE
    assert build(act=5) == DTYPE
    assert build(p=256 * 256 + 1) == BUDGET
    assert build(E=None) == INVALID
    assert build() == WORKSPACE
    assert b"plan needs" in q.qwha_last_error()
    need = q.qwha_plan_bytes(256, 256, 2048)
    assert build(nb=need, plan=FAKE + 64) == ALIGN

    def fp(**kw):
        a = dict(x=FAKE, z_in=None, act=1, T=16, d_in=256, d_out=256, p=2048, plan=FAKE,
                 c=FAKE, alpha=1.0, y=FAKE, acc=0, z_out=None, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_fwd_plan(a["x"], a["z_in"], a["act"], a["T"], a["d_in"], a["d_out"],
                               a["p"], a["plan"], a["c"], a["alpha"], a["y"], a["acc"],
                               a["z_out"], a["ws"], a["wsb"], None)
    assert fp(d_in=12) == SHAPE
    assert fp(act=7) == DTYPE
    assert fp(z_in=FAKE, z_out=FAKE) == INVALID
    assert fp(plan=None) == INVALID
    assert fp(x=None) == INVALID                         # neither x nor z_in
    assert fp(acc=2) == INVALID
    assert fp() == WORKSPACE                             # z needs room
    assert fp(T=0, x=None) == OK
    # with z kept by the caller no workspace is needed: the next check is y's
    assert fp(z_out=FAKE, y=FAKE + 8) == ALIGN
    assert fp(z_in=FAKE, x=None, y=FAKE + 8) == ALIGN

    def bp(**kw):
        a = dict(z=FAKE, dy=FAKE, act=1, T=16, d_in=256, d_out=256, p=2048, plan=FAKE, c=FAKE,
                 alpha=1.0, dx=FAKE, accx=0, dz=None, accz=0, dc=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_bwd_plan(a["z"], a["dy"], a["act"], a["T"], a["d_in"], a["d_out"],
                               a["p"], a["plan"], a["c"], a["alpha"], a["dx"], a["accx"],
                               a["dz"], a["accz"], a["dc"], a["ws"], a["wsb"], None)
    assert bp(dz=FAKE) == INVALID                        # dx and dz are exclusive
    assert bp(dc=None) == INVALID
    assert bp(dc=FAKE + 2) == ALIGN
    assert bp(accx=2) == INVALID
    assert bp(accz=3, dx=None, dz=FAKE) == INVALID
    assert bp(alpha=float("inf")) == INVALID
    assert bp(z=None) == INVALID
    assert bp() == WORKSPACE
    assert b"bwd workspace" in q.qwha_last_error()
    # qwha_bwd_workspace_bytes suffices for every form
    wb = q.qwha_bwd_workspace_bytes(16, 256, 256, 2048)
    assert bp(wsb=wb, ws=FAKE + 64) == ALIGN
    assert bp(wsb=wb, ws=FAKE + 64, dx=None, dz=FAKE) == ALIGN


def test_stream_position_limit(q):
    # the SpMM stream holds at most 2p + 16 entries at int32 positions: p is
    # capped at (2^31 - 65) // 2 for the calls that build it
    big = dict(d_out=65536, d_in=16384)
    limit = (2**31 - 1 - 64) // 2
    assert _fwd(q, p=limit + 1, **big) == BUDGET
    assert b"stream" in q.qwha_last_error()
    # at the limit the budget passes and the (absent) workspace is what fails
    assert _fwd(q, p=limit, **big) == WORKSPACE
    assert q.qwha_fwd_workspace_bytes(16, 16384, 65536, limit + 1) == 0
    assert q.qwha_bwd_workspace_bytes(16, 16384, 65536, limit + 1) == 0
    assert q.qwha_layer_fwd_workspace_bytes(16, 16384, 65536, limit + 1) == 0
    assert q.qwha_fwd_workspace_bytes(16, 16384, 65536, limit) > 0


def test_init_validation(q):
    def call(**kw):
        a = dict(dWq=FAKE, d_out=256, d_in=256, p=2048, m=3, t=1.0, row_ptr=FAKE, E=FAKE,
                 c=FAKE, col_ptr=FAKE, perm=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_init_select(a["dWq"], a["d_out"], a["d_in"], a["p"], a["m"], a["t"],
                                  a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["perm"],
                                  a["ws"], a["wsb"], None)
    assert call(p=3 * 256 - 1) == BUDGET            # below the per-row floor
    assert call(p=256 * 256 + 1) == BUDGET
    assert call(m=-1) == INVALID
    assert call(t=0.0) == INVALID
    assert call(t=float("nan")) == INVALID
    assert call(d_in=100) == SHAPE
    assert call(dWq=FAKE + 8) == ALIGN
    assert call(E=None) == INVALID
    assert call() == WORKSPACE                      # everything else fine, no workspace


def test_init_global_validation(q):
    def call(**kw):
        a = dict(dWq=FAKE, d_out=256, d_in=256, p=2048, st=1, seed=7, row_ptr=FAKE, E=FAKE,
                 c=FAKE, col_ptr=FAKE, perm=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_init_select_global(a["dWq"], a["d_out"], a["d_in"], a["p"], a["st"],
                                         a["seed"], a["row_ptr"], a["E"], a["c"], a["col_ptr"],
                                         a["perm"], a["ws"], a["wsb"], None)
    assert call(p=256 * 256 + 1) == BUDGET
    assert call(p=-1) == BUDGET
    assert call(st=0) == INVALID
    assert call(st=3) == INVALID
    assert call(d_in=100) == SHAPE
    assert call(d_out=0) == SHAPE
    assert call(dWq=FAKE + 8) == ALIGN
    assert call(E=None) == INVALID
    assert call(row_ptr=None) == INVALID
    assert call() == WORKSPACE                      # everything else fine, no workspace
    assert call(st=2, wsb=q.qwha_init_global_workspace_bytes(256, 256, 2) - 1) == WORKSPACE
    assert call(st=2, ws=FAKE + 16, wsb=1 << 30) == ALIGN
    assert call(seed=(1 << 64) - 1, ws=None) == WORKSPACE     # full 64-bit seeds accepted


def test_calibration_validation(q):
    # qwha_hessian(X, dtype, N, d_in, Hs, accumulate, stream)
    assert q.qwha_hessian(FAKE, 0, 10, 24, FAKE, 0, None) == SHAPE
    assert q.qwha_hessian(FAKE, 0, -1, 64, FAKE, 0, None) == SHAPE
    assert q.qwha_hessian(FAKE, 3, 10, 64, FAKE, 0, None) == DTYPE
    assert q.qwha_hessian(FAKE, 0, 10, 64, FAKE, 2, None) == INVALID
    assert q.qwha_hessian(FAKE, 0, 10, 64, None, 0, None) == INVALID
    assert q.qwha_hessian(FAKE + 4, 1, 10, 64, FAKE, 0, None) == ALIGN
    assert q.qwha_hessian(None, 0, 10, 64, FAKE, 0, None) == INVALID

    def init(**kw):
        a = dict(dWq=FAKE, d_out=256, d_in=256, Hs=FAKE, damp=0.0, p=2048, m=3, t=1.0,
                 row_ptr=FAKE, E=FAKE, c=FAKE, col_ptr=FAKE, perm=FAKE, G=FAKE, rhs=FAKE,
                 ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_init_select_calibrated(
            a["dWq"], a["d_out"], a["d_in"], a["Hs"], a["damp"], a["p"], a["m"], a["t"],
            a["row_ptr"], a["E"], a["c"], a["col_ptr"], a["perm"], a["G"], a["rhs"], a["ws"],
            a["wsb"], None)
    assert init(damp=-0.1) == INVALID
    assert init(damp=float("inf")) == INVALID
    assert init(p=3 * 256 - 1) == BUDGET
    assert init(Hs=None) == INVALID
    assert init(G=FAKE + 8) == ALIGN
    assert init(rhs=None) == INVALID
    assert init(d_in=96) == SHAPE
    assert init() == WORKSPACE
    need = q.qwha_init_calibrated_workspace_bytes(256, 256)
    assert need >= 256 * 256 * 8 * 2       # dW_Q Hs and one d_in x d_in temporary
    assert init(wsb=need - 1) == WORKSPACE

    def refine(**kw):
        a = dict(row_ptr=FAKE, E=FAKE, G=FAKE, rhs=FAKE, d_out=4, d_in=64, p=20, c=FAKE,
                 status=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return q.qwha_refine_values(a["row_ptr"], a["E"], a["G"], a["rhs"], a["d_out"],
                                    a["d_in"], a["p"], a["c"], a["status"], a["ws"], a["wsb"],
                                    None)
    assert refine(d_in=63) == SHAPE
    assert refine(p=4 * 64 + 1) == BUDGET
    assert refine(status=None) == INVALID
    assert refine(rhs=None) == INVALID
    assert refine() == WORKSPACE
    assert refine(ws=FAKE + 16, wsb=1 << 20) == ALIGN


def test_refine_workspace_query_on_host_row_ptr(q):
    rp = np.array([0, 3, 3, 10, 11], dtype=np.int32)
    got = q.qwha_refine_workspace_bytes(rp.ctypes.data, 4)
    tri = sum((k + 1) * (k + 2) // 2 for k in np.diff(rp))     # augmented triangles
    header = ((5 * 8 + 255) // 256) * 256
    assert got == header + 8 * tri
    assert q.qwha_refine_workspace_bytes(None, 4) == 0
    bad = np.array([0, 3, 2, 4, 5], dtype=np.int32)
    assert q.qwha_refine_workspace_bytes(bad.ctypes.data, 4) == 0
    assert q.qwha_refine_workspace_bytes(np.array([1, 2], np.int32).ctypes.data, 1) == 0


def test_quantized_base_validation(q):
    def merge(**kw):
        a = dict(codes=FAKE, s=FAKE, z=FAKE, bits=4, group=128, d_out=64, d_in=256, p=500,
                 row_ptr=FAKE, E=FAKE, c=FAKE, alpha=1.0, out=0, W=FAKE)
        a.update(kw)
        return q.qwha_merge(a["codes"], a["s"], a["z"], a["bits"], a["group"], a["d_out"],
                            a["d_in"], a["p"], a["row_ptr"], a["E"], a["c"], a["alpha"],
                            a["out"], a["W"], None)
    assert merge(bits=5) == INVALID
    assert merge(group=96) == INVALID
    assert merge(group=512) == INVALID
    assert merge(out=2) == DTYPE
    assert merge(codes=None) == INVALID
    assert merge(W=FAKE + 8) == ALIGN
    assert merge(d_in=100) == SHAPE
    assert merge(alpha=float("nan")) == INVALID
    # a block width (320 = 5 * 64) is a valid d_in, but groups of 128 would
    # leave a partial last group with no scale / zero of its own
    assert merge(d_in=320, group=128) == INVALID
    assert merge(d_in=320, group=64, W=FAKE + 8) == ALIGN   # passes the group check

    def fwd(**kw):
        a = dict(x=FAKE, act=1, T=128, d_in=256, d_out=64, codes=FAKE, s=FAKE, z=FAKE, bits=4,
                 group=128, p=500, row_ptr=FAKE, E=FAKE, c=FAKE, alpha=1.0, y=FAKE, ws=FAKE,
                 wsb=0)
        a.update(kw)
        return q.qwha_layer_fwd(a["x"], a["act"], a["T"], a["d_in"], a["d_out"], a["codes"],
                                a["s"], a["z"], a["bits"], a["group"], a["p"], a["row_ptr"],
                                a["E"], a["c"], a["alpha"], a["y"], a["ws"], a["wsb"], None)
    assert fwd(act=0) == DTYPE                  # the base GEMM takes bf16 activations
    assert fwd(d_in=16, group=16) == SHAPE
    assert fwd(d_in=32, group=32) == SHAPE       # below one 64-deep step
    assert fwd(group=16) == INVALID              # groups below one MFMA depth
    assert fwd(bits=1) == INVALID
    assert fwd(x=FAKE + 2) == ALIGN
    assert fwd(d_in=320, group=128) == INVALID   # group does not divide d_in
    assert fwd(d_in=320, group=64) == WORKSPACE
    assert fwd() == WORKSPACE
    need = q.qwha_layer_fwd_workspace_bytes(128, 256, 64, 500)
    assert need >= 128 * 64 * 4 + 128 * 256 * 4
    assert fwd(wsb=need - 1) == WORKSPACE
    assert fwd(T=0, x=None, y=None) == OK        # nothing to do


def test_block_widths_pass_shape_validation(q):
    # widths m * b with b >= 64 reach the workspace check; narrower blocks do not
    for d_in, ok in ((14336, True), (192, True), (11008, True), (96, False), (100, False),
                     (20480, False)):
        r = _fwd(q, d_in=d_in, p=2048)
        assert r == (WORKSPACE if ok else SHAPE), (d_in, r)
        r = q.qwha_init_select(FAKE, 64, d_in, 192, 3, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                               None)
        assert r == (WORKSPACE if ok else SHAPE), (d_in, r)
    assert q.qwha_fwht(FAKE, 0, FAKE, 0, 4, 192, 1.0, None) == SHAPE   # powers of two only


def test_saved_activation_validation(q):
    # qwha_fwd_save: as qwha_fwd plus z; qwha_bwd_saved: z in place of x
    r = q.qwha_fwd_save(FAKE, 1, 16, 256, 256, 2048, FAKE, FAKE, FAKE, 1.0, FAKE, 0, None,
                        FAKE, 1 << 30, None)
    assert r == INVALID
    r = q.qwha_fwd_save(FAKE, 1, 16, 256, 256, 2048, FAKE, FAKE, FAKE, 1.0, FAKE, 0, FAKE + 4,
                        FAKE, 1 << 30, None)
    assert r == ALIGN
    r = q.qwha_bwd_saved(None, FAKE, 1, 64, 256, 256, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0,
                         FAKE, 0, FAKE, FAKE, 1 << 30, None)
    assert r == INVALID                          # dc wanted, no z
    r = q.qwha_bwd_saved(FAKE + 8, FAKE, 1, 64, 256, 256, 2048, FAKE, FAKE, FAKE, FAKE, FAKE,
                         1.0, FAKE, 0, FAKE, FAKE, 1 << 30, None)
    assert r == ALIGN


def test_bwd_materialize_fwht_validation(q):
    assert q.qwha_materialize(FAKE, FAKE, FAKE, 4, 24, 8, 1.0, 0, FAKE, 0, None) == SHAPE
    assert q.qwha_materialize(FAKE, FAKE, FAKE, 4, 16, 8, 1.0, 5, FAKE, 0, None) == DTYPE
    assert q.qwha_materialize(FAKE, FAKE, FAKE, 4, 16, 8, 1.0, 0, None, 0, None) == INVALID
    assert q.qwha_fwht(FAKE, 0, FAKE, 0, 4, 48, 1.0, None) == SHAPE
    assert q.qwha_fwht(FAKE, 0, FAKE + 4, 0, 4, 64, 1.0, None) == ALIGN
    assert q.qwha_sign_update(FAKE, FAKE, -1, 1e-3, None) == BUDGET
    r = q.qwha_bwd(FAKE, FAKE, 1, 64, 256, 256, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0,
                   FAKE, 0, FAKE, FAKE, 0, None)
    assert r == WORKSPACE
    r = q.qwha_bwd(FAKE, FAKE, 1, 64, 256, 256, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0,
                   FAKE + 8, 0, FAKE, FAKE, 1 << 30, None)
    assert r == ALIGN
