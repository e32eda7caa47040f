"""Throughput of the Walsh-Hadamard adapter hot path on one MI355X.

One step = one pass of the whole hot path over one batch, every kernel in
the library's HIP code, on torch's current stream:
  init (row norms, AdaAlloc budgets, fp64 transform + in-row top-k, column
  index) -> materialize dW -> forward (FWHT(x), gather-SpMM; z = FWHT(x)/n
  kept as the saved activation) -> backward (gather-SpMM dz and dc partials
  against the saved z, FWHT(dz) -> dx, dc reduction) ->
  c += 1e-3 sign(dc) -> re-materialize dW.
value = tokens per second of that step (T / step time), inputs resident in HBM.

Workload (default): the 4096x4096 q_proj-shaped layer, 4-bit RTN (group 128)
error with 0.1% x20 outliers, budget p = 524288 (rank-64 LoRA parameter
count), 8192 bf16 tokens. Four copies of the inputs are rotated so the
working set exceeds the 256 MB Infinity Cache.

Per-kernel times come from HIP events recorded by the library around each
kernel launch (qwha_profile_next), on the launch stream, over the timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X vector fp32 (packed FMA)

# timed kernels of the step (the backward takes the forward's z, so the
# library's BWD_FWHT_X transform does not run)
K = dict(FWD_FWHT=1, FWD_SPMM=2, BWD_SPMM=4, BWD_FWHT_DX=5, BWD_DC_REDUCE=6,
         INIT_SELECT=7, MATERIALIZE=8)
GLOBAL_THRESHOLD = 10
KR = dict(HESSIAN=11, CALIB_PREPARE=12, CALIB_SYSTEM=13, REFINE=14)
KQ = dict(MERGE=15, QGEMM=16)
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix
FP64_MFMA_PEAK_TFLOPS = 78.6     # MI355X dense fp64 matrix
FP64_VECTOR_PEAK_TFLOPS = 78.6   # MI355X fp64 vector


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--sets", type=int, default=4, help="rotated input copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--refine-tokens", type=int, default=32768,
                    help="calibration tokens for the refinement measurement (0: skip)")
    ap.add_argument("--refine-reps", type=int, default=3)
    ap.add_argument("--base-reps", type=int, default=10,
                    help="timed calls of the quantized base layer (0: skip)")
    ap.add_argument("--variant-reps", type=int, default=10,
                    help="timed calls of each init selection strategy (0: skip)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: all of the workload's)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain fp32 copy kernel of this size (read + write) after the "
                         "warmup, to calibrate HBM byte counters")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvents from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return ms.value


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in the design notes, not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import quantization_aware_sparse_amd as q
    from quantization_aware_sparse_amd import check, lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    spec = synth.config_specs(args.config)[0]
    d_out, d_in, p, T = spec.d_out, spec.d_in, spec.p, spec.T
    act = q.QWHA_BF16 if spec.act == "bf16" else q.QWHA_F32
    adt = torch.bfloat16 if spec.act == "bf16" else torch.float32
    esz = 2 if spec.act == "bf16" else 4

    t_gen = time.perf_counter()
    layer = synth.make_layer(spec, seed=0)
    x_np, dy_np = synth.make_activations(spec, seed=0)
    gen_s = time.perf_counter() - t_gen

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    base = (up(layer.dwq), up(x_np), up(dy_np))
    for s in range(args.sets):
        sets.append(tuple(b.clone() for b in base))
    del base

    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr = torch.empty(d_out + 1, **i32)
    E = torch.empty((p, 2), **i32)
    c = torch.empty(p, dtype=torch.float32, device=dev)
    col_ptr = torch.empty(d_in + 1, **i32)
    perm = torch.empty(p, **i32)
    dW = torch.empty((d_out, d_in), dtype=torch.float32, device=dev)
    y = torch.empty((T, d_out), dtype=adt, device=dev)
    dx = torch.empty((T, d_in), dtype=adt, device=dev)
    dc = torch.empty(p, dtype=torch.float32, device=dev)
    zsave = torch.empty((T, d_in), dtype=torch.float32, device=dev)   # saved activation
    ws_i = torch.empty(lib.qwha_init_workspace_bytes(d_out, d_in), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(lib.qwha_bwd_workspace_bytes(T, d_in, d_out, p), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    hip = HipEvents()
    ev = {name: (hip.create(), hip.create()) for name in K}
    times = {name: [] for name in K}

    def step(s, record):
        dwq, x, dy = sets[s % len(sets)]
        if record:
            for name, kid in K.items():
                check(lib.qwha_profile_next(kid, ev[name][0], ev[name][1]), "profile")
        check(lib.qwha_init_select(dwq.data_ptr(), d_out, d_in, p, 3, 1.0, row_ptr.data_ptr(),
                                   E.data_ptr(), c.data_ptr(), col_ptr.data_ptr(),
                                   perm.data_ptr(), ws_i.data_ptr(), ws_i.numel(), stream),
              "init")
        check(lib.qwha_materialize(row_ptr.data_ptr(), E.data_ptr(), c.data_ptr(), d_out, d_in,
                                   p, 1.0, q.QWHA_F32, dW.data_ptr(), 0, stream), "materialize")
        check(lib.qwha_fwd_save(x.data_ptr(), act, T, d_in, d_out, p, row_ptr.data_ptr(),
                                E.data_ptr(), c.data_ptr(), 1.0, y.data_ptr(), 0,
                                zsave.data_ptr(), ws_f.data_ptr(), ws_f.numel(), stream), "fwd")
        check(lib.qwha_bwd_saved(zsave.data_ptr(), dy.data_ptr(), act, T, d_in, d_out, p,
                                 row_ptr.data_ptr(), E.data_ptr(), c.data_ptr(),
                                 col_ptr.data_ptr(), perm.data_ptr(), 1.0, dx.data_ptr(), 0,
                                 dc.data_ptr(), ws_b.data_ptr(), ws_b.numel(), stream), "bwd")
        check(lib.qwha_sign_update(c.data_ptr(), dc.data_ptr(), p, 1e-3, stream), "update")
        check(lib.qwha_materialize(row_ptr.data_ptr(), E.data_ptr(), c.data_ptr(), d_out, d_in,
                                   p, 1.0, q.QWHA_F32, dW.data_ptr(), 0, stream), "rematerialize")

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b
    print(f"# warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr,
          flush=True)

    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, True)
        # the next step's requests reuse these events: read them first
        torch.cuda.synchronize()
        for name in K:
            times[name].append(hip.elapsed_ms(*ev[name]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # clean timing without per-step host waits: the figure `value` reports
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        step(s, False)
    torch.cuda.synchronize()
    wall_clean = time.perf_counter() - t1
    ms_step = 1e3 * wall_clean / args.steps
    value = T / (ms_step / 1e3)

    avg_us = {k: 1e3 * float(np.mean(v)) for k, v in times.items()}
    # algorithmic work per launch
    nbytes = {
        "FWD_FWHT": T * d_in * (esz + 4),
        "BWD_FWHT_DX": T * d_in * (4 + esz),
        "INIT_SELECT": d_out * d_in * 4 + p * 12 + (d_out + 1) * 4,
        "MATERIALIZE": p * 12 + (d_out + 1) * 4 + d_out * d_in * 4,
        "BWD_DC_REDUCE": 0,
    }
    flops = {"FWD_SPMM": 2.0 * T * p, "BWD_SPMM": 4.0 * T * p}
    kern = {}
    for k, us in avg_us.items():
        if k in flops:
            a = flops[k] / (us * 1e-6) / 1e12
            kern[k] = dict(avg_us=round(us, 2), bound="alu", achieved=round(a, 3),
                           unit="TFLOP/s", peak=FP32_VECTOR_PEAK_TFLOPS,
                           frac=round(a / FP32_VECTOR_PEAK_TFLOPS, 4))
        elif nbytes.get(k):
            a = nbytes[k] / (us * 1e-6) / 1e9
            kern[k] = dict(avg_us=round(us, 2), bound="hbm", achieved=round(a, 1), unit="GB/s",
                           peak=HBM_PEAK_GBS, frac=round(a / HBM_PEAK_GBS, 4))
        else:
            kern[k] = dict(avg_us=round(us, 2))
    dom = max(avg_us, key=avg_us.get)
    roof = dict(kern[dom])
    roof.pop("avg_us", None)
    roof["kernel"] = dom
    roof["avg_us"] = round(avg_us[dom], 2)
    roof["traffic"] = measured_traffic(dom, args.config)

    fwd_bwd_us = sum(avg_us[k] for k in ("FWD_FWHT", "FWD_SPMM", "BWD_SPMM", "BWD_FWHT_DX",
                                         "BWD_DC_REDUCE"))
    out = {
        "metric": "adapter fwd+bwd tokens/s per layer; FWHT/gather achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{spec.name}: {d_out}x{d_in} layer, {spec.bits}-bit RTN g{spec.group} "
                        f"error with {spec.outlier_frac:.1%} x{spec.outlier_mult:g} outliers, "
                        f"p={p}, {T} {spec.act} tokens; step = init + materialize + fwd + bwd "
                        "+ sign update + re-materialize",
            "d_out": d_out, "d_in": d_in, "p": p, "tokens": T, "act": spec.act,
            "input_sets_rotated": args.sets,
        },
        "roofline": roof,
        "kernels": kern,
        "fwd_bwd_kernels_us": round(fwd_bwd_us, 2),
        "fwd_bwd_tokens_per_s": round(T / (fwd_bwd_us * 1e-6), 1),
        "profiled_steps_ms": round(1e3 * wall / args.steps, 4),
        "input_gen_s": round(gen_s, 2),
    }

    if args.variant_reps > 0:
        out["init_variants"] = init_variants(args.variant_reps, sets, (d_out, d_in, p),
                                             (row_ptr, E, c, col_ptr, perm), ws_i, stream, hip)

    if args.base_reps > 0:
        out["base_layer"] = base_layer_measure(args.base_reps, spec, layer, sets,
                                               (row_ptr, E, c), stream, hip)

    if args.refine_tokens > 0 and args.refine_reps > 0:
        out["refine"] = refine_measure(args.refine_tokens, args.refine_reps, spec, sets[0][0],
                                       stream, hip)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, layer, x_np, dy_np, args.cpu_tokens or T)
    print(json.dumps(out), flush=True)


def init_variants(reps, sets, dims, outs, ws_i, stream, hip):
    """Time the init under each selection strategy on the same layer and
    budget: AdaAlloc (qwha_init_select) and the global magnitude / random
    selections (qwha_init_select_global), whole call and, for the global
    ones, the threshold stage (keys, radix select, budgets) and the per-row
    select kernel. Achieved rates use the stage's own traffic by design:
    magnitude reads dW_Q once and writes its 8-byte keys once, then reads
    them in 8 radix passes and one tie count (84 B per position); random
    draws SplitMix64 in 9 passes over all positions and keeps nothing."""
    import numpy as np
    import torch
    from quantization_aware_sparse_amd import check, lib
    d_out, d_in, p = dims
    row_ptr, E, c, col_ptr, perm = (t.data_ptr() for t in outs)
    n = d_out * d_in
    ev = [hip.create() for _ in range(6)]
    res = {}
    for name, strat in (("adaalloc", 0), ("magnitude", 1), ("random", 2)):
        if strat:
            ws = torch.empty(lib.qwha_init_global_workspace_bytes(d_out, d_in, strat),
                             dtype=torch.uint8, device="cuda:0")
        else:
            ws = ws_i

        def call(s):
            dwq = sets[s % len(sets)][0].data_ptr()
            if strat:
                return lib.qwha_init_select_global(dwq, d_out, d_in, p, strat, 17 + s, row_ptr,
                                                   E, c, col_ptr, perm, ws.data_ptr(),
                                                   ws.numel(), stream)
            return lib.qwha_init_select(dwq, d_out, d_in, p, 3, 1.0, row_ptr, E, c, col_ptr,
                                        perm, ws.data_ptr(), ws.numel(), stream)
        for s in range(2):
            check(call(s), name)
        torch.cuda.synchronize()
        whole, thr, sel = [], [], []
        for s in range(reps):
            check(lib.qwha_profile_next(K["INIT_SELECT"], ev[2], ev[3]), "profile")
            if strat:
                check(lib.qwha_profile_next(GLOBAL_THRESHOLD, ev[4], ev[5]), "profile")
            hip.record(ev[0], stream)
            check(call(s), name)
            hip.record(ev[1], stream)
            torch.cuda.synchronize()
            whole.append(hip.elapsed_ms(ev[0], ev[1]))
            sel.append(hip.elapsed_ms(ev[2], ev[3]))
            if strat:
                thr.append(hip.elapsed_ms(ev[4], ev[5]))
        r = {"init_us": round(1e3 * float(np.mean(whole)), 2),
             "select_us": round(1e3 * float(np.mean(sel)), 2)}
        if strat:
            t_us = 1e3 * float(np.mean(thr))
            r["threshold_us"] = round(t_us, 2)
            if strat == 1:
                a = 84.0 * n / (t_us * 1e-6) / 1e9
                r["threshold_roofline"] = dict(bound="hbm", achieved=round(a, 1), unit="GB/s",
                                               peak=HBM_PEAK_GBS, frac=round(a / HBM_PEAK_GBS, 4),
                                               bytes_per_position=84)
            else:
                r["threshold_gdraws_per_s"] = round(9.0 * n / (t_us * 1e-6) / 1e9, 1)
        res[name] = r
        del ws
    res["calls"] = reps
    res["layer"] = f"{d_out}x{d_in}, p={p}"
    return res


def base_layer_measure(reps, spec, layer, sets, adapter, stream, hip):
    """Time the quantized base layer with the adapter on the workload: the
    layer forward y = x W_Q^T + alpha z F^T (qwha_layer_fwd, bf16 tokens;
    W_Q as the fixture's b-bit codes) and the merge W_Q + alpha dW
    (qwha_merge, bf16 out). Rates: the base GEMM's 2 T d_in d_out flops
    against the dense bf16 matrix peak; the merge's bytes (codes, scales and
    zeros, E and c, row_ptr, the bf16 output) against HBM peak."""
    import numpy as np
    import torch
    import synth
    from quantization_aware_sparse_amd import check, lib
    d_out, d_in, p, T = spec.d_out, spec.d_in, spec.p, spec.T
    qc, sc, zr = synth.rtn_codes(layer.w0, spec.bits, spec.group)
    words = synth.pack_codes(qc, spec.bits)
    dev = "cuda:0"
    codes = torch.from_numpy(words.view(np.int32)).to(dev)
    scales = torch.from_numpy(sc).to(dev)
    zeros = torch.from_numpy(zr).to(dev)
    row_ptr, E, c = adapter
    y = torch.empty((T, d_out), dtype=torch.bfloat16, device=dev)
    W = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.qwha_layer_fwd_workspace_bytes(T, d_in, d_out, p), dtype=torch.uint8,
                     device=dev)
    ev = {k: (hip.create(), hip.create()) for k in list(KQ) + ["LAYER"]}
    times = {k: [] for k in ev}
    for r in range(reps + 2):
        rec = r >= 2
        x = sets[r % len(sets)][1]
        if rec:
            for k, kid in KQ.items():
                check(lib.qwha_profile_next(kid, ev[k][0], ev[k][1]), "profile")
            hip.record(ev["LAYER"][0], stream)
        check(lib.qwha_layer_fwd(x.data_ptr(), 1, T, d_in, d_out, codes.data_ptr(),
                                 scales.data_ptr(), zeros.data_ptr(), spec.bits, spec.group, p,
                                 row_ptr.data_ptr(), E.data_ptr(), c.data_ptr(), 1.0,
                                 y.data_ptr(), ws.data_ptr(), ws.numel(), stream), "layer fwd")
        if rec:
            hip.record(ev["LAYER"][1], stream)
        check(lib.qwha_merge(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), spec.bits,
                             spec.group, d_out, d_in, p, row_ptr.data_ptr(), E.data_ptr(),
                             c.data_ptr(), 1.0, 1, W.data_ptr(), stream), "merge")
        torch.cuda.synchronize()
        if rec:
            for k in ev:
                times[k].append(hip.elapsed_ms(*ev[k]))
    us = {k: 1e3 * float(np.mean(v)) for k, v in times.items()}
    flops = 2.0 * T * d_in * d_out
    a_q = flops / (us["QGEMM"] * 1e-6) / 1e12
    mbytes = (words.nbytes + sc.nbytes + zr.nbytes + 12 * p + 4 * (d_out + 1)
              + 2 * d_out * d_in)
    a_m = mbytes / (us["MERGE"] * 1e-6) / 1e9
    return {
        "weights": f"{spec.bits}-bit codes, group {spec.group} (the fixture's RTN), "
                   f"{d_out}x{d_in}; adapter p={p}; {T} bf16 tokens",
        "reps": reps,
        "layer_fwd_us": round(us["LAYER"], 1),
        "layer_fwd_tokens_per_s": round(T / (us["LAYER"] * 1e-6), 1),
        "base_gemm_us": round(us["QGEMM"], 1),
        "merge_us": round(us["MERGE"], 1),
        "base_gemm_roofline": dict(bound="mfma", achieved=round(a_q, 1), unit="TFLOP/s",
                                   peak=BF16_MFMA_PEAK_TFLOPS,
                                   frac=round(a_q / BF16_MFMA_PEAK_TFLOPS, 4), dtype="bf16"),
        "merge_roofline": dict(bound="hbm", achieved=round(a_m, 1), unit="GB/s",
                               peak=HBM_PEAK_GBS, frac=round(a_m / HBM_PEAK_GBS, 4),
                               bytes=int(mbytes)),
    }


def refine_measure(N, reps, spec, dwq, stream, hip):
    """Time the init with a calibration Hessian on the layer: Hs = X^T X over
    N synthetic bf16 calibration tokens (qwha_hessian), the calibrated init
    (qwha_init_select_calibrated: dW_Q Hs, norms, AdaAlloc, selection, G and
    rhs) and the per-row solves (qwha_refine_values). Rates: the Hessian's
    N d_in (d_in + 1) flops (a symmetric rank-N update) against the fp64
    matrix-core peak; dW_Q Hs's 2 d_out d_in^2 flops inside the preparation
    step; the solves' sum over rows of (p_i + 1)^3 / 3 flops (Cholesky of the
    augmented system) + p_i^2 (back substitution) against the fp64 vector peak."""
    import numpy as np
    import torch
    import synth
    import quantization_aware_sparse_amd as q
    from quantization_aware_sparse_amd import check, lib
    d_out, d_in, p = spec.d_out, spec.d_in, spec.p
    X = synth.make_calibration(d_in, N, seed=1, act="bf16")
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    del X
    Hs = torch.empty((d_in, d_in), dtype=torch.float64, device="cuda:0")
    got = None
    ev = {k: (hip.create(), hip.create()) for k in list(KR) + ["WHOLE"]}
    times = {k: [] for k in ev}
    ws_c = q.workspace(lib.qwha_init_calibrated_workspace_bytes(d_out, d_in), "cuda:0")
    ws_r = None
    status = torch.empty(2, dtype=torch.int32, device="cuda:0")
    for r in range(reps + 1):
        timed_rep = r > 0
        if timed_rep:
            for k, kid in KR.items():
                check(lib.qwha_profile_next(kid, ev[k][0], ev[k][1]), "profile")
            hip.record(ev["WHOLE"][0], stream)
        check(lib.qwha_hessian(Xd.data_ptr(), q.QWHA_BF16, N, d_in, Hs.data_ptr(), 0, stream),
              "hessian")
        got = q.qwha_init_select_calibrated(dwq, Hs, p, 3, ws=ws_c)
        if ws_r is None:
            ws_r = q.workspace(q.refine_workspace_bytes(got["row_ptr"]), "cuda:0")
        check(lib.qwha_refine_values(got["row_ptr"].data_ptr(), got["E"].data_ptr(),
                                     got["G"].data_ptr(), got["rhs"].data_ptr(), d_out, d_in, p,
                                     got["c"].data_ptr(), status.data_ptr(), ws_r.data_ptr(),
                                     ws_r.numel(), stream), "refine")
        if timed_rep:
            hip.record(ev["WHOLE"][1], stream)
        torch.cuda.synchronize()
        if timed_rep:
            for k in ev:
                times[k].append(hip.elapsed_ms(*ev[k]))
    us = {k: 1e3 * float(np.mean(v)) for k, v in times.items()}
    budgets = np.diff(got["row_ptr"].cpu().numpy().astype(np.int64))
    refine_flops = float(np.sum((budgets + 1.0) ** 3 / 3.0 + budgets.astype(np.float64) ** 2))
    hess_flops = float(N) * d_in * (d_in + 1)
    gemm_flops = 2.0 * d_out * d_in * d_in
    a_h = hess_flops / (us["HESSIAN"] * 1e-6) / 1e12
    a_g = gemm_flops / (us["CALIB_PREPARE"] * 1e-6) / 1e12
    a_r = refine_flops / (us["REFINE"] * 1e-6) / 1e12
    return {
        "calibration": f"{N} synthetic bf16 tokens (per-channel scales, 0.5% x10 outlier "
                       "channels)",
        "reps": reps,
        "status": status.cpu().tolist(),
        "whole_us": round(us["WHOLE"], 1),
        "hessian_us": round(us["HESSIAN"], 1),
        "calib_prepare_us": round(us["CALIB_PREPARE"], 1),
        "calib_system_us": round(us["CALIB_SYSTEM"], 1),
        "refine_us": round(us["REFINE"], 1),
        "hessian_roofline": dict(bound="mfma", achieved=round(a_h, 2), unit="TFLOP/s",
                                 peak=FP64_MFMA_PEAK_TFLOPS,
                                 frac=round(a_h / FP64_MFMA_PEAK_TFLOPS, 4), dtype="f64"),
        "calib_gemm_roofline": dict(bound="mfma", achieved=round(a_g, 2), unit="TFLOP/s",
                                    peak=FP64_MFMA_PEAK_TFLOPS,
                                    frac=round(a_g / FP64_MFMA_PEAK_TFLOPS, 4), dtype="f64",
                                    note="time of the whole preparation step"),
        "refine_rate": dict(bound="alu", achieved=round(a_r, 3), unit="TFLOP/s",
                            peak=FP64_VECTOR_PEAK_TFLOPS,
                            frac=round(a_r / FP64_VECTOR_PEAK_TFLOPS, 4), dtype="f64"),
    }


# library sources that define each timed kernel (besides the shared headers
# and the launch layer, which every kernel depends on)
KERNEL_SOURCES = {
    "FWD_FWHT": ["fwht.hip", "fwht_core.h"], "BWD_FWHT_X": ["fwht.hip", "fwht_core.h"],
    "BWD_FWHT_DX": ["fwht.hip", "fwht_core.h"], "FWD_SPMM": ["spmm.hip"],
    "BWD_SPMM": ["spmm.hip"], "BWD_DC_REDUCE": ["spmm.hip"],
    "INIT_SELECT": ["init.hip", "fwht_core.h"], "MATERIALIZE": ["materialize.hip", "fwht_core.h"],
    "GLOBAL_THRESHOLD": ["select_global.hip", "fwht_core.h"],
    "HESSIAN": ["refine.hip", "fwht_core.h"], "CALIB_PREPARE": ["refine.hip", "fwht_core.h"],
    "CALIB_SYSTEM": ["refine.hip", "fwht_core.h"], "REFINE": ["refine.hip", "fwht_core.h"],
    "MERGE": ["quant.hip", "fwht_core.h"], "QGEMM": ["quant.hip"],
}
SHARED_SOURCES = ["common.h", "launch.h", "api.hip"]


def strip_comments(text):
    """C++ source without its comments and blank space: what the compiler
    sees, so that a comment edit does not count as a change of the code."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def source_digest(kernel):
    """sha256 over the code (comments and spacing left out) of the HIP
    sources a kernel is built from: a traffic figure measured on other code
    is stale."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantization_aware_sparse_amd", "csrc")
    for name in sorted(set(KERNEL_SOURCES[kernel] + SHARED_SOURCES)):
        with open(os.path.join(d, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, config):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none for this workload and these exact sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}.md")
    if not os.path.exists(path):
        return None
    digest = source_digest(kernel)
    with open(path) as f:
        for line in f:
            if line.startswith("traffic:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("kernel") == kernel and kv.get("sources") == digest:
                    return int(kv["bytes"])
    return None


def cpu_baseline(spec, layer, x_np, dy_np, n_tok, min_seconds=10.0):
    """The fp64 oracle (as it stands) on the host cores: whole steps of the
    same path (init, materialize, fwd, bwd, update, re-materialize) on the
    full layer with n_tok of the workload's tokens, repeated until at least
    min_seconds have passed. With n_tok < T the fwd+bwd share is scaled
    linearly to T tokens."""
    import numpy as np
    import oracle as O
    import synth
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # noqa: BLE001
        threadpool_info = limiter = None
    n_tok = min(n_tok, spec.T)
    x = synth.act_to_f64(x_np[:n_tok])
    dy = synth.act_to_f64(dy_np[:n_tok])
    fixed, tok, reps = 0.0, 0.0, 0
    t_start = time.perf_counter()
    while reps == 0 or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        r = O.init_select(layer.dwq, spec.p, m=3)
        dW = O.materialize(r["E"], r["c"], spec.d_out, spec.d_in, 1.0)
        t1 = time.perf_counter()
        O.forward(x, dW)
        _, dc = O.backward(x, dy, r["E"], r["c"], spec.d_out, spec.d_in, 1.0, dW=dW)
        t2 = time.perf_counter()
        c2 = O.sign_update(r["c"], dc)
        O.materialize(r["E"], c2, spec.d_out, spec.d_in, 1.0)
        t3 = time.perf_counter()
        fixed += (t1 - t0) + (t3 - t2)
        tok += t2 - t1
        reps += 1
    sec = time.perf_counter() - t_start
    fixed /= reps
    tok /= reps
    step_s = fixed + tok * spec.T / n_tok
    threads = cores
    if threadpool_info is not None:
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [cores])
    del limiter
    scaled = "" if n_tok == spec.T else f", scaled to {spec.T} tokens"
    return {"value": round(spec.T / step_s, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reps} oracle step(s) on the full {spec.d_out}x{spec.d_in} layer with "
                      f"{n_tok} of {spec.T} tokens ({sec:.1f} s): init + materialize + update + "
                      f"re-materialize {fixed:.2f} s, fwd + bwd {tok:.2f} s per step{scaled}"}


if __name__ == "__main__":
    main()
