"""Throughput of the Walsh-Hadamard adapter hot path on one MI355X.

One step = one pass of the whole hot path over one batch, every kernel in
the library's HIP code, on torch's current stream, for every adapter of the
workload:
  init (row norms, AdaAlloc budgets, fp64 transform + in-row top-k, column
  index) -> materialize dW -> forward (FWHT(x), gather-SpMM; z = FWHT(x)/n
  kept as the saved activation) -> backward (gather-SpMM dz and dc partials
  against the saved z, FWHT(dz) -> dx, dc reduction) ->
  c += 1e-3 sign(dc) -> re-materialize dW.
value = tokens per second of that step (T / step time), inputs resident in HBM.

Workload (default --config c2): the 4096x4096 q_proj-shaped layer, 4-bit
RTN (group 128) error with 0.1% x20 outliers, budget p = 524288 (rank-64
LoRA parameter count), 8192 bf16 tokens. The further workloads (--configs,
default c3, c4, c5) are measured after it in the same run, each with its own
step, kernel table, dominant-kernel roofline and oracle baseline: the
14336x4096 up_proj layer (3-bit), the 8192x8192 layer (2-bit, 16384 tokens)
and the GQA attention block (q/o 4096x4096, k/v 1024x4096, 32768 tokens),
whose q, k and v adapters share one FWHT(x) in the forward and one
FWHT(dz_q + dz_k + dz_v) in the backward. Four copies of the inputs are
rotated so the working set exceeds the 256 MB Infinity Cache.

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
    ap.add_argument("--configs", default="c3,c4,c5",
                    help="further workloads measured after --config, each its own step "
                         "('' for none)")
    ap.add_argument("--extra-cpu-tokens", type=int, default=1024,
                    help="tokens in the oracle's sample for the further workloads")
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


# kernel ids of the profiling hook (qwha.h qwha_kernel) by the step's calls
CALL_KERNELS = {
    "init": ["INIT_SELECT"],
    "materialize": ["MATERIALIZE"],
    "fwd_z": ["FWD_SPMM"],
    "bwd_dz": ["BWD_SPMM", "BWD_DC_REDUCE"],
    "fwht_dx": ["BWD_FWHT_DX@FWHT"],   # dx = FWHT(dz)/n by qwha_fwht
    "fwht_z": ["FWD_FWHT@FWHT"],   # z = FWHT(x)/n by qwha_fwht, reported as FWD_FWHT
}
KID = dict(K, FWHT=9)


class Block:
    """The device state of one workload: its adapters (one per projection),
    grouped by the activation they read (q, k, v of the attention block read
    one x; every other layer is a group of one), with `sets` rotated copies
    of every input so the working set exceeds the Infinity Cache.

    One step = the whole hot path over one batch: for every adapter the init
    (row norms, AdaAlloc, fp64 transform + in-row top-k, column index) and
    the materialisation of dW; per group the forward (one z = FWHT(x)/n for
    the group, kept, then each adapter's gather-SpMM) and the backward (each
    adapter's dz and dc against the kept z; one transform of the summed dz for
    a shared group); then every adapter's c += 1e-3 sign(dc) and
    re-materialisation. The transforms (x -> z, dz -> dx) and the first
    materialisations run on a second stream beside the inits, the forward
    and the updates, ordered by events."""

    def __init__(self, cfg, nsets, dev, hip):
        import numpy as np
        import torch
        import synth
        from quantization_aware_sparse_amd import lib
        self.cfg = cfg
        self.specs = synth.config_specs(cfg)
        self.hip = hip
        self.dev = dev
        t0 = time.perf_counter()
        self.layers = [synth.make_layer(sp, seed=0) for sp in self.specs]
        streams = {}
        self.host_x, self.host_dy = [], []
        for sp in self.specs:
            xs = synth.C5_X_STREAM.get(sp.name) if cfg == "c5" else None
            x, dy = synth.make_activations(sp, seed=0, x_stream=xs)
            key = xs if xs is not None else sp.name
            if key not in streams:
                streams[key] = (len(streams), x)
            self.host_x.append(streams[key][0])
            self.host_dy.append(dy)
        self.x_host = [None] * len(streams)
        for key, (g, x) in streams.items():
            self.x_host[g] = x
        self.gen_s = time.perf_counter() - t0

        def up(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        sp0 = self.specs[0]
        self.T = sp0.T
        self.act = sp0.act
        self.act_code = 1 if sp0.act == "bf16" else 0
        adt = torch.bfloat16 if sp0.act == "bf16" else torch.float32
        i32 = dict(dtype=torch.int32, device=dev)
        self.groups = []
        for g, x in enumerate(self.x_host):
            xd = up(x)
            members = [i for i, gi in enumerate(self.host_x) if gi == g]
            d_in = x.shape[1]
            grp = dict(members=members, d_in=d_in,
                       x=[xd] + [xd.clone() for _ in range(nsets - 1)],
                       z=torch.empty((self.T, d_in), dtype=torch.float32, device=dev),
                       dx=torch.empty((self.T, d_in), dtype=adt, device=dev))
            grp["dz"] = torch.empty((self.T, d_in), dtype=torch.float32, device=dev)
            self.groups.append(grp)
        self.ads = []
        for i, (sp, L) in enumerate(zip(self.specs, self.layers)):
            d_out, d_in, p, T = sp.d_out, sp.d_in, sp.p, sp.T
            dwq = up(L.dwq)
            dy = up(self.host_dy[i])
            a = dict(spec=sp, name=sp.name,
                     dwq=[dwq] + [dwq.clone() for _ in range(nsets - 1)],
                     dy=[dy] + [dy.clone() for _ in range(nsets - 1)],
                     row_ptr=torch.empty(d_out + 1, **i32), E=torch.empty((p, 2), **i32),
                     c=torch.empty(p, dtype=torch.float32, device=dev),
                     col_ptr=torch.empty(d_in + 1, **i32), perm=torch.empty(p, **i32),
                     dW=torch.empty((d_out, d_in), dtype=torch.float32, device=dev),
                     y=torch.empty((T, d_out), dtype=adt, device=dev),
                     dc=torch.empty(p, dtype=torch.float32, device=dev))
            a["ws_i"] = torch.empty(lib.qwha_init_workspace_bytes(d_out, d_in),
                                    dtype=torch.uint8, device=dev)
            a["ws_f"] = torch.empty(lib.qwha_fwd_workspace_bytes(T, d_in, d_out, p),
                                    dtype=torch.uint8, device=dev)
            a["ws_b"] = torch.empty(lib.qwha_bwd_workspace_bytes(T, d_in, d_out, p),
                                    dtype=torch.uint8, device=dev)
            a["ev"] = {k: (hip.create(), hip.create()) for k in KID}
            a["times"] = {k: [] for k in KID}
            self.ads.append(a)
        self.nsets = nsets
        self.main = torch.cuda.current_stream()
        self.stream = self.main.cuda_stream
        # a second stream (default priority) for the work that does not wait
        # for the init: z = FWHT(x)/n, and the first materialisation of dW
        self.side = torch.cuda.Stream(device=dev)
        self.ev_z, self.ev_init, self.ev_mat, self.ev_dz = (torch.cuda.Event() for _ in range(4))

    def _arm(self, a, call, record):
        from quantization_aware_sparse_amd import check, lib
        if not record:
            return
        for k in CALL_KERNELS[call]:
            label, _, kid = k.partition("@")
            check(lib.qwha_profile_next(KID[kid or label], a["ev"][label][0], a["ev"][label][1]),
                  "profile")
            a["armed"].append(label)

    def step(self, s, record=False):
        from quantization_aware_sparse_amd import check, lib
        st, A = self.stream, self.act_code
        # Timed steps overlap the two streams. Profiled steps (record) issue
        # everything on the main stream, so that each kernel's recorded time
        # is its own and not shared with a kernel running beside it.
        overlap = not record
        side = self.side.cuda_stream if overlap else st
        T = self.T
        for a in self.ads:
            a["armed"] = []

        def cross(ev, src, dst):   # dst waits for src's work so far
            if overlap:
                ev.record(src)
                dst.wait_event(ev)

        # side stream, once the previous step is done with z and dW: every
        # group's z = FWHT(x)/n (it needs no init, so it runs beside it)
        if overlap:
            self.side.wait_stream(self.main)
        for g in self.groups:
            x = g["x"][s % self.nsets]
            self._arm(self.ads[g["members"][0]], "fwht_z", record)
            d_in = g["d_in"]
            b = d_in & -d_in
            check(lib.qwha_fwht(x.data_ptr(), A, g["z"].data_ptr(), 0, T * (d_in // b), b,
                                1.0 / b, side), "fwht z")
        if overlap:
            self.ev_z.record(self.side)
        # main stream: each init; its dW materialised on the side stream
        for a in self.ads:
            sp = a["spec"]
            self._arm(a, "init", record)
            check(lib.qwha_init_select(a["dwq"][s % self.nsets].data_ptr(), sp.d_out, sp.d_in,
                                       sp.p, 3, 1.0, a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                       a["c"].data_ptr(), a["col_ptr"].data_ptr(),
                                       a["perm"].data_ptr(), a["ws_i"].data_ptr(),
                                       a["ws_i"].numel(), st), "init")
            cross(self.ev_init, self.main, self.side)
            self._arm(a, "materialize", record)
            check(lib.qwha_materialize(a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                       a["c"].data_ptr(), sp.d_out, sp.d_in, sp.p, 1.0, 0,
                                       a["dW"].data_ptr(), 0, side), "materialize")
        if overlap:
            self.ev_mat.record(self.side)
            self.main.wait_event(self.ev_z)
        for g in self.groups:
            for i in g["members"]:
                a, sp = self.ads[i], self.ads[i]["spec"]
                self._arm(a, "fwd_z", record)
                check(lib.qwha_fwd_z(g["z"].data_ptr(), A, T, sp.d_in, sp.d_out, sp.p,
                                     a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                     a["c"].data_ptr(), 1.0, a["y"].data_ptr(), 0,
                                     a["ws_f"].data_ptr(), a["ws_f"].numel(), st), "fwd_z")
        # backward: dz (summed over a shared group) and dc on the main stream;
        # dx = FWHT(dz)/n on the side stream, beside the updates, which need
        # only dc
        for g in self.groups:
            for n, i in enumerate(g["members"]):
                a, sp = self.ads[i], self.ads[i]["spec"]
                self._arm(a, "bwd_dz", record)
                check(lib.qwha_bwd_dz(g["z"].data_ptr(), a["dy"][s % self.nsets].data_ptr(), A,
                                      T, sp.d_in, sp.d_out, sp.p, a["E"].data_ptr(),
                                      a["c"].data_ptr(), a["col_ptr"].data_ptr(),
                                      a["perm"].data_ptr(), 1.0, g["dz"].data_ptr(),
                                      int(n > 0), a["dc"].data_ptr(), a["ws_b"].data_ptr(),
                                      a["ws_b"].numel(), st), "bwd_dz")
            cross(self.ev_dz, self.main, self.side)
            a0 = self.ads[g["members"][0]]
            self._arm(a0, "fwht_dx", record)
            d_in = g["d_in"]
            b = d_in & -d_in
            check(lib.qwha_fwht(g["dz"].data_ptr(), 0, g["dx"].data_ptr(), A, T * (d_in // b), b,
                                1.0 / b, side), "fwht dx")
        # the update changes c and the re-materialisation overwrites dW: both
        # after the side stream's first materialisation
        if overlap:
            self.main.wait_event(self.ev_mat)
        for a in self.ads:
            sp = a["spec"]
            check(lib.qwha_sign_update(a["c"].data_ptr(), a["dc"].data_ptr(), sp.p, 1e-3, st),
                  "update")
            check(lib.qwha_materialize(a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                       a["c"].data_ptr(), sp.d_out, sp.d_in, sp.p, 1.0, 0,
                                       a["dW"].data_ptr(), 0, st), "rematerialize")

    def build_plans(self):
        """The SpMM streams of every adapter from its current E (after an init)."""
        from quantization_aware_sparse_amd import check, lib
        import torch
        for a in self.ads:
            sp = a["spec"]
            nb = lib.qwha_plan_bytes(sp.d_in, sp.d_out, sp.p)
            a["plan"] = torch.empty(nb, dtype=torch.uint8, device=self.dev)
            check(lib.qwha_plan_build(a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                      a["col_ptr"].data_ptr(), a["perm"].data_ptr(), sp.d_in,
                                      sp.d_out, sp.p, self.act_code, a["plan"].data_ptr(), nb,
                                      self.stream),
                  "plan")

    def train_step(self, s):
        """One fine-tuning step once the init has run (E frozen, plans built):
        per group the forward (one kept z) and backward (dz summed over a
        shared group, one transform), then every adapter's sign update and
        re-materialisation of dW."""
        from quantization_aware_sparse_amd import check, lib
        st, A, T = self.stream, self.act_code, self.T
        for g in self.groups:
            x = g["x"][s % self.nsets]
            for n, i in enumerate(g["members"]):
                a, sp = self.ads[i], self.ads[i]["spec"]
                check(lib.qwha_fwd_plan(x.data_ptr() if n == 0 else None,
                                        None if n == 0 else g["z"].data_ptr(), A, T, sp.d_in,
                                        sp.d_out, sp.p, a["plan"].data_ptr(), a["c"].data_ptr(),
                                        1.0, a["y"].data_ptr(), 0,
                                        g["z"].data_ptr() if n == 0 else None,
                                        a["ws_f"].data_ptr(), a["ws_f"].numel(), st), "fwd_plan")
        for g in self.groups:
            shared = len(g["members"]) > 1
            for n, i in enumerate(g["members"]):
                a, sp = self.ads[i], self.ads[i]["spec"]
                check(lib.qwha_bwd_plan(g["z"].data_ptr(), a["dy"][s % self.nsets].data_ptr(), A,
                                        T, sp.d_in, sp.d_out, sp.p, a["plan"].data_ptr(),
                                        a["c"].data_ptr(), 1.0,
                                        None if shared else g["dx"].data_ptr(), 0,
                                        g["dz"].data_ptr() if shared else None, int(n > 0),
                                        a["dc"].data_ptr(), a["ws_b"].data_ptr(),
                                        a["ws_b"].numel(), st), "bwd_plan")
            if shared:
                d_in = g["d_in"]
                b = d_in & -d_in
                check(lib.qwha_fwht(g["dz"].data_ptr(), 0, g["dx"].data_ptr(), A,
                                    T * (d_in // b), b, 1.0 / b, st), "fwht dx")
        for a in self.ads:
            sp = a["spec"]
            check(lib.qwha_sign_update(a["c"].data_ptr(), a["dc"].data_ptr(), sp.p, 1e-3, st),
                  "update")
            check(lib.qwha_materialize(a["row_ptr"].data_ptr(), a["E"].data_ptr(),
                                       a["c"].data_ptr(), sp.d_out, sp.d_in, sp.p, 1.0, 0,
                                       a["dW"].data_ptr(), 0, st), "rematerialize")

    def read_times(self):
        for a in self.ads:
            for k in a["armed"]:
                a["times"][k].append(self.hip.elapsed_ms(*a["ev"][k]))


def kernel_rates(sp, esz, times):
    """Per kernel: average launch time and the achieved rate against its roof
    (algorithmic bytes or flops per launch; SURVEY-style counts: each
    activation once, E / c once, dW_Q once)."""
    import numpy as np
    d_out, d_in, p, T = sp.d_out, sp.d_in, sp.p, sp.T
    nbytes = {
        "FWD_FWHT": T * d_in * (esz + 4),
        "BWD_FWHT_DX": T * d_in * (4 + esz),
        "FWHT": T * d_in * (4 + esz),
        "INIT_SELECT": d_out * d_in * 4 + p * 12 + (d_out + 1) * 4,
        "MATERIALIZE": p * 12 + (d_out + 1) * 4 + d_out * d_in * 4,
    }
    flops = {"FWD_SPMM": 2.0 * T * p, "BWD_SPMM": 4.0 * T * p}
    kern = {}
    for k, v in times.items():
        if not v:
            continue
        us = 1e3 * float(np.mean(v))
        if k in flops:
            a = flops[k] / (us * 1e-6) / 1e12
            kern[k] = dict(avg_us=round(us, 2), bound="alu", achieved=round(a, 3),
                           unit="TFLOP/s", peak=FP32_VECTOR_PEAK_TFLOPS,
                           frac=round(a / FP32_VECTOR_PEAK_TFLOPS, 4))
        elif k in nbytes:
            a = nbytes[k] / (us * 1e-6) / 1e9
            kern[k] = dict(avg_us=round(us, 2), bound="hbm", achieved=round(a, 1), unit="GB/s",
                           peak=HBM_PEAK_GBS, frac=round(a / HBM_PEAK_GBS, 4))
        else:
            kern[k] = dict(avg_us=round(us, 2))
    return kern


def measure(block, steps, warmup, config_name):
    """Warm up, time `steps` profiled steps (per-kernel HIP events, one host
    wait per step) and then `steps` clean steps (no host waits): the clean
    steps give the throughput."""
    import torch
    for s in range(warmup):
        block.step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        block.step(s, True)
        torch.cuda.synchronize()     # the next step re-arms the same events
        block.read_times()
    wall = time.perf_counter() - t0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(steps):
        block.step(s, False)
    torch.cuda.synchronize()
    wall_clean = time.perf_counter() - t1
    ms_step = 1e3 * wall_clean / steps
    esz = 2 if block.act == "bf16" else 4
    per = {a["name"]: kernel_rates(a["spec"], esz, a["times"]) for a in block.ads}
    # the dominant kernel: the longest launch of any adapter
    best = None
    for name, kern in per.items():
        for k, v in kern.items():
            if best is None or v["avg_us"] > best[2]["avg_us"]:
                best = (name, k, v)
    name, k, v = best
    roof = {kk: vv for kk, vv in v.items() if kk != "avg_us"}
    roof["kernel"] = k if len(per) == 1 else f"{k} ({name})"
    roof["avg_us"] = v["avg_us"]
    roof["traffic"] = measured_traffic(k, config_name) if len(per) == 1 else None
    return dict(value=round(block.T / (ms_step / 1e3), 1), ms_per_step=round(ms_step, 4),
                profiled_steps_ms=round(1e3 * wall / steps, 4), roofline=roof,
                kernels=per[block.ads[0]["name"]] if len(per) == 1 else per)


def measure_train(block, steps, warmup):
    """The fine-tuning step after a one-time init (plans built once): what a
    training loop repeats. Reported beside the whole-path step, not as it."""
    import torch
    block.step(0, False)
    block.build_plans()
    for s in range(warmup):
        block.train_step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        block.train_step(s)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    return dict(what="fwd + bwd + sign update + re-materialize per step after one init, "
                     "SpMM streams planned once from E (values gathered from c per call)",
                tokens_per_s=round(block.T / (ms / 1e3), 1), ms_per_step=round(ms, 4))


def workload_text(block):
    sps = block.specs
    if len(sps) == 1:
        sp = sps[0]
        return (f"{sp.name}: {sp.d_out}x{sp.d_in} layer, {sp.bits}-bit RTN g{sp.group} error "
                f"with {sp.outlier_frac:.1%} x{sp.outlier_mult:g} outliers, p={sp.p}, "
                f"{sp.T} {sp.act} tokens; step = init + materialize + fwd + bwd + sign update "
                "+ re-materialize")
    parts = ", ".join(f"{sp.name.split('.')[-1]} {sp.d_out}x{sp.d_in} p={sp.p}" for sp in sps)
    return (f"{block.cfg}: GQA attention block ({parts}), {sps[0].bits}-bit RTN "
            f"g{sps[0].group}, {sps[0].T} {sps[0].act} tokens (16 x 2048); step = for all four "
            "adapters init + materialize + fwd + bwd + sign update + re-materialize, q/k/v "
            "sharing one FWHT(x) and one FWHT(dz_q + dz_k + dz_v)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in the design notes, not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantization_aware_sparse_amd as q  # noqa: F401  (fails loudly without the library)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    hip = HipEvents()

    block = Block(args.config, args.sets, dev, hip)
    spec = block.specs[0]
    if args.calib_copy_mib > 0:
        for s in range(args.warmup):
            block.step(s, False)
        torch.cuda.synchronize()
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b
    print(f"# {args.config}: inputs ready; warmup {args.warmup}, timing {args.steps} steps",
          file=sys.stderr, flush=True)
    m = measure(block, args.steps, args.warmup, args.config)
    kern = m["kernels"]
    out = {
        "metric": "adapter fwd+bwd tokens/s per layer; FWHT/gather achieved HBM GB/s vs peak",
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": block.act,
        "data": "synthetic",
        "config": {
            "workload": workload_text(block),
            "d_out": spec.d_out, "d_in": spec.d_in, "p": spec.p, "tokens": spec.T,
            "act": spec.act, "math": "f32 (fp64 init transform)",
            "input_sets_rotated": args.sets,
        },
        "roofline": m["roofline"],
        "kernels": kern,
        "profiled_steps_ms": m["profiled_steps_ms"],
        "input_gen_s": round(block.gen_s, 2),
    }
    if len(block.ads) == 1:
        fb = ("FWD_FWHT", "FWD_SPMM", "BWD_SPMM", "BWD_FWHT_DX", "BWD_DC_REDUCE")
        fwd_bwd_us = sum(kern[k]["avg_us"] for k in fb if k in kern)
        out["fwd_bwd_kernels_us"] = round(fwd_bwd_us, 2)
        out["fwd_bwd_tokens_per_s"] = round(spec.T / (fwd_bwd_us * 1e-6), 1)

    a0 = block.ads[0]
    sets = [(a0["dwq"][s], block.groups[0]["x"][s], a0["dy"][s]) for s in range(args.sets)]
    stream = block.stream
    if args.variant_reps > 0 and len(block.ads) == 1:
        out["init_variants"] = init_variants(args.variant_reps, sets,
                                             (spec.d_out, spec.d_in, spec.p),
                                             (a0["row_ptr"], a0["E"], a0["c"], a0["col_ptr"],
                                              a0["perm"]), a0["ws_i"], stream, hip)
    if args.base_reps > 0 and len(block.ads) == 1:
        out["base_layer"] = base_layer_measure(args.base_reps, spec, block.layers[0], sets,
                                               (a0["row_ptr"], a0["E"], a0["c"]), stream, hip)
    if args.refine_tokens > 0 and args.refine_reps > 0 and len(block.ads) == 1:
        out["refine"] = refine_measure(args.refine_tokens, args.refine_reps, spec, sets[0][0],
                                       stream, hip)
    out["train_step"] = measure_train(block, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(block, args.cpu_tokens or spec.T)

    # the other workloads of the configuration list, each its own step
    extra = [c for c in args.configs.split(",") if c and c != args.config]
    if extra:
        del block, sets, a0
        torch.cuda.empty_cache()
        out["configs"] = {}
        for cfg in extra:
            blk = Block(cfg, args.sets, dev, hip)
            print(f"# {cfg}: inputs ready; warmup {args.warmup}, timing {args.steps} steps",
                  file=sys.stderr, flush=True)
            mm = measure(blk, args.steps, args.warmup, cfg)
            entry = dict(workload=workload_text(blk), unit="tokens/s", value=mm["value"],
                         ms_per_step=mm["ms_per_step"], dtype=blk.act, roofline=mm["roofline"],
                         kernels=mm["kernels"], input_gen_s=round(blk.gen_s, 2),
                         train_step=measure_train(blk, args.steps, args.warmup))
            if not args.no_cpu_baseline:
                entry["cpu_baseline"] = cpu_baseline(blk, min(args.extra_cpu_tokens, blk.T),
                                                     min_seconds=1.0)
            out["configs"][cfg] = entry
            del blk
            torch.cuda.empty_cache()
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
    "BWD_FWHT_DX": ["fwht.hip", "fwht_core.h"], "FWHT": ["fwht.hip", "fwht_core.h"],
    "FWD_SPMM": ["spmm.hip"],
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


def cpu_baseline(block, n_tok, min_seconds=10.0):
    """The fp64 oracle (as it stands) on the host cores: whole steps of the
    same path for every adapter of the workload (init, materialize, fwd, bwd,
    update, re-materialize) on the full layers with n_tok of the workload's
    tokens, repeated until at least min_seconds have passed. With n_tok < T
    the fwd+bwd share is scaled linearly to T tokens."""
    import oracle as O
    import synth
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # noqa: BLE001
        threadpool_info = limiter = None
    T = block.T
    n_tok = min(n_tok, T)
    xs = [synth.act_to_f64(x[:n_tok]) for x in block.x_host]
    dys = [synth.act_to_f64(dy[:n_tok]) for dy in block.host_dy]
    fixed, tok, reps = 0.0, 0.0, 0
    t_start = time.perf_counter()
    while reps == 0 or time.perf_counter() - t_start < min_seconds:
        for i, (sp, L) in enumerate(zip(block.specs, block.layers)):
            x, dy = xs[block.host_x[i]], dys[i]
            t0 = time.perf_counter()
            r = O.init_select(L.dwq, sp.p, m=3)
            dW = O.materialize(r["E"], r["c"], sp.d_out, sp.d_in, 1.0)
            t1 = time.perf_counter()
            O.forward(x, dW)
            _, dc = O.backward(x, dy, r["E"], r["c"], sp.d_out, sp.d_in, 1.0, dW=dW)
            t2 = time.perf_counter()
            c2 = O.sign_update(r["c"], dc)
            O.materialize(r["E"], c2, sp.d_out, sp.d_in, 1.0)
            t3 = time.perf_counter()
            fixed += (t1 - t0) + (t3 - t2)
            tok += t2 - t1
        reps += 1
    sec = time.perf_counter() - t_start
    fixed /= reps
    tok /= reps
    step_s = fixed + tok * T / n_tok
    threads = cores
    if threadpool_info is not None:
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [cores])
    del limiter
    scaled = "" if n_tok == T else f", scaled to {T} tokens"
    what = (f"the full {block.specs[0].d_out}x{block.specs[0].d_in} layer"
            if len(block.specs) == 1 else f"all {len(block.specs)} full layers")
    return {"value": round(T / step_s, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reps} oracle step(s) on {what} with {n_tok} of {T} tokens "
                      f"({sec:.1f} s): init + materialize + update + re-materialize "
                      f"{fixed:.2f} s, fwd + bwd {tok:.2f} s per step{scaled}"}


if __name__ == "__main__":
    main()
