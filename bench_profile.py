"""Turn rocprofv3 output of a bench.py run into the short text summaries kept
under profiles/.

  python bench_profile.py stats KERNEL_STATS_CSV OUT_MD --title T --command C
      per-kernel call count and average / min / max duration
  python bench_profile.py traffic FETCH_CSV WRITE_CSV OUT_MD --config c2 \\
          --calib-mib 256 --command-fetch C1 --command-write C2
      HBM bytes per launch of each library kernel from two counter runs
      (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled by
      what the same counter reads for a plain fp32 copy of known size
      (bench.py --calib-copy-mib). Writes one `traffic:` line per kernel,
      tagged with the digest of the library's sources, which bench.py reads.
  python bench_profile.py counters OUT_MD CSV... --ids FWD_SPMM,BWD_SPMM --title T \\
          --intro I --command C1 --command C2 [--entries-per-wave FWD_SPMM=N,...]
      SQ counters per profiling id from separate counter passes, with ratios

The library's kernels are named by the profiling ids bench.py reports.
"""
from __future__ import annotations

import argparse
import collections
import csv
import re

import bench

# ids timed over several kernels: listed in the table, no per-launch traffic line
MULTI_KERNEL_IDS = {"GLOBAL_THRESHOLD", "CALIB_PREPARE", "CALIB_SYSTEM", "REFINE"}
# ids with no bench.py event of their own: listed in the table only
TABLE_ONLY_IDS = {"INIT_SELECT_GLOBAL", "LAYER_SPMM"}

# kernel symbol prefix -> profiling ids (spmm and fwht resolved by template arguments)
KERNEL_IDS = {
    "materialize_kernel": ["MATERIALIZE"],
    "materialize_rows_kernel": ["MATERIALIZE"],
    "dc_reduce_kernel": ["BWD_DC_REDUCE"],
    # global selection: the threshold stage
    "mag_keys_kernel": ["GLOBAL_THRESHOLD"],
    "radix_hist_kernel": ["GLOBAL_THRESHOLD"],
    "radix_pick_kernel": ["GLOBAL_THRESHOLD"],
    "row_ties_kernel": ["GLOBAL_THRESHOLD"],
    "global_budget_kernel": ["GLOBAL_THRESHOLD"],
    "gsel_init_kernel": ["GLOBAL_THRESHOLD"],
    # calibrated init and refinement
    "delta_kernel": ["CALIB_PREPARE"],
    "calib_rows_kernel": ["CALIB_PREPARE"],
    "fwht64_rows_kernel": ["CALIB_SYSTEM"],
    "transpose64_kernel": ["CALIB_SYSTEM"],
    "rhs_gather_kernel": ["CALIB_SYSTEM"],
    "refine_offsets_kernel": ["REFINE"],
    "refine_kernel": ["REFINE"],
    "fill_i32_kernel": ["REFINE"],
    # quantized base layer
    "merge_kernel": ["MERGE"],
    "qgemm_kernel": ["QGEMM"],
    "qgemm4_ring_kernel": ["QGEMM"],
}


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    n = re.sub(r"\(.*", "", n)
    return n.replace("qwha::", "").replace("void ", "")


def template_args(n: str):
    return [a.strip() for a in n[n.index("<") + 1:n.rindex(">")].split(",")]


def kernel_ids(name: str):
    n = short(name)
    if n.startswith("rows_dc_kernel<") or n.startswith("rows_dc16_kernel<"):
        return ["BWD_SPMM"]
    if n.startswith("rows_kernel<"):
        # the plain gather: forward (source z, fp32; bf16 output as in the
        # step); the quantized layer's adapter writes fp32; bench.py's
        # backward always forms dc
        a = template_args(n)
        if a[0] != "float":
            return []
        return ["FWD_SPMM"] if a[1] == "unsigned short" else ["LAYER_SPMM"]
    if n.startswith("gemm64_kernel<"):
        # A read k-major (calibration tokens): the Hessian; else dW_Q Hs
        return ["HESSIAN"] if template_args(n)[1] == "true" else ["CALIB_PREPARE"]
    if n.startswith("init_select_kernel<"):
        # the AdaAlloc instance (selection mode 0) is the one of the step
        return ["INIT_SELECT"] if template_args(n)[1] == "0" else ["INIT_SELECT_GLOBAL"]
    if n.startswith("fwht_rows_kernel<"):
        # FWHT(x) -> fp32 z (the forward's, kept for the backward); FWHT(dz) -> activations
        return ["FWD_FWHT"] if template_args(n)[2] == "float" else ["BWD_FWHT_DX"]
    for key, kids in KERNEL_IDS.items():
        if n.startswith(key):
            return kids
    return []


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    with open(a.out, "w") as f:
        f.write(f"# {a.title}\n\n")
        f.write("Command (from /tmp with TMPDIR=/tmp, one MI355X; $REPO is the repository "
                "root):\n\n```\n" + a.command + "\n```\n\n")
        f.write("| kernel | calls | avg us | min us | max us | % of traced GPU time |\n"
                "|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                    f"{float(r['Percentage']):.2f} |\n")
    print("wrote", a.out)


def per_kernel(path, counter):
    """mean counter value per dispatch, by demangled kernel name"""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc[(r["Kernel_Name"], r.get("Dispatch_Id", ""))].append(float(r["Counter_Value"]))
    by_name = collections.defaultdict(list)
    for (name, _), vals in acc.items():
        by_name[name].append(sum(vals))   # summed over dimensions / instances
    return {n: sum(v) / len(v) for n, v in by_name.items()}


def cmd_traffic(a):
    fetch = per_kernel(a.fetch_csv, "FETCH_SIZE")
    write = per_kernel(a.write_csv, "WRITE_SIZE")
    known_kib = a.calib_mib * 1024.0
    calib = [n for n in fetch if "elementwise" in n and "Mul" in n] or \
            [n for n in fetch if "elementwise" in n]
    if not calib:
        raise SystemExit("no copy kernel in the FETCH_SIZE run (bench.py --calib-copy-mib)")
    cname = max(calib, key=lambda n: fetch[n])
    f_fetch = known_kib / fetch[cname]
    f_write = known_kib / write[cname]
    lines = []
    table = []
    for name in sorted(set(fetch) & set(write)):
        kids = kernel_ids(name)
        if not kids:
            continue
        fb = fetch[name] * f_fetch * 1024.0
        wb = write[name] * f_write * 1024.0
        table.append(("/".join(kids), short(name), fetch[name], write[name], fb, wb))
        for kid in kids:
            if kid in MULTI_KERNEL_IDS or kid in TABLE_ONLY_IDS:
                continue
            lines.append(f"traffic: kernel={kid} config={a.config} bytes={int(round(fb + wb))} "
                         f"fetch={int(round(fb))} write={int(round(wb))} "
                         f"sources={bench.source_digest(kid)}")
    with open(a.out, "w") as f:
        f.write(f"# HBM traffic per launch, workload {a.config}\n\n")
        f.write("FETCH_SIZE and WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc) in two runs, "
                "each scaled by its reading for a plain fp32 copy of "
                f"{a.calib_mib} MiB read + {a.calib_mib} MiB written in the same run.\n\n")
        f.write("Commands (from /tmp with TMPDIR=/tmp, one MI355X; $REPO is the repository "
                "root):\n\n```\n" + a.command_fetch + "\n" + a.command_write + "\n```\n\n")
        f.write(f"Copy kernel `{short(cname)}`: FETCH_SIZE {fetch[cname]:.0f} KiB, WRITE_SIZE "
                f"{write[cname]:.0f} KiB for {known_kib:.0f} KiB each way; scale factors "
                f"fetch {f_fetch:.4f}, write {f_write:.4f}.\n\n")
        f.write("| id | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch MB (scaled) | "
                "write MB (scaled) |\n|---|---|---|---|---|---|\n")
        for kid, n, fk, wk, fb, wb in table:
            f.write(f"| {kid} | `{n}` | {fk:.0f} | {wk:.0f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |\n")
        f.write("\nMachine-readable lines (sources = digest of the kernel's HIP sources when "
                "the counters were taken; bench.py reports traffic only while it matches):\n\n")
        for ln in lines:
            f.write(ln + "\n")
    print("wrote", a.out)


SQ_DERIVED = [
    ("VALU busy per SIMD (4 waves x SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES)",
     lambda m: f"{100 * 4 * m['SQ_ACTIVE_INST_VALU'] / m['SQ_WAVE_CYCLES']:.0f}%"),
    ("wave lifetime spent waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)",
     lambda m: f"{100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.0f}%"),
    ("waiting on a dependency (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
     lambda m: f"{100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.0f}%"),
    ("issue slots a wave uses (all instructions / SQ_WAVE_CYCLES)",
     lambda m: f"{100 * sum(m[c] for c in ('SQ_INSTS_VALU', 'SQ_INSTS_SALU', 'SQ_INSTS_LDS', 'SQ_INSTS_VMEM_RD', 'SQ_INSTS_SMEM')) / m['SQ_WAVE_CYCLES']:.0f}%"),
    ("VALU instructions per wave", lambda m: f"{m['SQ_INSTS_VALU'] / m['SQ_WAVES']:.0f}"),
    ("SALU instructions per wave", lambda m: f"{m['SQ_INSTS_SALU'] / m['SQ_WAVES']:.0f}"),
    ("SALU per VALU instruction", lambda m: f"{m['SQ_INSTS_SALU'] / m['SQ_INSTS_VALU']:.2f}"),
    ("LDS instructions per wave", lambda m: f"{m['SQ_INSTS_LDS'] / m['SQ_WAVES']:.0f}"),
    ("global load instructions per wave", lambda m: f"{m['SQ_INSTS_VMEM_RD'] / m['SQ_WAVES']:.0f}"),
    ("LDS bank-conflict cycles / LDS active cycles",
     lambda m: f"{100 * m['SQ_LDS_BANK_CONFLICT'] / m['SQ_ACTIVE_INST_LDS']:.1f}%"),
    ("waiting on LDS (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES)",
     lambda m: f"{100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.1f}%"),
]


def cmd_counters(a):
    """SQ counters of the profiling ids in --ids, from one or more counter runs
    (each its own pass): the mean per dispatch, the launch shape and ratios."""
    ids = a.ids.split(",")
    vals = {k: collections.defaultdict(list) for k in ids}
    shape = {}
    for path in a.csvs:
        for r in csv.DictReader(open(path)):
            for kid in kernel_ids(r["Kernel_Name"]):
                if kid in vals:
                    vals[kid][r["Counter_Name"]].append(float(r["Counter_Value"]))
                    shape[kid] = (r["Grid_Size"], r["Workgroup_Size"], r["LDS_Block_Size"])
    m = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    n = {k: len(vals[k]["SQ_WAVES"]) for k in ids}
    with open(a.out, "w") as f:
        f.write(f"# {a.title}\n\n{a.intro} Each counter pass is its own run (from /tmp with "
                "TMPDIR=/tmp, one MI355X; $REPO is the repository root):\n\n```\n"
                + "\n".join(a.command) + "\n```\n\n")
        f.write("Per dispatch, mean over " + ", ".join(f"{n[k]} ({k})" for k in ids)
                + " dispatches (counter values summed over the chip; cycle counters in the SQ's "
                "own units, used only in ratios):\n\n")
        f.write("| counter | " + " | ".join(ids) + " |\n|---" + "|---" * len(ids) + "|\n")
        for c in sorted(set().union(*(m[k] for k in ids))):
            f.write(f"| {c} | " + " | ".join(f"{m[k].get(c, 0):.4g}" for k in ids) + " |\n")
        f.write("\n| launch | " + " | ".join(ids) + " |\n|---" + "|---" * len(ids) + "|\n")
        for i, lab in enumerate(("grid (threads)", "workgroup", "LDS bytes per workgroup")):
            f.write(f"| {lab} | " + " | ".join(shape[k][i] for k in ids) + " |\n")
        f.write(f"\nDerived ({a.derived_note}):\n\n| quantity | " + " | ".join(ids)
                + " |\n|---" + "|---" * len(ids) + "|\n")
        for lab, fn in SQ_DERIVED:
            f.write(f"| {lab} | " + " | ".join(fn(m[k]) for k in ids) + " |\n")
        if a.entries_per_wave:
            per = dict(kv.split("=") for kv in a.entries_per_wave.split(","))
            f.write("| VALU instructions per entry (entries a wave covers in its tile: "
                    + ", ".join(f"{k} {v}" for k, v in per.items()) + ") | "
                    + " | ".join(f"{m[k]['SQ_INSTS_VALU'] / m[k]['SQ_WAVES'] / float(per[k]):.1f}"
                                 if k in per else "" for k in ids) + " |\n")
    print("wrote", a.out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--config", required=True)
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("csvs", nargs="+")
    c.add_argument("--ids", required=True, help="profiling ids, comma-separated")
    c.add_argument("--title", required=True)
    c.add_argument("--intro", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--derived-note", default="a SIMD holds 4 of a workgroup's 16 waves; one "
                   "workgroup per CU")
    c.add_argument("--entries-per-wave", default="",
                   help="ID=entries pairs: the nonzeros one wave covers in its token tile")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
