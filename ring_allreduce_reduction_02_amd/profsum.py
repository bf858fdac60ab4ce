"""Summarize rocprofv3 CSV output for one kernel into a short text record.

Reads a --kernel-trace --stats run (<name>_kernel_stats.csv) and two --pmc runs
(FETCH_SIZE, WRITE_SIZE; <name>_counter_collection.csv) of the same command.
The counters are scaled by what they read for a plain device copy of known
size that ran in the same process (the copy-probe kernel), because on this
part FETCH_SIZE under-reports by a constant factor.

    python -m ring_allreduce_reduction_02_amd.profsum \\
        --trace rocprof/prof_trace --fetch rocprof/prof_fetch --write rocprof/prof_write \\
        --kernel "k_ring_fused<1, 0, 8>" --copy-bytes 1073741824 --alg-bytes 4294967296 \\
        --out profiles/ring_fused_f32_n8_m67108864 --command "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _one(path_glob: str) -> str:
    hits = sorted(glob.glob(path_glob, recursive=True))
    if not hits:
        raise FileNotFoundError(path_glob)
    return hits[0]


def counter_means(run_dir: str, counter: str):
    rows = list(csv.DictReader(open(_one(os.path.join(run_dir, "**", "*counter_collection.csv")))))
    agg = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in agg.items()}


def pick(means, needle):
    for k, v in means.items():
        if needle in k:
            return k, v
    raise KeyError(needle)


def kernel_stats(trace_dir: str, needle: str):
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    for r in rows:
        if needle in r["Name"]:
            return r
    raise KeyError(needle)


def kernel_stats_of_grid(trace_dir: str, needle: str, grid: int):
    """Stats of the dispatches of the kernel whose grid holds `grid`
    work-items (x), from the per-dispatch trace: a run that launches the
    kernel at several sizes then averages only the launches of one size."""
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    mine = [r for r in rows if needle in r["Kernel_Name"]]
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in mine if int(r["Grid_Size_X"]) == grid]
    if not durs:
        raise KeyError(f"{needle} with a grid of {grid}")
    return {"Calls": len(durs), "AverageNs": sum(durs) / len(durs), "MinNs": min(durs), "MaxNs": max(durs),
            "other_calls": len(mine) - len(durs)}


# The files a kernel's code comes from, besides its own source file: what the
# kernel sources share, and the launch interface.
SHARED_SOURCES = ("cc_device.h", "cc_launch.h")


def kernel_sources(source: str):
    """The csrc files whose text decides a kernel defined in `source`."""
    return [source, *SHARED_SOURCES]


def sources_hash(names) -> str:
    """sha256 (first 16 hex digits) of the named csrc files, in order: the
    counters recorded for a kernel stay valid while this is unchanged."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def xcheck_bytes(run_dir: str, kernel: str, copy_bytes: int):
    """A second counter family: DRAM request counts at the L2 (TCC_EA0_*) and
    L1-to-L2 request counts (TCP_TCC_*), each turned into bytes by what the
    same counter reads for the plain copy of copy_bytes (which reads and
    writes copy_bytes once)."""
    rows = list(csv.DictReader(open(_one(os.path.join(run_dir, "**", "*counter_collection.csv")))))
    out = {}
    for name in sorted({r["Counter_Name"] for r in rows}):
        m = counter_means(run_dir, name)
        _, (kv, _) = pick(m, kernel)
        _, (cv, _) = pick(m, COPY_KERNEL)
        out[name] = {"kernel_per_dispatch": kv, "copy_per_dispatch": cv,
                     "bytes": kv * copy_bytes / cv if cv else None}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--xcheck", default="", help="a --pmc run of DRAM / L2 request counters")
    ap.add_argument("--kernel", required=True, help="substring of the kernel name")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--alg-bytes", type=int, required=True, help="algorithmic bytes per launch")
    ap.add_argument("--out", required=True, help="output path without extension")
    ap.add_argument("--trace-command", required=True)
    ap.add_argument("--pmc-command", required=True)
    ap.add_argument("--xcheck-command", default="")
    ap.add_argument("--limiter", default="", help="a --pmc run of wave / VALU / wait counters")
    ap.add_argument("--limiter-command", default="")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--note", default="", help="how the algorithmic bytes per launch are counted")
    ap.add_argument("--source", default="cc_kernels.hip", help="the csrc file that defines the kernel")
    ap.add_argument("--grid", type=int, default=0,
                    help="time only the dispatches of this many work-items (x) (0: every dispatch of the kernel)")
    args = ap.parse_args()

    st = kernel_stats_of_grid(args.trace, args.kernel, args.grid) if args.grid else kernel_stats(args.trace, args.kernel)
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    kname, (f_kib, f_n) = pick(fetch, args.kernel)
    _, (w_kib, w_n) = pick(write, args.kernel)
    _, (cf_kib, _) = pick(fetch, COPY_KERNEL)
    _, (cw_kib, _) = pick(write, COPY_KERNEL)
    fetch_scale = args.copy_bytes / (cf_kib * 1024.0)
    write_scale = args.copy_bytes / (cw_kib * 1024.0)
    traffic = f_kib * 1024.0 * fetch_scale + w_kib * 1024.0 * write_scale
    avg_ns = float(st["AverageNs"])
    xc = xcheck_bytes(args.xcheck, args.kernel, args.copy_bytes) if args.xcheck else {}
    lim = limiter_counters(args.limiter, args.kernel) if args.limiter else {}
    rec = {
        "kernel": kname,
        "workload": args.workload,
        "kernel_sources": kernel_sources(args.source),
        "kernel_source_sha256_16": sources_hash(kernel_sources(args.source)),
        "calls": int(st["Calls"]),
        "grid_size_x": args.grid or None,
        "calls_at_other_grids": st.get("other_calls", 0),
        "avg_ns": avg_ns,
        "min_ns": float(st["MinNs"]),
        "max_ns": float(st["MaxNs"]),
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "fetch_dispatches": f_n,
        "write_dispatches": w_n,
        "copy_probe_bytes": args.copy_bytes,
        "copy_fetch_kib": cf_kib,
        "copy_write_kib": cw_kib,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": args.alg_bytes,
        "algorithmic_bytes_note": args.note,
        "traffic_over_algorithmic": traffic / args.alg_bytes,
        "achieved_GBps_from_trace": args.alg_bytes / avg_ns,
        "xcheck": xc,
        "limiter": lim,
        "trace_command": args.trace_command,
        "pmc_command": args.pmc_command,
        "xcheck_command": args.xcheck_command,
        "limiter_command": args.limiter_command,
    }
    with open(args.out + "_pmc.json", "w") as f:
        json.dump(rec, f, indent=1)
    with open(args.out + ".md", "w") as f:
        f.write(f"# {args.workload}\n\n")
        f.write(f"Kernel: `{kname}`  (sources {', '.join(rec['kernel_sources'])}: sha256/16 "
                f"`{rec['kernel_source_sha256_16']}`)\n\n")
        if args.note:
            f.write(f"Algorithmic bytes per launch: {args.alg_bytes} ({args.note}).\n\n")
        f.write("## rocprofv3 --kernel-trace --stats\n\n")
        f.write(f"Command: `{args.trace_command}`\n\n")
        if args.grid:
            f.write(f"Only the dispatches with a grid of {args.grid} work-items are timed; the run also launches the "
                    f"kernel {rec['calls_at_other_grids']} times at other sizes.\n\n")
        f.write("| calls | avg us | min us | max us | algorithmic GB | GB/s at avg |\n|---|---|---|---|---|---|\n")
        f.write(f"| {rec['calls']} | {avg_ns / 1e3:.2f} | {rec['min_ns'] / 1e3:.2f} | {rec['max_ns'] / 1e3:.2f} | "
                f"{args.alg_bytes / 1e9:.3f} | {rec['achieved_GBps_from_trace']:.1f} |\n\n")
        f.write("## rocprofv3 --pmc (one counter per run)\n\n")
        f.write(f"Command (run once with FETCH_SIZE, once with WRITE_SIZE): `{args.pmc_command}`\n\n")
        f.write("| counter | kernel KiB/dispatch | plain copy of "
                f"{args.copy_bytes} B reads KiB | scale | kernel bytes |\n|---|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {f_kib:.1f} | {cf_kib:.1f} | {fetch_scale:.4f} | {f_kib * 1024 * fetch_scale:.4e} |\n")
        f.write(f"| WRITE_SIZE | {w_kib:.1f} | {cw_kib:.1f} | {write_scale:.4f} | {w_kib * 1024 * write_scale:.4e} |\n\n")
        f.write(f"HBM traffic per launch {traffic:.4e} B = {rec['traffic_over_algorithmic']:.4f} x the algorithmic "
                f"{args.alg_bytes} B.\n")
        if xc:
            f.write("\n## Cross-check: request counters (one --pmc run)\n\n")
            f.write(f"Command: `{args.xcheck_command}`\n\n")
            f.write("Each counter is scaled by what it reads for the same plain copy (which reads and writes "
                    f"{args.copy_bytes} B once).\n\n")
            f.write("| counter | kernel per dispatch | copy per dispatch | kernel bytes | / algorithmic |\n"
                    "|---|---|---|---|---|\n")
            for name, v in xc.items():
                b = v["bytes"]
                f.write(f"| {name} | {v['kernel_per_dispatch']:.4e} | {v['copy_per_dispatch']:.4e} | "
                        f"{b:.4e} | {b / args.alg_bytes:.4f} |\n")
            for fam, tag in (("TCC_EA0_", "DRAM requests"), ("TCP_TCC_", "L1-to-L2 requests")):
                r_ = [v["bytes"] for k, v in xc.items() if k.startswith(fam) and ("RDREQ" in k or "READ" in k)]
                w_ = [v["bytes"] for k, v in xc.items() if k.startswith(fam) and ("WRREQ" in k or "WRITE" in k)]
                if r_ and w_:
                    f.write(f"\n{tag}: read + write {r_[0] + w_[0]:.4e} B = "
                            f"{(r_[0] + w_[0]) / args.alg_bytes:.4f} x algorithmic.\n")
        if lim:
            f.write("\n## What the waves do (one --pmc run)\n\n")
            f.write(f"Command: `{args.limiter_command}`\n\n")
            f.write("| counter | per dispatch |\n|---|---|\n")
            for name, v in lim["raw"].items():
                f.write(f"| {name} | {v:.4e} |\n")
            f.write("\n| derived | value |\n|---|---|\n")
            for name, v in lim["derived"].items():
                f.write(f"| {name} | {v:.4f} |\n")
    print(json.dumps(rec, indent=1))


XCDS = 8


def limiter_counters(run_dir: str, kernel: str):
    """Per-dispatch wave counters of the kernel and the ratios read from them:
    the share of the waves' cycles spent issuing VALU instructions, and spent
    waiting for an operand (a load in flight, mostly), and the VALU busy share
    of the SIMDs (SQ_ACTIVE_INST_VALU counts per wave in 4-cycle units; 1024
    SIMDs; GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs: 1.18e7 for a
    665.7 us launch is 8 x 2.2 GHz)."""
    rows = list(csv.DictReader(open(_one(os.path.join(run_dir, "**", "*counter_collection.csv")))))
    raw = {}
    for name in sorted({r["Counter_Name"] for r in rows}):
        _, (v, _) = pick(counter_means(run_dir, name), kernel)
        raw[name] = v
    der = {}
    if raw.get("SQ_WAVE_CYCLES"):
        der["valu_cycles_over_wave_cycles"] = raw.get("SQ_ACTIVE_INST_VALU", 0.0) / raw["SQ_WAVE_CYCLES"]
        der["wait_any_over_wave_cycles"] = raw.get("SQ_WAIT_INST_ANY", 0.0) / raw["SQ_WAVE_CYCLES"]
    if raw.get("GRBM_GUI_ACTIVE"):
        der["valu_busy_of_simds"] = raw.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / 1024 / (raw["GRBM_GUI_ACTIVE"] / XCDS)
    if raw.get("SQ_WAVES"):
        der["valu_insts_per_wave"] = raw.get("SQ_INSTS_VALU", 0.0) / raw["SQ_WAVES"]
        der["vmem_rd_insts_per_wave"] = raw.get("SQ_INSTS_VMEM_RD", 0.0) / raw["SQ_WAVES"]
        der["trans_f32_insts_per_wave"] = raw.get("SQ_INSTS_VALU_TRANS_F32", 0.0) / raw["SQ_WAVES"]
    return {"raw": raw, "derived": der}


if __name__ == "__main__":
    main()
