"""Regenerate the rocprofv3 summaries under profiles/ (run from the repository
root on a machine with the GPU):

    python -m ring_allreduce_reduction_02_amd.profiles_all run DIR [ENTRY ...]
    python -m ring_allreduce_reduction_02_amd.profiles_all sum DIR [ENTRY ...]

`run` executes, for every entry, a --kernel-trace --stats run and three --pmc
runs (FETCH_SIZE; WRITE_SIZE; DRAM and L1-to-L2 request counts) of bench.py
(with --limiter a fourth: wave, VALU and wait cycles),
each in its own process under a time limit, writing under DIR, and stops at
the first failure.  `sum` turns DIR into profiles/<entry output>.md and
_pmc.json with profsum.  The headline kernels (fp32 and bf16 ring AllReduce at
8 x 67,108,864) take their trace from the default bench.py run itself, so the
average launch time in the summary is that of the command the benchmark line
comes from; every counter run replays the kernel alone (--profile-section).
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

COPY_BYTES = 1 << 30
XCHECK = "TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum TCP_TCC_READ_REQ_sum TCP_TCC_WRITE_REQ_sum"
# what the waves do (one run, 8 SQ counters and the GPU's busy clock): with
# `--limiter`, for naming what bounds a kernel below the HBM roofline
LIMITER = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_WAIT_INST_ANY "
           "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE")

# name: (trace source, kernel name substring, csrc file, profiles/ output, workload)
# The default benchmark run also launches the bf16 ring kernel once per
# gradient bucket: the headline entries time only the dispatches of their own
# grid (one work-item per 16-byte vector of a rank's M elements).
BENCH_GRID = {"ring_f32": 67108864 * 4 // 16, "ring_bf16": 67108864 * 2 // 16}
ENTRIES = {
    "ring_f32": ("bench", "k_ring_fused<1, 0, 8, 1>", "cc_kernels.hip", "ring_fused_f32_n8_m67108864",
                 "fused ring AllReduce, N=8 logical ranks, M=67108864 fp32 per rank (the benchmark's headline)"),
    "ring_bf16": ("bench", "k_ring_fused<2, 0, 8, 1>", "cc_kernels.hip", "ring_fused_bf16_n8_m67108864",
                  "fused ring AllReduce, N=8 logical ranks, M=67108864 bf16 per rank (the headline's bf16 twin)"),
    "int32_ring_rot": ("section", "k_ring_fused<0, 0, 4, 2>", "cc_kernels.hip",
                       "ring_fused_int32_n4_m1048576_rotating64",
                       "fused ring AllReduce, N=4, M=1048576 int32 per rank, 64 rotating buffer sets (2 GiB)"),
    "buckets_ring": ("section", "k_fused_seg<2, 0, 8, 0>", "cc_trees.hip", "fused_seg_bf16_n8_120_tensors",
                     "bucketed bf16 ring AllReduce, N=8, 120 tensors in 25 MiB buckets, up to 16 buckets per launch"),
    "rs_ring_n16": ("section", "k_ring_fused<1, 0, 16, 1>", "cc_kernels.hip", "ring_fused_rs_f32_n16_m33554432",
                    "fused ring ReduceScatter, N=16, M=33554432 fp32 per rank"),
    "ag_ring_n16": ("section", "k_ag_groups<4, 2>", "cc_steps.hip", "ag_groups_f32_n16_m33554432",
                    "fused AllGather (two store groups per tile), N=16, 2097152 fp32 per rank gathered to 33554432"),
    "moe_dropless": ("section", "k_copies", "cc_copy.hip", "copies_moe_dispatch_dropless_n8_t4096_h7168",
                     "MoE AllToAll(v) dispatch, N=8, 4096 tokens top-8 of 64 experts (Zipf 1.2), rows of 7168 bf16"),
    "hier_2x2x2": ("section", "k_hier_fused<1, 0>", "cc_hier.hip", "hier_fused_f32_2x2x2_m67108864",
                   "fused hierarchical AllReduce, grid 2x2x2 (N=8), M=67108864 fp32 per rank"),
    "hier_8x8": ("section", "k_hier_fused<1, 0>", "cc_hier.hip", "hier_fused_f32_8x8_m8388608",
                 "hierarchical AllReduce, grid 8x8 (N=64), M=8388608 fp32 per rank: the split form's first "
                 "launch (nested fold stored once, to the owner of the element's flat ring chunk)"),
    "hier_8x8_ag": ("section", "k_ag_groups<4, 2>", "cc_steps.hip", "ag_groups_hier_f32_8x8_m8388608",
                    "hierarchical AllReduce, grid 8x8 (N=64), M=8388608 fp32 per rank: the split form's "
                    "AllGather launch (owners' chunks to the other 63 ranks)"),
    "ring_n64": ("section", "k_ring_fused<1, 0, 0, 1>", "cc_kernels.hip", "ring_split_rs_f32_n64_m8388608",
                 "ring AllReduce, N=64, M=8388608 fp32 per rank: the split form's ReduceScatter launch "
                 "(each chunk's fold stored to its owner)"),
    "ring_n64_ag": ("section", "k_ag_groups<4, 2>", "cc_steps.hip", "ag_groups_ring_f32_n64_m8388608",
                    "ring AllReduce, N=64, M=8388608 fp32 per rank: the split form's AllGather launch "
                    "(owners' chunks to the other 63 ranks)"),
    "dbt_n8": ("section", "k_dbt_fused<1, 0, 8, true>", "cc_trees.hip", "dbt_fused_f32_n8_m67108864",
               "fused double binary tree AllReduce, N=8, M=67108864 fp32 per rank"),
    "int8_ef_f32": ("section", "k_quant_ef_fused<1, 2>", "cc_quant.hip", "quant_ef_fused_f32_n8_m67108864",
                    "fused INT8 AllReduce with error feedback, N=8, M=67108864 fp32 gradients per rank"),
    "int8_ef_bf16": ("section", "k_quant_ef_fused<2, 2>", "cc_quant.hip", "quant_ef_fused_bf16_n8_m67108864",
                     "fused INT8 AllReduce with error feedback, N=8, M=67108864 bf16 gradients per rank"),
    "int8_quant_f32": ("section", "k_quant_ef<1>", "cc_quant.hip", "quant_ef_f32_n8_m67108864",
                       "INT8 compression step with error feedback, N=8, M=67108864 fp32 gradients per rank"),
    "int8_dequant_f32": ("section", "k_dequant_reduce<1>", "cc_quant.hip", "dequant_reduce_f32_n8_m67108864",
                         "AllReduce of INT8 messages, N=8, M=67108864 elements per rank, fp32 result"),
    "moe_padded_c125": ("section", "k_copies", "cc_copy.hip", "copies_moe_dispatch_padded_c125_n8_t4096_h7168",
                        "capacity-padded MoE dispatch (C=1.25, capacity 640), N=8, 4096 tokens top-8 of 64 experts, "
                        "rows of 7168 bf16"),
}


def commands(name, d):
    src = ENTRIES[name][0]
    if src == "bench":
        trace = (f"rocprofv3 --kernel-trace --stats -f csv -d {d}/bench_trace -o k -- "
                 f"python3 bench.py --steps 20 --warmup 5")
    else:
        trace = (f"rocprofv3 --kernel-trace --stats -f csv -d {d}/{name}_trace -o k -- "
                 f"python3 bench.py --profile-section {name} --steps 20 --warmup 2")
    pmc = {tag: (f"rocprofv3 --pmc {ctr} -f csv -d {d}/{name}_{tag} -o k -- python3 bench.py --profile-section {name} "
                 f"--steps 5 --warmup 1 --copy-probe-bytes {COPY_BYTES}")
           for tag, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"), ("xcheck", XCHECK), ("limiter", LIMITER))}
    return trace, pmc


def _sh(cmd, out, limit):
    print(f"+ {cmd}", flush=True)
    with open(out, "w") as f:
        r = subprocess.run(["timeout", "-k", "10", str(limit), *cmd.split()], stdout=f, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(f"failed ({r.returncode}): {cmd}; see {out}", flush=True)
        sys.exit(r.returncode)


def run(d, names, limiter=False):
    """Every run whose output directory is not there yet (a second call
    resumes; with limiter, adds the wave-counter runs)."""
    os.makedirs(d, exist_ok=True)
    for name in names:
        trace, pmc = commands(name, d)
        tdir = "bench_trace" if ENTRIES[name][0] == "bench" else f"{name}_trace"
        if not os.path.isdir(os.path.join(d, tdir)):
            _sh(trace, os.path.join(d, f"{tdir}.out"), 900 if tdir == "bench_trace" else 300)
        for tag in ("fetch", "write", "xcheck") + (("limiter",) if limiter else ()):
            if not os.path.isdir(os.path.join(d, f"{name}_{tag}")):
                _sh(pmc[tag], os.path.join(d, f"{name}_{tag}.out"), 120)


def _alg_bytes(d, name):
    """Algorithmic bytes per launch, as the counter runs' bench.py printed it."""
    with open(os.path.join(d, f"{name}_fetch.out")) as f:
        for line in f:
            if line.startswith("{") and "alg_bytes_per_launch" in line:
                return json.loads(line)["alg_bytes_per_launch"], json.loads(line)["launches_per_call"]
    raise RuntimeError(f"no alg_bytes_per_launch in {name}_fetch.out")


def summarize(d, names):
    for name in names:
        src, kernel, csrc, out, workload = ENTRIES[name]
        trace, pmc = commands(name, d)
        alg, launches = _alg_bytes(d, name)
        note = ("the collective's definition: every input read once, every output written once"
                + ("" if launches == 1 else f"; one call is {launches} launches, bytes per call / launches"))
        tdir = f"{d}/bench_trace" if src == "bench" else f"{d}/{name}_trace"
        cmd = [sys.executable, "-m", "ring_allreduce_reduction_02_amd.profsum", "--trace", tdir,
               "--fetch", f"{d}/{name}_fetch", "--write", f"{d}/{name}_write", "--kernel", kernel,
               "--copy-bytes", str(COPY_BYTES), "--alg-bytes", str(alg), "--out", f"profiles/{out}",
               "--trace-command", trace, "--pmc-command", pmc["fetch"].replace("FETCH_SIZE", "<FETCH_SIZE|WRITE_SIZE>"),
               "--workload", workload, "--note", note, "--source", csrc]
        if name in BENCH_GRID:
            cmd += ["--grid", str(BENCH_GRID[name])]
        if os.path.isdir(f"{d}/{name}_xcheck"):
            cmd += ["--xcheck", f"{d}/{name}_xcheck", "--xcheck-command", pmc["xcheck"]]
        if os.path.isdir(f"{d}/{name}_limiter"):
            cmd += ["--limiter", f"{d}/{name}_limiter", "--limiter-command", pmc["limiter"]]
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
        print(f"profiles/{out}.md", flush=True)


def main():
    args = [a for a in sys.argv[1:] if a != "--limiter"]
    mode, d, names = args[0], args[1].rstrip("/"), args[2:] or list(ENTRIES)
    for n in names:
        if n not in ENTRIES:
            raise SystemExit(f"unknown entry {n}; known: {', '.join(ENTRIES)}")
    if mode == "run":
        run(d, names, "--limiter" in sys.argv)
    else:
        summarize(d, names)


if __name__ == "__main__":
    main()
