#!/usr/bin/env python
"""Benchmark of the ring AllReduce on one MI355X.

Headline workload: ring AllReduce SUM of synthetic gradients, N = 8 logical
ranks, M = 67,108,864 fp32 elements per rank (256 MiB each), Gaussian values
with sigma = 1e-3, rank rows 256 MiB + 256 KiB apart (rank_stride_bytes).  One
step is one cc_all_reduce call (the fused ring kernel) over inputs already
resident in HBM; its algorithmic traffic is 2*N*M*4 bytes (every rank's input
read once, every rank's output written once).

stdout carries one JSON object per line:
  * first, one record per other workload -- the int32 ring at N = 4, a small
    bf16 ring (4 ranks x 131,072), the bucketed bf16 gradient sync, the
    ZeRO-3 ReduceScatter / AllGather at N = 16 and the MoE AllToAll(v) --
    each with its timing, rank stride and a bit-for-bit parity verdict
    against the oracle run on the same inputs;
  * LAST, the headline line (at most 2 KB): GB/s, ms per step, % of peak,
    simulated busbw, the fused kernel's roofline (per-launch HIP event
    durations; HBM traffic from committed rocprofv3 counters while the kernel
    source is unchanged), the bf16 twin, the alpha-beta fit of the stepwise
    ring at N = 8, the oracle's time on the host cores, and whether the timed
    output equals the oracle's bit for bit.
--extras PATH writes the longer sweeps (rank-stride pads, alpha-beta at
N = 4, 8, 16, every schedule, hierarchical grids, AllToAll variants, INT8
with error feedback) to PATH as one JSON document.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) + simulated busbw for N-rank ring AllReduce"
PMC_FILE = os.path.join(ROOT, "profiles", "ring_fused_f32_n8_m67108864_pmc.json")
HEADLINE_MAX_BYTES = 2048
BUCKET_CAP_BYTES = 25 * 1024 * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def emit(rec: dict) -> None:
    print(json.dumps(rec, separators=(",", ":")), flush=True)


# ---------------------------------------------------------------- layout

def rank_stride_bytes(row_bytes):
    """Rank stride for rows of row_bytes: the payload rounded up to a power of
    two P, plus max(32 KiB, P/1024) (equal offsets of the ranks then spread
    over the HBM channels), or plus 1 MiB for P of 4 to 32 MiB, where the
    smaller pad measured 1-40% slower at 4 to 64 ranks."""
    p = 256
    while p < row_bytes:
        p *= 2
    if (4 << 20) <= p <= (32 << 20):
        return p + (1 << 20)
    return p + max(32_768, p // 1024)


def strided_ranks(N, L, dtype, device):
    """N x L rank rows, rank_stride_bytes(L * element size) apart."""
    import torch
    es = torch.tensor([], dtype=dtype).element_size()
    S = rank_stride_bytes(L * es) // es
    return torch.empty(N * S, dtype=dtype, device=device).view(N, S)[:, :L]


def rank_tensor(N, M, dtype, pad_bytes, device):
    import torch
    es = torch.tensor([], dtype=dtype).element_size()
    S = M + pad_bytes // es
    return torch.empty(N * S, dtype=dtype, device=device).view(N, S)[:, :M]


def randn_ranks(N, M, gen, device, pad_bytes):
    """N x M fp32 Gaussian (sigma 1e-3) rank rows, M*4 + pad_bytes apart."""
    import torch
    t = rank_tensor(N, M, torch.float32, pad_bytes, device)
    # sampled in place: a torch copy here would share its kernel with the
    # copy probe whose counters scale the profiles' HBM traffic
    t.normal_(0.0, 1e-3, generator=gen)
    return t


def _host_tensor(x):
    import numpy as np
    import torch
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else torch.from_numpy(x)


def upload(xs, t):
    """Row r of the device tensor t takes xs[r] (bf16 as uint16 bits); a
    shorter array fills the row's prefix."""
    for r, x in enumerate(xs):
        t[r, :len(x)].copy_(_host_tensor(x), non_blocking=False)


def download(t):
    """[N, L] device tensor -> numpy (bf16 as uint16 bits)."""
    import numpy as np
    import torch
    h = t.detach().cpu().contiguous()
    if h.dtype == torch.bfloat16:
        return h.view(torch.int16).numpy().view(np.uint16)
    return h.numpy()


def same_bits(a, b) -> bool:
    import numpy as np
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ---------------------------------------------------------------- timing

def time_launches(fn, steps, warmup):
    """Warm up, then time `steps` launches with a HIP event pair around each
    launch (on the launching stream) and a pair around the whole region."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [a.elapsed_time(b) for a, b in evs]
    return {"total_ms": t0.elapsed_time(t1), "per_launch_ms": per, "wall_s": wall}


def time_steps(fn, steps, warmup):
    """Warm up, then time exactly `steps` back-to-back calls between one HIP
    event pair on the launching stream, with a device synchronization on both
    sides (no instrumentation between the calls)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return {"total_ms": t0.elapsed_time(t1), "wall_s": time.perf_counter() - wall0}


def time_graph(fn, reps=20, per_graph=1):
    """GPU time per call of fn without host launch overhead: `per_graph` calls
    captured into one HIP graph (torch.cuda.CUDAGraph), replayed `reps` times
    between HIP events.  The captured kernels are the library's own (no
    memset nodes)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_graph)


def _time_gpu(fn, reps, per):
    """GPU time of fn from graph replays; eager back-to-back launches between
    HIP events if the call cannot be captured."""
    try:
        return time_graph(fn, reps, per), "graph"
    except Exception:  # noqa: BLE001 - capture unsupported for this launch kind
        import torch
        torch.cuda.synchronize()
        r = time_steps(fn, reps * per, 3)
        return r["total_ms"] / (reps * per), "eager"


def _avg_ms(fn, steps=10, warmup=3):
    r = time_steps(fn, steps, warmup)
    return r["total_ms"] / steps


def gbps(nbytes, ms):
    return nbytes / ms / 1e6


def traffic_from_profile(pmc_file=PMC_FILE):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs,
    scaled by the copy-kernel calibration; None if the kernel changed."""
    if not os.path.exists(pmc_file):
        return None, "no counter file"
    with open(pmc_file) as f:
        p = json.load(f)
    from ring_allreduce_reduction_02_amd.profsum import sources_hash
    if not p.get("kernel_sources") or p.get("kernel_source_sha256_16") != sources_hash(p["kernel_sources"]):
        return None, "kernel changed since the counters were taken"
    fetch = p["fetch_kib_per_dispatch"] * 1024.0 * p["fetch_scale"]
    write = p["write_kib_per_dispatch"] * 1024.0 * p["write_scale"]
    return fetch + write, "rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE (scaled by a plain copy)"


# ---------------------------------------------------------------- the oracle leg
# The only code in this file that runs the oracle: the step-explicit CPU
# simulator, on the same inputs as the GPU, timed on the host cores.  Its
# outputs also decide the parity verdicts below.

def _oracle():
    from oracle import ccsim
    return ccsim


def oracle_run(fn, min_seconds=0.0, max_runs=25):
    """Run fn() (an oracle call) until min_seconds of CPU time have passed
    (at least once); returns (median seconds, runs, total seconds, last
    output)."""
    times, out = [], None
    t_all = time.perf_counter()
    while not times or (len(times) < max_runs and time.perf_counter() - t_all < min_seconds) or \
            (min_seconds > 0 and len(times) < 3):
        t = time.perf_counter()
        out = fn()
        times.append(time.perf_counter() - t)
    return sorted(times)[len(times) // 2], len(times), sum(times), out


def host_info():
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "cpu_model": cpu_model or platform.processor()}


def cpu_baseline(xs, dtype, min_seconds=10.0):
    """The oracle as it stands on the host cores: the step-explicit ring
    AllReduce simulator on the headline's own inputs, repeated until
    min_seconds of CPU work (median run reported).  Returns the record and
    the oracle's output."""
    cs = _oracle()
    N, M = len(xs), len(xs[0])
    es = 4 if dtype == "f32" else 2
    t, runs, total, out = oracle_run(lambda: cs.ring_all_reduce(xs, "sum", dtype), min_seconds)
    h = host_info()
    rec = {"value": round(2 * N * M * es / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"the whole workload (ring AllReduce SUM, N={N}, M={M} {dtype}), step-explicit NumPy "
                     f"simulator, single-threaded; {runs} runs in {total:.1f} s, median {t:.3f} s",
           "host": f"{h['cpu_model']}, {h['host_logical_cpus']} logical CPUs, {h['affinity_cpus']} in affinity"}
    return rec, out


# ---------------------------------------------------------------- headline

def run_headline(args, dev):
    """The timed steps of the headline AllReduce.  Returns the measurements
    and the recv buffer downloaded to the host."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    N, M = args.ranks, args.count
    tdt = torch.float32 if args.dtype == "f32" else torch.bfloat16
    es = 4 if args.dtype == "f32" else 2
    log(f"generating {N} x {M} {args.dtype} synthetic gradients")
    xs = synth.gradient_inputs(N, M, args.dtype)
    send = rank_tensor(N, M, tdt, args.pad_bytes, dev)
    recv = rank_tensor(N, M, tdt, args.pad_bytes, dev)
    upload(xs, send)
    ws = ccgpu.make_workspace("all_reduce", N, M, args.dtype, args.algo, args.fuse_depth, dev)
    if args.copy_probe_bytes:
        copy_probe(args.copy_probe_bytes, dev)

    def step():
        ccgpu.all_reduce(send, recv, op="sum", algo=args.algo, fuse_depth=args.fuse_depth, workspace=ws,
                         blocks_per_cu=args.blocks_per_cu)

    log("timing")
    # the K timed steps run back to back; the per-launch durations behind the
    # roofline come from a second, instrumented pass of K launches (an event
    # pair around every launch adds a few us per step to the first)
    recv.fill_(float("nan"))
    res = time_steps(step, args.steps, args.warmup)
    per = time_launches(step, args.steps, 2)["per_launch_ms"]
    torch.cuda.synchronize()
    got = download(recv) if not args.no_cpu_baseline else None
    m = {"N": N, "M": M, "es": es, "ms_per_step": res["total_ms"] / args.steps, "per_launch_ms": per,
         "rank_stride_bytes": send.stride(0) * es, "xs": xs, "got": got}
    del send, recv, ws
    torch.cuda.empty_cache()
    return m


def bf16_twin(args, dev):
    """The same AllReduce on the bf16 rounding of the same samples."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    N, M = args.ranks, args.count
    xb = synth.gradient_inputs(N, M, "bf16")
    sb = rank_tensor(N, M, torch.bfloat16, args.pad_bytes, dev)
    rb = rank_tensor(N, M, torch.bfloat16, args.pad_bytes, dev)
    upload(xb, sb)
    r = time_steps(lambda: ccgpu.all_reduce(sb, rb, algo="ring", fuse_depth=0), args.steps, args.warmup)
    ms = r["total_ms"] / args.steps
    out = {"ms_per_step": round(ms, 5), "GBps": round(gbps(2 * N * M * 2, ms), 1),
           "pct_of_peak": round(100 * gbps(2 * N * M * 2, ms) / PEAK_HBM_GBPS, 2)}
    got = download(rb) if not args.no_cpu_baseline else None
    del sb, rb
    torch.cuda.empty_cache()
    if got is not None:
        cs = _oracle()
        log("  oracle: bf16 ring AllReduce")
        t, _, _, exp = oracle_run(lambda: cs.ring_all_reduce(xb, "sum", "bf16"))
        out["parity"] = all(same_bits(got[r], exp[r]) for r in range(N))
        out["oracle_s"] = round(t, 3)
    return out


def alpha_beta_n8(dev, pad_bytes):
    """alpha-beta fit of the stepwise ring AllReduce (one kernel per ring
    step, fp32 SUM) at N = 8 over per-rank sizes 4 KiB .. 64 MiB, GPU time
    from HIP-graph replays: T = alpha * 2(N-1) + beta * bytes sent per rank."""
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu
    N = 8
    sizes = [1 << k for k in range(10, 25, 2)]
    gen = torch.Generator(device=dev).manual_seed(20261202)
    send = randn_ranks(N, sizes[-1], gen, dev, pad_bytes)
    recv = rank_tensor(N, sizes[-1], torch.float32, pad_bytes, dev)
    st, by, ts = [], [], []
    for m in sizes:
        s_, r_ = send[:, :m], recv[:, :m]
        t, _ = _time_gpu(lambda: ccgpu.all_reduce(s_, r_, fuse_depth=1), 10, 16 if m <= (1 << 20) else 2)
        b, n = ccgpu.get_traffic("all_reduce", N, m, "f32", "ring")
        st.append(n); by.append(b); ts.append(t / 1e3)
    fit = calib.fit_alpha_beta(st, by, ts)
    del send, recv
    torch.cuda.empty_cache()
    return {"n": N, "alpha_us": round(fit["alpha_us_per_step"], 3), "beta_ps_per_byte": round(fit["beta_ps_per_byte"], 3),
            "link_GBps": round(fit["link_GBps"], 1), "n_star_bytes": round(fit["n_star_bytes"]),
            "sizes": "4KiB..64MiB per rank", "max_rel_residual": round(fit["max_rel_residual"], 3)}


def make_headline(m, args, roof, twin, ab, cpu, parity):
    """The headline record (the last stdout line)."""
    N, M, es = m["N"], m["M"], m["es"]
    ms = m["ms_per_step"]
    alg_bytes = 2 * N * M * es
    value = gbps(alg_bytes, ms)
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"ring_allreduce_sum_n{N}_m{M}_{args.dtype}",
            "nranks": N,
            "count_per_rank": M,
            "algo": args.algo,
            "fuse_depth": args.fuse_depth,
            "rank_stride_bytes": m["rank_stride_bytes"],
            "values": "Gaussian sigma=1e-3" + (" (bf16 RNE)" if args.dtype == "bf16" else ""),
            "parallelism": f"{N} logical ranks in one GPU's HBM",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "busbw_GBps": round((M * es) / (ms / 1e3) * 2 * (N - 1) / N / 1e9, 2),
        "algorithmic_bytes_per_step": alg_bytes,
        "parity": parity,
        "roofline": roof,
        "bf16_twin": twin,
        "alpha_beta": ab,
        "cpu_baseline": cpu,
    }


def headline_line(h: dict) -> str:
    s = json.dumps(h, separators=(",", ":"))
    if len(s.encode()) > HEADLINE_MAX_BYTES:
        raise ValueError(f"headline line is {len(s.encode())} bytes (at most {HEADLINE_MAX_BYTES})")
    return s


def roofline_of(m, args):
    per = m["per_launch_ms"]
    alg_bytes = 2 * m["N"] * m["M"] * m["es"]
    avg = sum(per) / len(per)
    traffic, _src = traffic_from_profile() if (args.algo == "ring" and args.fuse_depth == 0 and args.dtype == "f32"
                                                and m["N"] == 8 and m["M"] == 67_108_864) else (None, "")
    kname = {"ring": "k_ring_fused", "hd": "k_tree_fused", "butterfly": "k_tree_fused"}[args.algo]
    if args.fuse_depth:
        kname = "stepwise (several kernels per step)"
    achieved = gbps(alg_bytes, avg)
    return {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": round(traffic) if traffic else None,
            "traffic_over_algorithmic": round(traffic / alg_bytes, 4) if traffic else None,
            "avg_launch_ms": round(avg, 5), "min_launch_ms": round(min(per), 5)}


# ---------------------------------------------------------------- other workloads (one record each)

def rec_int32_ring(dev, nsets=64):
    """Ring AllReduce SUM, N = 4, M = 1,048,576 int32 uniform in [-1000, 1000]:
    one buffer set (cache-resident) and `nsets` rotating sets (2 GiB, beyond
    the 256 MB last-level cache), GPU time from HIP-graph replays."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    N, M = 4, 1 << 20
    xs = synth.uniform_int32(synth.W_INT_RING, N, M)
    base = strided_ranks(N, M, torch.int32, dev)
    upload(xs, base)
    sets = []
    for i in range(nsets):
        s_ = base if i == 0 else strided_ranks(N, M, torch.int32, dev)
        if i:
            s_.copy_(base)
        sets.append((s_, strided_ranks(N, M, torch.int32, dev)))
    alg = 2 * N * M * 4
    ms1 = time_graph(lambda: ccgpu.all_reduce(sets[0][0], sets[0][1]), 10, 32)

    def rot():
        for s_, r_ in sets:
            ccgpu.all_reduce(s_, r_)
    msr = time_graph(rot, 10, 1) / nsets
    torch.cuda.synchronize()
    got0, got_last = download(sets[0][1]), download(sets[-1][1])
    cs = _oracle()
    t, _, _, exp = oracle_run(lambda: cs.ring_all_reduce(xs, "sum", "int32"))
    par = all(same_bits(got0[r], exp[r]) and same_bits(got_last[r], exp[r]) for r in range(N))
    del sets, base
    torch.cuda.empty_cache()
    return {"section": "int32_ring_n4_m1048576", "dtype": "int32", "algo": "ring",
            "rank_stride_bytes": rank_stride_bytes(M * 4),
            "same_set_us": round(ms1 * 1e3, 2), "same_set_GBps": round(gbps(alg, ms1), 1),
            "rotating_sets": nsets, "rotating_us": round(msr * 1e3, 2), "rotating_GBps": round(gbps(alg, msr), 1),
            "parity": par, "oracle_s": round(t, 3)}


def rec_small_ring(dev):
    """A small message: ring AllReduce SUM of 131,072 bf16 elements over 4
    ranks, the size of the 4-chip SCCL measurement the AllReduce algorithm
    notes quote in their 2-port ring section (15.757 us there, other
    hardware: context, not a target).  GPU time from HIP-graph replays of the
    fused ring, the fused 2-port ring, the stepwise ring (one kernel per
    step, 6 steps) and the standalone ReduceScatter and AllGather; every
    output compared bit for bit with the oracle."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    N, M = 4, 131_072
    S = M // N
    xs = synth.gradient_inputs(N, M, "bf16", sigma=1e-2, workload=synth.W_SMALL_RING)
    send = strided_ranks(N, M, torch.bfloat16, dev)
    upload(xs, send)
    outs = {k: strided_ranks(N, M, torch.bfloat16, dev) for k in ("ring", "ring_2port", "stepwise", "ag")}
    shard = strided_ranks(N, S, torch.bfloat16, dev)
    ws = ccgpu.make_workspace("all_reduce", N, M, "bf16", "ring", 1, dev)
    us = {
        "ring_fused_us": time_graph(lambda: ccgpu.all_reduce(send, outs["ring"]), 10, 32),
        "ring_2port_fused_us": time_graph(lambda: ccgpu.all_reduce(send, outs["ring_2port"], algo="ring_2port"),
                                          10, 32),
        "ring_stepwise_us": time_graph(lambda: ccgpu.all_reduce(send, outs["stepwise"], fuse_depth=1, workspace=ws),
                                       10, 32),
        "reduce_scatter_us": time_graph(lambda: ccgpu.reduce_scatter(send, shard), 10, 32),
        "all_gather_us": time_graph(lambda: ccgpu.all_gather(shard, outs["ag"]), 10, 32),
    }
    torch.cuda.synchronize()
    got = {k: download(v) for k, v in outs.items()}
    got_shard = download(shard)
    cs = _oracle()
    t, _, _, exp = oracle_run(lambda: cs.ring_all_reduce(xs, "sum", "bf16"))
    exp2 = cs.ring2_all_reduce(xs, "sum", "bf16")
    exp_rs = cs.ring_reduce_scatter(xs, "sum", "bf16")
    exp_ag = cs.ring_all_gather(exp_rs, "bf16")
    par = (all(same_bits(got["ring"][r], exp[r]) and same_bits(got["stepwise"][r], exp[r])
               and same_bits(got["ring_2port"][r], exp2[r]) and same_bits(got_shard[r], exp_rs[r])
               and same_bits(got["ag"][r], exp_ag[r]) for r in range(N)))
    del outs, shard, send, ws
    torch.cuda.empty_cache()
    rec = {"section": "ring_n4_m131072_bf16", "rank_stride_bytes": rank_stride_bytes(M * 2)}
    rec.update({k: round(v * 1e3, 2) for k, v in us.items()})
    rec.update({"page_sccl_4chip_fp16_us": 15.757, "parity": par, "oracle_s": round(t, 3)})
    return rec


def bucket_layout(N, sizes, tensors):
    """The bucketed workload's per-rank flat buffers: tensors at the
    cc_bucket_plan offsets (25 MiB buckets, 128-element aligned), zero
    between them."""
    import numpy as np

    from ring_allreduce_reduction_02_amd import ccgpu
    bof, toff, boff, bcnt = ccgpu.bucket_plan(sizes, 2, BUCKET_CAP_BYTES, 128)
    extent = boff[-1] + bcnt[-1]
    host = np.zeros((N, extent), dtype=np.uint16)
    for r in range(N):
        for t, x in enumerate(tensors[r]):
            host[r, toff[t]:toff[t] + len(x)] = x
    return host, toff, boff, bcnt


def rec_buckets(dev):
    """Bucketed bf16 gradient sync, N = 8: 120 tensors with log-uniform sizes
    in [4K, 16M] elements, N(0, 1e-2) values, 25 MiB buckets, one fused launch
    per 16 buckets; ring, halving-doubling and butterfly on the same data,
    each checked bit for bit against the oracle's per-bucket AllReduce; the
    per-bucket GB/s of the ring with one launch per bucket."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    N = 8
    sizes = synth.tensor_sizes_log_uniform()
    log("  generating 120 tensors per rank")
    tensors = synth.bucket_tensors(N, sizes)
    host, toff, boff, bcnt = bucket_layout(N, sizes, tensors)
    extent = host.shape[1]
    send = strided_ranks(N, extent, torch.bfloat16, dev)
    upload(host, send)
    del host
    recv = strided_ranks(N, extent, torch.bfloat16, dev)
    alg = 2 * N * sum(bcnt) * 2
    cs = _oracle()
    ref_buckets = cs.bucket_pack(sizes, 2, BUCKET_CAP_BYTES)
    out = {"section": "bucketed_bf16_n8_120_tensors", "dtype": "bf16", "tensors": len(sizes), "buckets": len(boff),
           "elements_per_rank": sum(bcnt), "rank_stride_bytes": send.stride(0) * 2}
    for algo in ("hd", "butterfly", "ring"):
        ms = _avg_ms(lambda: ccgpu.all_reduce_buckets(send, recv, boff, bcnt, algo=algo))
        out[algo] = {"ms": round(ms, 4), "GBps": round(gbps(alg, ms), 1)}
    # the ring's output (the last run) against the oracle; halving-doubling
    # and butterfly are compared whole by the tests
    torch.cuda.synchronize()
    got = download(recv)
    log("  oracle: ring AllReduce of every bucket")
    t, _, _, exp = oracle_run(lambda: cs.bucketed_all_reduce(tensors, ref_buckets, "ring", "sum", "bf16"))
    out["ring"]["parity"] = all(same_bits(got[r, toff[k]:toff[k] + len(tensors[r][k])], exp[r][k])
                                for r in range(N) for k in range(len(sizes)))
    out["ring"]["oracle_s"] = round(t, 2)
    del got, exp
    per = []
    for o, c in zip(boff, bcnt):
        s_, r_ = send[:, o:o + c], recv[:, o:o + c]
        t, _ = _time_gpu(lambda: ccgpu.all_reduce(s_, r_), 10, 1)
        per.append(round(gbps(2 * N * c * 2, t)))
    out["ring_per_bucket_GBps"] = per
    del send, recv
    torch.cuda.empty_cache()
    return out


def rec_zero3(dev):
    """ZeRO-3-style standalone ReduceScatter then AllGather, N = 16,
    M = 33,554,432 fp32 uniform [-1, 1) per rank, plus int32 MAX / PROD
    ReduceScatters on 1,048,576 elements; every output compared whole with
    the oracle."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    cs = _oracle()
    N, M = 16, 1 << 25
    S = M // N
    xs = synth.uniform_f32(synth.W_ZERO3, N, M)
    send = strided_ranks(N, M, torch.float32, dev)
    upload(xs, send)
    shard = strided_ranks(N, S, torch.float32, dev)
    full = strided_ranks(N, M, torch.float32, dev)
    alg = (N + 1) * M * 4
    out = {"section": "zero3_rs_ag_n16_m33554432_f32",
           "rank_stride_bytes": [send.stride(0) * 4, shard.stride(0) * 4]}
    shards = None
    for algo, oracle_fn in (("hd", cs.hd_reduce_scatter), ("ring", cs.ring_reduce_scatter)):
        ms = _avg_ms(lambda: ccgpu.reduce_scatter(send, shard, algo=algo))
        torch.cuda.synchronize()
        got = download(shard)
        log(f"  oracle: {algo} ReduceScatter")
        t, _, _, exp = oracle_run(lambda: oracle_fn(xs, "sum", "f32"))
        out[f"reduce_scatter_{algo}"] = {"ms": round(ms, 4), "GBps": round(gbps(alg, ms), 1),
                                         "parity": all(same_bits(got[r], exp[r]) for r in range(N)),
                                         "oracle_s": round(t, 2)}
        if algo == "ring":
            shards = [got[r].copy() for r in range(N)]   # the AllGather below gathers these
    del xs, send
    ms = _avg_ms(lambda: ccgpu.all_gather(shard, full))
    torch.cuda.synchronize()
    fg = download(full)
    t, _, _, exp = oracle_run(lambda: cs.ring_all_gather(shards, "f32"))
    out["all_gather_ring"] = {"ms": round(ms, 4), "GBps": round(gbps(alg, ms), 1),
                              "parity": all(same_bits(fg[r], exp[r]) for r in range(N)), "oracle_s": round(t, 2)}
    del fg, exp, shard, full
    torch.cuda.empty_cache()
    Mi = 1 << 20
    ints = {}
    for op, kind, xs_i in (("max", "full", synth.uniform_int32(synth.W_ZERO3, N, Mi, sub=1)),
                           ("prod", "small", synth.choice_int32(synth.W_ZERO3, N, Mi, [-2, -1, 1, 2], sub=2)),
                           ("prod", "full", synth.uniform_int32(synth.W_ZERO3, N, Mi, sub=3))):
        si = strided_ranks(N, Mi, torch.int32, dev)
        ri = strided_ranks(N, Mi // N, torch.int32, dev)
        upload(xs_i, si)
        ccgpu.reduce_scatter(si, ri, op=op)
        torch.cuda.synchronize()
        got = download(ri)
        exp = cs.ring_reduce_scatter(xs_i, op, "int32")
        ints[f"{op}_{kind}"] = all(same_bits(got[r], exp[r]) for r in range(N))
    out["int32_reduce_scatter_parity"] = ints
    torch.cuda.empty_cache()
    return out


def moe_inputs(N=8, T=4096, E=64, K=8, H=7168):
    """Counts matrix and tagged bf16 payload rows of the MoE workload."""
    import numpy as np

    from ring_allreduce_reduction_02_amd import synth
    ch = synth.moe_routing(N, T, E, K)
    C = np.zeros((N, N), dtype=np.int64)
    for i in range(N):
        _, C[i] = synth.moe_send_layout(ch[i], N, E)
    rows = [synth.moe_payload_rows(i, int(C[i].sum()), H) for i in range(N)]
    return C, rows


def rec_moe(dev):
    """MoE AllToAll(v) dispatch and combine, N = 8, 4096 tokens per rank, top-8
    of 64 experts with Zipf(1.2) loads, rows of 7168 bf16: the dispatch (direct
    and pairwise) compared with the oracle's blocked transpose byte for byte,
    the combine (the transposed exchange) with the original rows."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu
    N, H = 8, 7168
    log("  generating routed rows")
    C, rows = moe_inputs(N, H=H)
    Ls, Lr = int(C.sum(1).max()), int(C.sum(0).max())
    send = strided_ranks(N, Ls * H, torch.bfloat16, dev)
    upload([r.reshape(-1) for r in rows], send)
    recv = strided_ranks(N, Lr * H, torch.bfloat16, dev)
    back = strided_ranks(N, Ls * H, torch.bfloat16, dev)
    alg = 2 * int(C.sum()) * H * 2
    out = {"section": "moe_alltoall_n8_t4096_h7168_bf16", "rows_received": C.sum(0).tolist(),
           "skew_max_over_mean": round(float(C.sum(0).max() / C.sum(0).mean()), 3),
           "rank_stride_bytes": [send.stride(0) * 2, recv.stride(0) * 2]}
    cs = _oracle()
    t, _, _, exp = oracle_run(lambda: cs.all_to_all([r.reshape(-1) for r in rows], C, row=H))
    for fd, name in ((1, "pairwise"), (0, "direct")):
        ms = _avg_ms(lambda: ccgpu.all_to_all(send, recv, C.tolist(), H, fuse_depth=fd))
        torch.cuda.synchronize()
        got = download(recv)
        out[f"dispatch_{name}"] = {"ms": round(ms, 4), "GBps": round(gbps(alg, ms), 1),
                                   "parity": all(same_bits(got[j, :len(exp[j])], exp[j]) for j in range(N))}
        del got
    out["oracle_s"] = round(t, 2)
    ms = _avg_ms(lambda: ccgpu.all_to_all(recv, back, C.T.tolist(), H))
    torch.cuda.synchronize()
    got = download(back)
    out["combine_direct"] = {"ms": round(ms, 4), "GBps": round(gbps(alg, ms), 1),
                             "round_trip_identical": all(same_bits(got[i, :rows[i].size], rows[i].reshape(-1))
                                                         for i in range(N))}
    del send, recv, back
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- extras (--extras PATH)

def pad_sweep(N, M, dev, pads=(0, 65_792, 262_144, 2_097_152), steps=10):
    """The headline AllReduce with rank buffers `pad` bytes apart beyond the
    payload."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu
    gen = torch.Generator(device=dev).manual_seed(20261202)
    res = {}
    for pad in pads:
        s = randn_ranks(N, M, gen, dev, pad)
        r = rank_tensor(N, M, torch.float32, pad, dev)
        t = time_launches(lambda: ccgpu.all_reduce(s, r), steps, 3)
        per = sorted(t["per_launch_ms"])
        ms = per[len(per) // 2]
        res[str(pad)] = {"median_launch_ms": round(ms, 5), "min_launch_ms": round(per[0], 5),
                         "GBps": round(gbps(2 * N * M * 4, ms), 1)}
        del s, r
        torch.cuda.empty_cache()
    return res


def alpha_beta(dev, ranks=(4, 8, 16), max_bytes=1 << 30):
    """Stepwise ring AllReduce (fp32 SUM) at N = 4, 8, 16 over per-rank sizes
    4 KiB .. 1 GiB (x4), GPU time from HIP-graph replays, in two variants:
    one kernel per ring step, and all steps in one launch with a grid-wide
    barrier between steps.  Fits T = alpha * 2(N-1) + beta * bytes sent
    per rank per N, and over all N together with a per-call constant t0
    (T = t0 + alpha * steps + beta * bytes).  The fused kernel's
    T = t0 + bytes / BW is fitted on the same sizes."""
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu
    sizes = [m for m in (1 << k for k in range(10, 29, 2)) if m * 4 <= max_bytes]
    gen = torch.Generator(device=dev).manual_seed(20261202)
    out = {"schedule": "ring AllReduce, fp32 SUM, fuse_depth=1 (one ring step per pass)",
           "variants": {"kernel_per_step": "one kernel launch per ring step",
                        "grid_barrier": "one launch, grid barrier between ring steps"},
           "per_n": {}}
    glob = {"kernel_per_step": ([], [], []), "grid_barrier": ([], [], [])}
    for N in ranks:
        send = strided_ranks(N, sizes[-1], torch.float32, dev)
        send.normal_(0.0, 1e-3, generator=gen)
        recv = strided_ranks(N, sizes[-1], torch.float32, dev)
        ws = ccgpu.make_workspace("all_reduce", N, sizes[-1], "f32", "ring", 1, dev, grid_sync=True)
        for _ in range(10):
            ccgpu.all_reduce(send, recv, fuse_depth=0)
        torch.cuda.synchronize()
        pts, st, by, t_ks, t_gb, fb, ft, how = [], [], [], [], [], [], [], set()
        for m in sizes:
            s, r = send[:, :m], recv[:, :m]
            per = 16 if m <= (1 << 20) else 2
            b, n = ccgpu.get_traffic("all_reduce", N, m, "f32", "ring")
            tk, h1 = _time_gpu(lambda: ccgpu.all_reduce(s, r, fuse_depth=1), 10, per)
            tg, h2 = _time_gpu(lambda: ccgpu.all_reduce(s, r, fuse_depth=1, workspace=ws, grid_sync=True), 10, per)
            tf, h3 = _time_gpu(lambda: ccgpu.all_reduce(s, r, fuse_depth=0), 10, per)
            how |= {h1, h2, h3}
            st.append(n); by.append(b); t_ks.append(tk / 1e3); t_gb.append(tg / 1e3)
            fb.append(2 * N * m * 4); ft.append(tf / 1e3)
            pts.append({"bytes_per_rank": m * 4, "kernel_per_step_us": round(tk * 1e3, 3),
                        "grid_barrier_us": round(tg * 1e3, 3), "fused_us": round(tf * 1e3, 3)})
        torch.cuda.synchronize()
        out["per_n"][str(N)] = {
            "kernel_per_step": calib.fit_alpha_beta(st, by, t_ks),
            "grid_barrier": calib.fit_alpha_beta(st, by, t_gb),
            "fused": calib.fit_fixed_plus_bandwidth(fb, ft),
            "points": pts,
            "timing": sorted(how),
            "barrier_timed_out": ccgpu.grid_sync_timed_out(ws),
        }
        for key, ts in (("kernel_per_step", t_ks), ("grid_barrier", t_gb)):
            glob[key][0].extend(st); glob[key][1].extend(by); glob[key][2].extend(ts)
        del send, recv, ws
        torch.cuda.empty_cache()
    out["all_n"] = {k: calib.fit_launch_alpha_beta(*v) for k, v in glob.items()}
    return out


def schedules(dev, pad_bytes=262_144):
    """Every AllReduce schedule on one GPU: fused throughput at the headline
    size (N = 8, 67,108,864 fp32 per rank; N = 12 for the pair-folded
    halving-doubling and butterfly), and the stepwise schedules over per-rank
    sizes 4 KiB .. 64 MiB at N = 8 (HIP-graph replays) with an alpha-beta fit
    each, the measured ring/tree crossover and the model's crossover from the
    ring's fitted alpha and beta."""
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu
    out = {"fused": {}, "stepwise_n8": {}}
    gen = torch.Generator(device=dev).manual_seed(20261202)
    N, M = 8, 1 << 26
    send = randn_ranks(N, M, gen, dev, pad_bytes)
    recv = rank_tensor(N, M, torch.float32, pad_bytes, dev)
    for algo in ("ring", "hd", "butterfly", "tree", "double_tree", "ring_2port"):
        ms = _avg_ms(lambda: ccgpu.all_reduce(send, recv, algo=algo), 10, 3)
        out["fused"][f"{algo}_n8"] = {"ms": round(ms, 4), "GBps": round(gbps(2 * N * M * 4, ms), 1)}
    del send, recv
    torch.cuda.empty_cache()
    N12, M12 = 12, 1 << 25
    send = torch.randn(N12, M12, generator=gen, device=dev) * 1e-3
    recv = torch.empty_like(send)
    for algo in ("hd", "butterfly"):
        ms = _avg_ms(lambda: ccgpu.all_reduce(send, recv, algo=algo), 10, 3)
        out["fused"][f"{algo}_n12_pair_folded"] = {"ms": round(ms, 4), "GBps": round(gbps(2 * N12 * M12 * 4, ms), 1)}
    del send, recv
    torch.cuda.empty_cache()

    sizes = [1 << k for k in range(10, 25, 2)]          # 1 Ki .. 16 Mi fp32 = 4 KiB .. 64 MiB per rank
    send = randn_ranks(N, sizes[-1], gen, dev, pad_bytes)
    recv = rank_tensor(N, sizes[-1], torch.float32, pad_bytes, dev)
    for _ in range(10):
        ccgpu.all_reduce(send, recv)
    torch.cuda.synchronize()
    times = {}
    for algo in ("ring", "hd", "butterfly", "tree", "double_tree", "ring_2port"):
        pts, st, by, ts = [], [], [], []
        for m in sizes:
            s_, r_ = send[:, :m], recv[:, :m]
            per = 16 if m <= (1 << 20) else 2
            t, how = _time_gpu(lambda: ccgpu.all_reduce(s_, r_, algo=algo, fuse_depth=1), 10, per)
            b, n = ccgpu.get_traffic("all_reduce", N, m, "f32", algo)
            st.append(n); by.append(b); ts.append(t / 1e3)
            pts.append({"bytes_per_rank": m * 4, "us": round(t * 1e3, 3), "steps": n, "max_bytes_sent_per_rank": b})
        times[algo] = ts
        out["stepwise_n8"][algo] = {"fit": calib.fit_alpha_beta(st, by, ts), "points": pts}
    ring_fit = out["stepwise_n8"]["ring"]["fit"]
    model = calib.ring_tree_crossover(N, ring_fit["alpha_us_per_step"] * 1e-6, ring_fit["beta_ps_per_byte"] * 1e-12)
    measured = {}
    for other in ("tree", "double_tree", "butterfly"):
        first = next((sizes[i] * 4 for i in range(len(sizes)) if times["ring"][i] < times[other][i]), None)
        measured[f"ring_faster_than_{other}_from_bytes_per_rank"] = first
    out["crossover_n8"] = {"measured": measured, "model_from_ring_fit_bytes": model,
                           "note": "model: the pages' T_ring = T_tree with the ring's fitted alpha, beta; "
                                   "on one GPU a tree step's HBM traffic scales with its number of senders, "
                                   "which the per-link model does not see"}
    del send, recv
    torch.cuda.empty_cache()
    return out


def hierarchical(dev, pad_bytes=262_144):
    """Hierarchical AllReduce on one GPU: fused throughput of two- and
    three-level rank grids against the flat ring at the same N (8 ranks of
    67,108,864 fp32; 64 ranks of 8,388,608), the stepwise form against the
    stepwise flat ring over per-rank sizes 4 KiB .. 64 MiB at N = 8 and 64
    (HIP-graph replays) with an alpha-beta fit each, per-level traffic, and
    the two-tier model (AllReduce notes, BlueConnect cost; Napkin Math 1.6:
    450 GB/s inside a node, 50 GB/s across) for the same grids."""
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu
    out = {"fused": {}, "stepwise": {}, "level_traffic": {}, "two_tier_model": {}}
    gen = torch.Generator(device=dev).manual_seed(20261203)
    # 8 ranks of 256 MiB in the headline's layout; 64 ranks of 32 MiB
    # unpadded (a 256 KiB pad aliases at 64 ranks: 4.0 against 5.7 TB/s)
    for N, M, grids in ((8, 1 << 26, [(8,), (4, 2), (2, 4), (2, 2, 2)]), (64, 1 << 23, [(64,), (8, 8), (4, 4, 4)])):
        pad = pad_bytes if N == 8 else 0
        send = randn_ranks(N, M, gen, dev, pad)
        recv = rank_tensor(N, M, torch.float32, pad, dev)
        for dims in grids:
            if len(dims) == 1:
                fn = lambda: ccgpu.all_reduce(send, recv, algo="ring")
            else:
                fn = lambda d=dims: ccgpu.all_reduce_hierarchical(send, recv, d)
            ms = _avg_ms(fn, 10, 3)
            out["fused"]["x".join(map(str, dims))] = {"ms": round(ms, 4), "GBps": round(gbps(2 * N * M * 4, ms), 1)}
        del send, recv
        torch.cuda.empty_cache()

    sizes = [1 << k for k in range(10, 25, 2)]
    for N, grids in ((8, [(8,), (4, 2), (2, 2, 2)]), (64, [(64,), (8, 8), (4, 4, 4)])):
        top = sizes[-1] if N == 8 else sizes[-2]
        send = torch.randn(N, top, generator=gen, device=dev) * 1e-3
        recv = torch.empty_like(send)
        for dims in grids:
            pts, st, by, ts = [], [], [], []
            for m in (x for x in sizes if x <= top):
                s_, r_ = send[:, :m], recv[:, :m]
                per = 16 if m <= (1 << 20) else 2
                if len(dims) == 1:
                    fn = lambda: ccgpu.all_reduce(s_, r_, algo="ring", fuse_depth=1)
                    b, n = ccgpu.get_traffic("all_reduce", N, m, "f32", "ring")
                else:
                    fn = lambda d=dims: ccgpu.all_reduce_hierarchical(s_, r_, d, fuse_depth=1)
                    lv = ccgpu.hierarchical_traffic(dims, m, "f32")
                    b, n = sum(x for x, _ in lv), sum(y for _, y in lv)
                t, how = _time_gpu(fn, 10, per)
                st.append(n); by.append(b); ts.append(t / 1e3)
                pts.append({"bytes_per_rank": m * 4, "us": round(t * 1e3, 3), "steps": n, "timing": how})
            key = "x".join(map(str, dims))
            out["stepwise"][key] = {"fit": calib.fit_alpha_beta(st, by, ts), "points": pts}
            if len(dims) > 1:
                out["level_traffic"][key] = [{"bytes_per_rank": b, "steps": n}
                                             for b, n in ccgpu.hierarchical_traffic(dims, 1 << 24, "f32")]
        del send, recv
        torch.cuda.empty_cache()
    for dims in ((8, 8), (4, 2), (2, 2, 2)):
        N = 1
        for p in dims:
            N *= p
        lv = calib.multidim_time(1e9, dims, [5e-6] * len(dims), [1 / 450e9] + [1 / 50e9] * (len(dims) - 1))
        flat = calib.multidim_time(1e9, (N,), [5e-6], [1 / 50e9])[0]
        out["two_tier_model"]["x".join(map(str, dims))] = {
            "bytes": 1e9, "alpha_us": 5, "beta_GBps": [450] + [50] * (len(dims) - 1),
            "levels_ms": [round(x * 1e3, 3) for x in lv], "hier_ms": round(sum(lv) * 1e3, 3),
            "flat_ring_ms": round(flat * 1e3, 3), "speedup": round(flat / sum(lv), 2)}
    return out


def alltoall_variants(dev):
    """AllToAll variants on the MoE workload (8 ranks, 4096 tokens each, top-8
    of 64 experts with Zipf loads, rows of 7168 bf16): the capacity-padded
    dispatch and combine at C = 1 and 1.25 against the dropless AllToAll(v),
    the hierarchical exchange at 2 and 4 ranks per node, and the pairwise
    schedule's model (blog, Pairwise performance model) fitted on uniform
    exchanges and checked on the routed counts.  GB/s counts the bytes the
    kernels read and write."""
    import numpy as np
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu, synth
    N, H, T, K, E = 8, 7168, 4096, 8, 64
    rowb = H * 2
    ch = synth.moe_routing(N, T, E, K)
    Ce = np.stack([np.bincount(c.reshape(-1), minlength=E) for c in ch]).astype(np.int64)  # rows per (source, expert)
    C = Ce.reshape(N, N, E // N).sum(axis=2)                                                 # rows per (source, rank)
    gen = torch.Generator(device=dev).manual_seed(20261204)
    Ls, Lr = int(Ce.sum(1).max()), int(C.sum(0).max())
    send = torch.randn(N, Ls * H, generator=gen, device=dev).to(torch.bfloat16)
    out = {"tokens_per_rank": T, "topk": K, "experts": E, "hidden": H,
           "rows_per_expert_max_over_mean": round(float(Ce.sum(0).max() / Ce.sum(0).mean()), 2)}
    recv = torch.empty(N, Lr * H, device=dev, dtype=torch.bfloat16)
    ms = _avg_ms(lambda: ccgpu.all_to_all(send, recv, C.tolist(), H))
    moved = 2 * int(C.sum()) * rowb
    out["dropless_direct"] = {"ms": round(ms, 4), "GBps": round(gbps(moved, ms), 1), "wire_rows": int(C.sum())}
    del recv
    torch.cuda.empty_cache()
    for num, den in ((1, 1), (5, 4)):
        cap = ccgpu.moe_capacity(1, T, K, E, num, den)
        exp = torch.empty(N, E * cap * H, device=dev, dtype=torch.bfloat16)
        kept = int(np.minimum(Ce, cap).sum())
        wire = N * E * cap
        d_moved = kept * rowb + wire * rowb                 # kept rows read, every slot written
        c_moved = kept * rowb + int(Ce.sum()) * rowb        # kept rows read, every token row written
        r = {"capacity": cap, "dropped_rows": int(Ce.sum()) - kept,
             "dropped_frac": round(1 - kept / int(Ce.sum()), 4),
             "wire_rows": wire, "wire_over_dropless": round(wire / int(C.sum()), 3)}
        for fd, name in ((0, "direct"), (1, "pairwise")):
            ms = _avg_ms(lambda f=fd: ccgpu.moe_dispatch_padded(send, exp, Ce.tolist(), cap, H, fuse_depth=f))
            r[f"dispatch_{name}"] = {"ms": round(ms, 4), "GBps": round(gbps(d_moved, ms), 1)}
        ms = _avg_ms(lambda: ccgpu.moe_combine_padded(exp, send, Ce.tolist(), cap, H))
        r["combine_direct"] = {"ms": round(ms, 4), "GBps": round(gbps(c_moved, ms), 1)}
        out[f"padded_C{num / den:g}"] = r
        del exp
        torch.cuda.empty_cache()
    recv = torch.empty(N, Lr * H, device=dev, dtype=torch.bfloat16)
    for L in (2, 4):
        ws = ccgpu.make_all_to_all_hierarchical_workspace(C.tolist(), H, "bf16", L, dev)
        ms = _avg_ms(lambda: ccgpu.all_to_all_hierarchical(send, recv, C.tolist(), L, H, workspace=ws))
        tr = ccgpu.all_to_all_traffic(C.tolist(), H, "bf16", L)
        phases = ("flat", "aggregate", "exchange", "distribute")
        # every block is copied once in phase 1; inter-node bytes twice more
        moved_h = 2 * (int(C.sum()) * rowb + 2 * tr[2][1])
        out[f"hierarchical_L{L}"] = {
            "ms": round(ms, 4), "GBps_moved": round(gbps(moved_h, ms), 1),
            "transfers": {ph: f for ph, (f, _, _) in zip(phases, tr)},
            "bytes": {ph: t for ph, (_, t, _) in zip(phases, tr)}}
        del ws
        torch.cuda.empty_cache()
    # pairwise model: fit T = alpha * (launched steps) + beta * sum_k max_i n_(i,i+k) on uniform exchanges
    pts, st, by, ts = [], [], [], []
    for rows in (1, 4, 16, 64, 256, 1024):
        U = [[rows] * N for _ in range(N)]
        su = send[:, :N * rows * H]
        ru = recv[:, :N * rows * H]
        t, how = _time_gpu(lambda: ccgpu.all_to_all(su, ru, U, H, fuse_depth=1), 10, 4 if rows <= 64 else 1)
        mx, _ = ccgpu.all_to_all_step_bytes(U, H, "bf16")
        st.append(N); by.append(sum(mx)); ts.append(t / 1e3)
        pts.append({"rows_per_block": rows, "us": round(t * 1e3, 2), "timing": how})
    fit = calib.fit_alpha_beta(st, by, ts)
    mx, tot = ccgpu.all_to_all_step_bytes(C.tolist(), H, "bf16")
    t_moe, how = _time_gpu(lambda: ccgpu.all_to_all(send, recv, C.tolist(), H, fuse_depth=1), 10, 1)
    a, b = fit["alpha_us_per_step"] * 1e-6, fit["beta_ps_per_byte"] * 1e-12
    out["pairwise_model"] = {
        "uniform_fit": fit, "uniform_points": pts,
        "moe_step_max_bytes": mx, "moe_step_total_bytes": tot,
        "moe_measured_us": round(t_moe * 1e3, 2),
        "moe_predicted_us": round((N * a + b * sum(mx)) * 1e6, 2),
        "moe_predicted_pages_form_us": round(calib.pairwise_time(mx, a, b) * 1e6, 2),
        # uniform exchanges have step total = N x step max, so the same fit prices
        # total bytes at beta / N: the one-HBM reading of a step
        "moe_predicted_from_step_totals_us": round((N * a + b / N * sum(tot)) * 1e6, 2),
        "note": "one GPU: a step moves all N blocks through the one HBM, so its time follows the step's total "
                "bytes, not its largest block; the predicted figure uses the largest block as the blog's model does"}
    del send, recv
    torch.cuda.empty_cache()
    return out


def int8_ef(dev):
    """Block-wise INT8 AllReduce with error feedback at the headline shape
    (8 ranks, 67,108,864 gradients each): the fused kernel and the two-kernel
    form (message in a workspace) beside the plain fused ring AllReduce, for
    float32 and bf16 gradients; GB/s counts the bytes the kernels move
    (gradients read, error accumulators read and written, results written).
    The wire side: the message is M + 4 M / 128 bytes per rank against 4 M
    for float32 (3.88x less).  Accuracy: one step's norm-wise error against
    the float64 sum, and over 10 steps the error of the running sum of the
    results against the true running sum (bounded by the last accumulators,
    the telescoping identity)."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu
    N, M = 8, 1 << 26
    gen = torch.Generator(device=dev).manual_seed(20261205)
    out = {"ranks": N, "count": M, "message_bytes_per_rank": ccgpu.int8_message_bytes(M),
           "float32_bytes_per_rank": 4 * M, "wire_ratio": round(4 * M / ccgpu.int8_message_bytes(M), 4)}
    for dtype in ("f32", "bf16"):
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        es = 4 if dtype == "f32" else 2
        g = strided_ranks(N, M, tdt, dev)
        g.copy_((torch.randn(N, M, generator=gen, device=dev) * 1e-3).to(tdt))
        e = strided_ranks(N, M, torch.float32, dev).zero_()
        r = strided_ranks(N, M, tdt, dev)
        ms_f = _avg_ms(lambda: ccgpu.all_reduce_int8_ef(g, e, r, fuse_depth=0))
        ws = torch.empty(ccgpu.int8_ef_workspace_size(N, M, dtype, 1), dtype=torch.uint8, device=dev)
        ms_2 = _avg_ms(lambda: ccgpu.all_reduce_int8_ef(g, e, r, fuse_depth=1, workspace=ws))
        ms_p = _avg_ms(lambda: ccgpu.all_reduce(g, r, algo="ring"))
        fused_bytes = N * M * (2 * es + 8)
        two_bytes = N * M * (es + 8) + 2 * N * ccgpu.int8_message_bytes(M) + N * M * es
        out[dtype] = {
            "fused_ms": round(ms_f, 4), "fused_GBps": round(gbps(fused_bytes, ms_f), 1),
            "fused_pct_of_peak": round(100 * gbps(fused_bytes, ms_f) / PEAK_HBM_GBPS, 2),
            "two_kernel_ms": round(ms_2, 4), "two_kernel_GBps": round(gbps(two_bytes, ms_2), 1),
            "plain_ring_ms": round(ms_p, 4),
        }
        del g, e, r, ws
        torch.cuda.empty_cache()
    Ms = 1 << 20
    e = torch.zeros(N, Ms, device=dev)
    run_v = torch.zeros(Ms, dtype=torch.float64, device=dev)
    run_g = torch.zeros(Ms, dtype=torch.float64, device=dev)
    step_err = []
    for _ in range(10):
        g = torch.randn(N, Ms, generator=gen, device=dev) * 1e-3
        exact = g.double().sum(0)
        r = torch.empty_like(g)
        ccgpu.all_reduce_int8_ef(g, e, r)
        torch.cuda.synchronize()
        step_err.append(float((r[0].double() - exact).norm() / exact.norm()))
        run_v += r[0].double()
        run_g += exact
    out["accuracy_f32_1048576"] = {
        "step_norm_rel_err": [round(x, 6) for x in step_err],
        "running_sum_norm_rel_err_after_10": float((run_v - run_g).norm() / run_g.norm()),
        "running_sum_err_norm": float((run_v - run_g).norm()),
        "sum_of_last_accumulators_norm": float(e.double().sum(0).norm())}
    return out


def run_extras(path, dev, N, M, pad_bytes):
    out = {}
    for name, fn in (("pad_sweep", lambda: pad_sweep(N, M, dev)), ("alpha_beta", lambda: alpha_beta(dev)),
                     ("schedules", lambda: schedules(dev, pad_bytes)),
                     ("hierarchical", lambda: hierarchical(dev, pad_bytes)),
                     ("alltoall_variants", lambda: alltoall_variants(dev)), ("int8_ef", lambda: int8_ef(dev))):
        log(f"extras: {name}")
        out[name] = fn()
        with open(path, "w") as f:
            json.dump(out, f, indent=1)


# ---------------------------------------------------------------- rocprofv3 sections

def copy_probe(nbytes, dev):
    """A plain device copy of a known size, 3 times: the kernel whose HBM
    counters scale the profiled kernel's."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def profile_section(name, dev, steps, warmup, pad_bytes=262_144):
    """Run one kernel `steps` times (after `warmup`) for rocprofv3, with the
    workload's own inputs and layout.  Returns (algorithmic bytes per call,
    kernel launches per call): the bytes the kernel must read and write by
    the collective's definition."""
    import numpy as np
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    gen = torch.Generator(device=dev).manual_seed(20261206)
    N, M = 8, 1 << 26
    launches = 1
    if name in ("ring_f32", "ring_bf16"):
        dt = "f32" if name == "ring_f32" else "bf16"
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        x = rank_tensor(N, M, tdt, pad_bytes, dev)
        upload(synth.gradient_inputs(N, M, dt), x)
        y = rank_tensor(N, M, tdt, pad_bytes, dev)
        fn, nbytes = (lambda: ccgpu.all_reduce(x, y)), 2 * N * M * x.element_size()
    elif name == "int32_ring_rot":
        N, M, nsets = 4, 1 << 20, 64
        base = strided_ranks(N, M, torch.int32, dev)
        upload(synth.uniform_int32(synth.W_INT_RING, N, M), base)
        sets = [(base, strided_ranks(N, M, torch.int32, dev))]
        for _ in range(nsets - 1):
            s_ = strided_ranks(N, M, torch.int32, dev)
            s_.copy_(base)
            sets.append((s_, strided_ranks(N, M, torch.int32, dev)))

        def fn():
            for s_, r_ in sets:
                ccgpu.all_reduce(s_, r_)
        nbytes, launches = 2 * N * M * 4 * nsets, nsets
    elif name == "buckets_ring":
        sizes = synth.tensor_sizes_log_uniform()
        host, _, boff, bcnt = bucket_layout(N, sizes, synth.bucket_tensors(N, sizes))
        x = strided_ranks(N, host.shape[1], torch.bfloat16, dev)
        upload(host, x)
        y = strided_ranks(N, host.shape[1], torch.bfloat16, dev)
        fn = lambda: ccgpu.all_reduce_buckets(x, y, boff, bcnt)
        nbytes, launches = 2 * N * sum(bcnt) * 2, (len(boff) + 15) // 16
    elif name in ("rs_ring_n16", "ag_ring_n16"):
        N, M = 16, 1 << 25
        x = strided_ranks(N, M, torch.float32, dev)
        upload(synth.uniform_f32(synth.W_ZERO3, N, M), x)
        sh = strided_ranks(N, M // N, torch.float32, dev)
        ccgpu.reduce_scatter(x, sh)
        if name == "rs_ring_n16":
            fn = lambda: ccgpu.reduce_scatter(x, sh)
        else:
            y = strided_ranks(N, M, torch.float32, dev)
            fn = lambda: ccgpu.all_gather(sh, y)
        nbytes = (N + 1) * M * 4
    elif name == "moe_dropless":
        H = 7168
        C, rows = moe_inputs(N, H=H)
        x = strided_ranks(N, int(C.sum(1).max()) * H, torch.bfloat16, dev)
        upload([r.reshape(-1) for r in rows], x)
        y = strided_ranks(N, int(C.sum(0).max()) * H, torch.bfloat16, dev)
        fn = lambda: ccgpu.all_to_all(x, y, C.tolist(), H)
        nbytes = 2 * int(C.sum()) * H * 2
    elif name in ("hier_2x2x2", "dbt_n8", "hier_8x8", "hier_8x8_ag"):
        pad = pad_bytes
        if name.startswith("hier_8x8"):
            N, M, pad = 64, 1 << 23, 0   # 64 ranks of 32 MiB stream best unpadded
        x = randn_ranks(N, M, gen, dev, pad)
        y = rank_tensor(N, M, torch.float32, pad, dev)
        if name == "dbt_n8":
            fn = lambda: ccgpu.all_reduce(x, y, algo="double_tree")
        else:
            dims = (2, 2, 2) if name == "hier_2x2x2" else (8, 8)
            fn = lambda: ccgpu.all_reduce_hierarchical(x, y, dims)
        # 64 ranks of 32 MiB take the split form: the nested fold stored once
        # (N M reads, M writes), then the AllGather from the owners (M reads,
        # (N - 1) M writes); each launch is profiled against its own bytes
        nbytes = {"hier_8x8": (N + 1) * M * 4, "hier_8x8_ag": N * M * 4}.get(name, 2 * N * M * 4)
    elif name in ("ring_n64", "ring_n64_ag"):
        N, M = 64, 1 << 23
        x = randn_ranks(N, M, gen, dev, 0)
        y = rank_tensor(N, M, torch.float32, 0, dev)
        fn = lambda: ccgpu.all_reduce(x, y)   # the split form: ReduceScatter launch, AllGather launch
        nbytes = (N + 1) * M * 4 if name == "ring_n64" else N * M * 4
    elif name in ("int8_ef_f32", "int8_ef_bf16", "int8_quant_f32", "int8_dequant_f32"):
        tdt = torch.bfloat16 if name == "int8_ef_bf16" else torch.float32
        g = strided_ranks(N, M, tdt, dev)
        g.copy_((torch.randn(N, M, generator=gen, device=dev) * 1e-3).to(tdt))
        e = strided_ranks(N, M, torch.float32, dev).zero_()
        r = strided_ranks(N, M, tdt, dev)
        q = strided_ranks(N, M, torch.int8, dev)
        sc = strided_ranks(N, M // 128, torch.float32, dev)
        if name in ("int8_ef_f32", "int8_ef_bf16"):
            fn, nbytes = (lambda: ccgpu.all_reduce_int8_ef(g, e, r)), N * M * (2 * g.element_size() + 8)
        elif name == "int8_quant_f32":
            fn, nbytes = (lambda: ccgpu.quantize_ef(g, e, q, sc)), N * M * 13 + N * (M // 128) * 4
        else:
            ccgpu.quantize_ef(g, e, q, sc)
            fn, nbytes = (lambda: ccgpu.all_reduce_dequant(q, sc, r)), N * M * 5 + N * (M // 128) * 4
    elif name == "moe_padded_c125":
        H, T, K, E = 7168, 4096, 8, 64
        ch = synth.moe_routing(N, T, E, K)
        Ce = np.stack([np.bincount(c.reshape(-1), minlength=E) for c in ch]).astype(np.int64)
        cap = ccgpu.moe_capacity(1, T, K, E, 5, 4)
        x = torch.randn(N, int(Ce.sum(1).max()) * H, generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty(N, E * cap * H, device=dev, dtype=torch.bfloat16)
        fn = lambda: ccgpu.moe_dispatch_padded(x, y, Ce.tolist(), cap, H)
        nbytes = (int(np.minimum(Ce, cap).sum()) + N * E * cap) * H * 2
        # the copy launches of one call: each step's descriptors in launches of
        # up to 64 (a launch whose descriptors are all empty is skipped)
        recs = ccgpu.all_to_all_plan("moe_dispatch", ccgpu.RankBuf(x.data_ptr(), x.stride(0) * 2),
                                     ccgpu.RankBuf(y.data_ptr(), y.stride(0) * 2), Ce.tolist(), N,
                                     elem_per_row=H, dtype="bf16", nexperts=E, capacity=cap)
        by_step = {}
        for st, _, _, nb in recs:
            by_step.setdefault(st, []).append(nb)
        launches = sum(1 for d in by_step.values() for i in range(0, len(d), 64) if sum(d[i:i + 64]) > 0)
    else:
        raise SystemExit(f"unknown profile section {name}")
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return nbytes, launches


PROFILE_SECTIONS = ("ring_f32, ring_bf16, int32_ring_rot, buckets_ring, rs_ring_n16, ag_ring_n16, moe_dropless, "
                    "hier_2x2x2, hier_8x8, hier_8x8_ag, ring_n64, ring_n64_ag, dbt_n8, int8_ef_f32, int8_ef_bf16, "
                    "int8_quant_f32, int8_dequant_f32, moe_padded_c125")


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ranks", type=int, default=8)
    ap.add_argument("--count", type=int, default=67_108_864)
    ap.add_argument("--dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--algo", default="ring", choices=["ring", "hd", "butterfly"])
    ap.add_argument("--fuse-depth", type=int, default=0)
    ap.add_argument("--pad-bytes", type=int, default=262_144)
    ap.add_argument("--blocks-per-cu", type=int, default=0, help="occupancy cap passed to the library (0 = its default)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle on the host (and with it the parity verdict of the headline)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the records of the other workloads")
    ap.add_argument("--no-twin", action="store_true", help="skip the bf16 twin and the alpha-beta fit")
    ap.add_argument("--extras", default="", metavar="PATH", help="also run the long sweeps and write them to PATH")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="before timing, run a plain device copy of this many bytes 3 times "
                         "(a known-size kernel for scaling HBM counters)")
    ap.add_argument("--profile-section", default="",
                    help="run only this kernel --steps times (for rocprofv3): " + PROFILE_SECTIONS)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the N logical ranks live in one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    from ring_allreduce_reduction_02_amd import ccgpu

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ccgpu.load()
    dev = "cuda:0"
    if args.profile_section:
        if args.copy_probe_bytes:
            copy_probe(args.copy_probe_bytes, dev)
        nbytes, launches = profile_section(args.profile_section, dev, args.steps, args.warmup, args.pad_bytes)
        emit({"profile_section": args.profile_section, "alg_bytes_per_call": nbytes, "launches_per_call": launches,
              "alg_bytes_per_launch": nbytes // launches})
        return

    m = run_headline(args, dev)
    roof = roofline_of(m, args)
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        log("oracle on the host (cpu baseline and parity of the timed output)")
        rec, exp = cpu_baseline(m["xs"], args.dtype)
        parity = all(same_bits(m["got"][r], exp[r]) for r in range(m["N"]))
        cpu = rec
        del exp
    m["xs"] = m["got"] = None
    twin = ab = None
    if not args.no_twin and args.dtype == "f32":
        log("bf16 twin")
        twin = bf16_twin(args, dev)
        log("alpha-beta fit at N=8")
        ab = alpha_beta_n8(dev, args.pad_bytes)
    if not args.no_workloads:
        for name, fn in (("int32 ring", rec_int32_ring), ("small bf16 ring", rec_small_ring), ("buckets", rec_buckets),
                         ("zero3", rec_zero3), ("moe", rec_moe)):
            log(f"workload: {name}")
            emit(fn(dev))
    if args.extras:
        run_extras(args.extras, dev, m["N"], m["M"], args.pad_bytes)
    line = headline_line(make_headline(m, args, roof, twin, ab, cpu, parity))
    print(line, flush=True)


if __name__ == "__main__":
    main()
