#!/usr/bin/env python
"""Benchmark of the ring AllReduce on one MI355X.

Workload: ring AllReduce SUM of synthetic gradients, N = 8 logical ranks,
M = 67,108,864 fp32 elements per rank (256 MiB each), Gaussian values with
sigma = 1e-3, the rank buffers 64 KiB + 256 B apart.  One step is one
cc_all_reduce call (the fused ring kernel) over inputs already resident in
HBM.  The step's algorithmic traffic is 2*N*M*4 bytes (read every rank's
input once, write every rank's output once).

Prints one JSON line: achieved GB/s (value) and its fraction of the 8 TB/s
HBM peak, the simulated ring busbw, the roofline object of the fused kernel
(with HBM bytes from committed rocprofv3 counters when they match the
current kernel source), the oracle's time on the host cores for a bounded
sample, a bf16 twin and an alpha-beta calibration of the stepwise ring.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) + simulated busbw for N-rank ring AllReduce"
KERNEL_SRC = os.path.join(ROOT, "ring_allreduce_reduction_02_amd", "csrc", "cc_kernels.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "ring_fused_f32_n8_m67108864_pmc.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def rank_stride_bytes(row_bytes):
    """Rank stride for rows of row_bytes: the payload rounded up to a power of
    two P, plus max(32 KiB, P/1024) (equal offsets of the ranks then spread
    over the HBM channels)."""
    p = 256
    while p < row_bytes:
        p *= 2
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
    # sampled in place: a torch copy here would share its kernel with the
    # copy probe whose counters scale the profiles' HBM traffic
    t = rank_tensor(N, M, torch.float32, pad_bytes, device)
    t.normal_(0.0, 1e-3, generator=gen)
    return t


def upload(xs, t):
    import numpy as np
    import torch
    for r, x in enumerate(xs):
        h = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else torch.from_numpy(x)
        t[r].copy_(h, non_blocking=False)


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


def traffic_from_profile(nbytes_alg):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs,
    scaled by the copy-kernel calibration; None if the kernel changed."""
    if not os.path.exists(PMC_FILE):
        return None, "no counter file"
    with open(PMC_FILE) as f:
        p = json.load(f)
    if p.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    fetch = p["fetch_kib_per_dispatch"] * 1024.0 * p["fetch_scale"]
    write = p["write_kib_per_dispatch"] * 1024.0 * p["write_scale"]
    return fetch + write, "rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE (scaled by a plain copy)"


def cpu_baseline(N, M_sample, min_seconds=10.0, max_runs=25):
    """The oracle as it stands, on the host cores: the step-explicit ring
    simulator on the same workload, repeated until at least `min_seconds` of
    CPU work (median run reported)."""
    from oracle import ccsim
    from ring_allreduce_reduction_02_amd import synth
    xs = synth.gradient_inputs(N, M_sample, "f32")
    times = []
    t_all = time.perf_counter()
    while len(times) < max_runs and (time.perf_counter() - t_all < min_seconds or len(times) < 3):
        t = time.perf_counter()
        ccsim.ring_all_reduce(xs, "sum", "f32")
        times.append(time.perf_counter() - t)
    t = sorted(times)[len(times) // 2]
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": 2 * N * M_sample * 4 / t / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"ring AllReduce SUM, N={N}, M={M_sample} fp32 per rank, step-explicit NumPy simulator "
                  f"(single-threaded elementwise ops), {len(times)} runs in {sum(times):.1f} s, median {t:.3f} s",
        "host_logical_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "cpu_model": cpu_model or platform.processor(),
    }


def pad_sweep(src, N, M, dev, pads=(0, 65_792, 262_144, 2_097_152), steps=10):
    """The headline AllReduce with rank buffers `pad` bytes apart beyond the
    payload (same data, copied on the device)."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu
    res = {}
    for pad in pads:
        s = rank_tensor(N, M, src.dtype, pad, dev)
        r = rank_tensor(N, M, src.dtype, pad, dev)
        s.copy_(src)
        t = time_launches(lambda: ccgpu.all_reduce(s, r), steps, 3)
        per = sorted(t["per_launch_ms"])
        ms = per[len(per) // 2]
        res[str(pad)] = {"median_launch_ms": round(ms, 5), "min_launch_ms": round(per[0], 5),
                         "GBps": round(2 * N * M * src.element_size() / ms / 1e6, 1)}
        del s, r
        torch.cuda.empty_cache()
    return res


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


def alpha_beta(dev, ranks=(4, 8, 16), max_bytes=1 << 30):
    """Stepwise ring AllReduce (fp32 SUM) at N = 4, 8, 16 over per-rank sizes
    4 KiB .. 1 GiB (x4), GPU time from HIP-graph replays, in two variants:
    one kernel per ring step, and all steps in one cooperative launch with a
    grid barrier between steps.  Fits T = alpha * 2(N-1) + beta * bytes sent
    per rank per N, and over all N together with a per-call constant t0
    (T = t0 + alpha * steps + beta * bytes).  The fused kernel's
    T = t0 + bytes / BW is fitted on the same sizes."""
    import torch

    from ring_allreduce_reduction_02_amd import calib, ccgpu
    sizes = [m for m in (1 << k for k in range(10, 29, 2)) if m * 4 <= max_bytes]
    gen = torch.Generator(device=dev).manual_seed(20261202)
    out = {"schedule": "ring AllReduce, fp32 SUM, fuse_depth=1 (one ring step per pass)",
           "variants": {"kernel_per_step": "one kernel launch per ring step",
                        "grid_barrier": "one cooperative launch, grid barrier between ring steps"},
           "per_n": {}}
    glob = {"kernel_per_step": ([], [], []), "grid_barrier": ([], [], [])}
    for N in ranks:
        # rank rows by the stride rule (1 GiB + 1 MiB): a stride of exactly
        # 1 GiB puts every rank's same offset on the same HBM channels
        send = strided_ranks(N, sizes[-1], torch.float32, dev)
        send.copy_(torch.randn(N, sizes[-1], generator=gen, device=dev) * 1e-3)
        recv = strided_ranks(N, sizes[-1], torch.float32, dev)
        ws = ccgpu.make_workspace("all_reduce", N, sizes[-1], "f32", "ring", 1, dev, grid_sync=True)
        # steady clocks before the smallest, most clock-sensitive points
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
        timed_out = ccgpu.grid_sync_timed_out(ws)
        out["per_n"][str(N)] = {
            "kernel_per_step": calib.fit_alpha_beta(st, by, t_ks),
            "grid_barrier": calib.fit_alpha_beta(st, by, t_gb),
            "fused": calib.fit_fixed_plus_bandwidth(fb, ft),
            "points": pts,
            "timing": sorted(how),
            "barrier_timed_out": timed_out,
        }
        for key, ts in (("kernel_per_step", t_ks), ("grid_barrier", t_gb)):
            glob[key][0].extend(st); glob[key][1].extend(by); glob[key][2].extend(ts)
        del send, recv, ws
        torch.cuda.empty_cache()
    out["all_n"] = {k: calib.fit_launch_alpha_beta(*v) for k, v in glob.items()}
    return out


def _avg_ms(fn, steps=10, warmup=3):
    r = time_steps(fn, steps, warmup)
    return r["total_ms"] / steps


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
    # the headline's layout: 256 MiB rows, `pad_bytes` apart
    send = randn_ranks(N, M, gen, dev, pad_bytes)
    recv = rank_tensor(N, M, torch.float32, pad_bytes, dev)
    for algo in ("ring", "hd", "butterfly", "tree", "double_tree", "ring_2port"):
        ms = _avg_ms(lambda: ccgpu.all_reduce(send, recv, algo=algo), 10, 3)
        out["fused"][f"{algo}_n8"] = {"ms": round(ms, 4), "GBps": round(2 * N * M * 4 / ms / 1e6, 1)}
    del send, recv
    torch.cuda.empty_cache()
    N12, M12 = 12, 1 << 25
    send = torch.randn(N12, M12, generator=gen, device=dev) * 1e-3
    recv = torch.empty_like(send)
    for algo in ("hd", "butterfly"):
        ms = _avg_ms(lambda: ccgpu.all_reduce(send, recv, algo=algo), 10, 3)
        out["fused"][f"{algo}_n12_pair_folded"] = {"ms": round(ms, 4), "GBps": round(2 * N12 * M12 * 4 / ms / 1e6, 1)}
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
            key = "x".join(map(str, dims))
            out["fused"][key] = {"ms": round(ms, 4), "GBps": round(2 * N * M * 4 / ms / 1e6, 1)}
        del send, recv
        torch.cuda.empty_cache()

    sizes = [1 << k for k in range(10, 25, 2)]          # 1 Ki .. 16 Mi fp32 = 4 KiB .. 64 MiB per rank
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
    out["dropless_direct"] = {"ms": round(ms, 4), "GBps": round(moved / ms / 1e6, 1), "wire_rows": int(C.sum())}
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
            r[f"dispatch_{name}"] = {"ms": round(ms, 4), "GBps": round(d_moved / ms / 1e6, 1)}
        ms = _avg_ms(lambda: ccgpu.moe_combine_padded(exp, send, Ce.tolist(), cap, H))
        r["combine_direct"] = {"ms": round(ms, 4), "GBps": round(c_moved / ms / 1e6, 1)}
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
            "ms": round(ms, 4), "GBps_moved": round(moved_h / ms / 1e6, 1),
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
        g = (torch.randn(N, M, generator=gen, device=dev) * 1e-3).to(tdt)
        e = torch.zeros(N, M, device=dev)
        r = torch.empty_like(g)
        ms_f = _avg_ms(lambda: ccgpu.all_reduce_int8_ef(g, e, r, fuse_depth=0))
        ws = torch.empty(ccgpu.int8_ef_workspace_size(N, M, dtype, 1), dtype=torch.uint8, device=dev)
        ms_2 = _avg_ms(lambda: ccgpu.all_reduce_int8_ef(g, e, r, fuse_depth=1, workspace=ws))
        ms_p = _avg_ms(lambda: ccgpu.all_reduce(g, r, algo="ring"))
        fused_bytes = N * M * (2 * es + 8)
        two_bytes = N * M * (es + 8) + 2 * N * ccgpu.int8_message_bytes(M) + N * M * es
        out[dtype] = {
            "fused_ms": round(ms_f, 4), "fused_GBps": round(fused_bytes / ms_f / 1e6, 1),
            "fused_pct_of_peak": round(100 * fused_bytes / ms_f / 1e6 / PEAK_HBM_GBPS, 2),
            "two_kernel_ms": round(ms_2, 4), "two_kernel_GBps": round(two_bytes / ms_2 / 1e6, 1),
            "plain_ring_ms": round(ms_p, 4),
        }
        del g, e, r, ws
        torch.cuda.empty_cache()
    # accuracy over steps (float32 gradients, 1,048,576 per rank)
    Ms = 1 << 20
    e = torch.zeros(N, Ms, device=dev)
    run_v = torch.zeros(Ms, dtype=torch.float64, device=dev)
    run_g = torch.zeros(Ms, dtype=torch.float64, device=dev)
    step_err = []
    for t in range(10):
        g = torch.randn(N, Ms, generator=gen, device=dev) * 1e-3
        exact = g.double().sum(0)
        r = torch.empty_like(g)
        ccgpu.all_reduce_int8_ef(g, e, r)
        torch.cuda.synchronize()
        step_err.append(float((r[0].double() - exact).norm() / exact.norm()))
        run_v += r[0].double()
        run_g += exact
    resid = float(e.double().sum(0).norm())
    out["accuracy_f32_1048576"] = {
        "step_norm_rel_err": [round(x, 6) for x in step_err],
        "running_sum_norm_rel_err_after_10": float((run_v - run_g).norm() / run_g.norm()),
        "running_sum_err_norm": float((run_v - run_g).norm()), "sum_of_last_accumulators_norm": resid}
    return out


def norm_rel_err_fp64(send, recv, offsets, counts, step=1 << 24):
    """max over ranks of ||y_r - y64|| / ||y64|| over the given element
    ranges, y64 = the order-free fp64 sum of the inputs (a measurement of the
    output, computed with torch on the device in slices)."""
    import torch
    N = send.shape[0]
    num = torch.zeros(N, dtype=torch.float64, device=send.device)
    den = torch.zeros((), dtype=torch.float64, device=send.device)
    for o, c in zip(offsets, counts):
        for a in range(o, o + c, step):
            e = min(a + step, o + c)
            y64 = send[:, a:e].to(torch.float64).sum(0)
            num += ((recv[:, a:e].to(torch.float64) - y64) ** 2).sum(1)
            den += (y64 ** 2).sum()
    return float((num / den).sqrt().max().item())


def workloads(dev):
    """The other workloads, timed with inputs resident in HBM (inputs drawn on
    the device; their parity is checked by the tests).  GB/s = algorithmic
    bytes / time."""
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    out = {}
    gen = torch.Generator(device=dev).manual_seed(synth.SEED)

    # int32 ring AllReduce, N=4, M=1,048,576 (32 MiB per call): one buffer set
    # (cache-resident) and 64 rotating sets (2 GiB, beyond the 256 MB cache)
    N, M = 4, 1 << 20
    nsets = 64
    sets = [(torch.randint(-1000, 1001, (N, M), generator=gen, device=dev, dtype=torch.int32),
             torch.empty(N, M, device=dev, dtype=torch.int32)) for _ in range(nsets)]
    alg = 2 * N * M * 4
    ms1 = time_graph(lambda: ccgpu.all_reduce(sets[0][0], sets[0][1]), 10, 32)

    def rot():
        for s_, r_ in sets:
            ccgpu.all_reduce(s_, r_)
    msr = time_graph(rot, 10, 1) / nsets
    host = _avg_ms(lambda: ccgpu.all_reduce(sets[0][0], sets[0][1]), 50, 10)
    out["int32_ring_n4_m1048576"] = {"same_set_us": round(ms1 * 1e3, 2), "same_set_GBps": round(alg / ms1 / 1e6, 1),
                                     "rotating_2GiB_us": round(msr * 1e3, 2),
                                     "rotating_2GiB_GBps": round(alg / msr / 1e6, 1),
                                     "eager_python_call_us": round(host * 1e3, 2),
                                     "timing": "HIP-graph replays (GPU time); eager figure includes host launch cost"}
    del sets
    torch.cuda.empty_cache()

    # bucketed bf16 gradient sync, N=8, 120 tensors in 25 MiB buckets
    N = 8
    sizes = synth.tensor_sizes_log_uniform()
    _, _, boff, bcnt = ccgpu.bucket_plan(sizes, 2, 25 * 1024 * 1024, 128)
    extent = boff[-1] + bcnt[-1]
    send = strided_ranks(N, extent, torch.bfloat16, dev)
    send.copy_((torch.randn(N, extent, generator=gen, device=dev) * 1e-2).to(torch.bfloat16))
    recv = strided_ranks(N, extent, torch.bfloat16, dev)
    alg = 2 * N * sum(bcnt) * 2
    b = {"tensors": len(sizes), "buckets": len(boff), "elements_per_rank": sum(bcnt),
         "rank_stride_bytes": rank_stride_bytes(extent * 2)}
    for algo in ("ring", "hd", "butterfly"):
        ms = _avg_ms(lambda: ccgpu.all_reduce_buckets(send, recv, boff, bcnt, algo=algo))
        b[algo] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1),
                   "max_norm_rel_err_vs_fp64": norm_rel_err_fp64(send, recv, boff, bcnt)}
    ms = _avg_ms(lambda: [ccgpu.all_reduce(send[:, o:o + c], recv[:, o:o + c]) for o, c in zip(boff, bcnt)], 5, 2)
    b["ring_one_launch_per_bucket"] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1)}
    out["bucketed_bf16_n8"] = b
    del send, recv
    torch.cuda.empty_cache()

    # ZeRO-3 style standalone ReduceScatter then AllGather, N=16, M=33,554,432 fp32
    N, M = 16, 1 << 25
    S = M // N
    send = strided_ranks(N, M, torch.float32, dev)
    send.uniform_(-1.0, 1.0, generator=gen)
    shard = strided_ranks(N, S, torch.float32, dev)
    full = strided_ranks(N, M, torch.float32, dev)
    alg = (N + 1) * M * 4
    z = {"rank_stride_bytes": [rank_stride_bytes(M * 4), rank_stride_bytes(S * 4)]}
    for algo in ("ring", "hd"):
        ms = _avg_ms(lambda: ccgpu.reduce_scatter(send, shard, algo=algo))
        z[f"reduce_scatter_{algo}"] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1)}
    ms = _avg_ms(lambda: ccgpu.all_gather(shard, full))
    z["all_gather"] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1)}
    out["zero3_rs_ag_n16_m33554432_f32"] = z
    del send, shard, full
    torch.cuda.empty_cache()

    # MoE AllToAll(v) dispatch and combine, N=8, 4096 tokens, top-8 of 64, hidden 7168 bf16
    N, H = 8, 7168
    C = synth.moe_counts(N)
    Ls, Lr = int(C.sum(1).max()), int(C.sum(0).max())
    send = torch.randn(N, Ls * H, generator=gen, device=dev).to(torch.bfloat16)
    recv = torch.empty(N, Lr * H, device=dev, dtype=torch.bfloat16)
    alg = 2 * int(C.sum()) * H * 2
    m = {"rows_received": C.sum(0).tolist(), "skew_max_over_mean": round(float(C.sum(0).max() / C.sum(0).mean()), 3)}
    for fd, name in ((0, "direct"), (1, "pairwise")):
        ms = _avg_ms(lambda: ccgpu.all_to_all(send, recv, C.tolist(), H, fuse_depth=fd))
        m[f"dispatch_{name}"] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1)}
    ms = _avg_ms(lambda: ccgpu.all_to_all(recv, send, C.T.tolist(), H))
    m["combine_direct"] = {"ms": round(ms, 4), "GBps": round(alg / ms / 1e6, 1)}
    out["moe_alltoall_n8_t4096_h7168_bf16"] = m
    del send, recv
    torch.cuda.empty_cache()
    return out


def profile_section(name, dev, steps, warmup, pad_bytes=262_144):
    """Run one kernel of the next-row schedules `steps` times (after `warmup`)
    for rocprofv3, and return its algorithmic bytes per call: the kernel's
    HBM reads and writes by the schedule's definition."""
    import numpy as np
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth
    gen = torch.Generator(device=dev).manual_seed(20261206)
    N, M = 8, 1 << 26
    if name in ("hier_2x2x2", "dbt_n8", "hier_8x8"):
        pad = pad_bytes
        if name == "hier_8x8":
            N, M, pad = 64, 1 << 23, 0   # 64 ranks of 32 MiB stream best unpadded
        x = randn_ranks(N, M, gen, dev, pad)
        y = rank_tensor(N, M, torch.float32, pad, dev)
        if name == "dbt_n8":
            fn = lambda: ccgpu.all_reduce(x, y, algo="double_tree")
        else:
            dims = (2, 2, 2) if name == "hier_2x2x2" else (8, 8)
            fn = lambda: ccgpu.all_reduce_hierarchical(x, y, dims)
        nbytes = 2 * N * M * 4
    elif name in ("int8_ef_f32", "int8_quant_f32", "int8_dequant_f32"):
        g = torch.randn(N, M, generator=gen, device=dev) * 1e-3
        e = torch.zeros(N, M, device=dev)
        r = torch.empty_like(g)
        q = torch.empty(N, M, dtype=torch.int8, device=dev)
        sc = torch.empty(N, M // 128, device=dev)
        ccgpu.quantize_ef(g, e, q, sc)
        if name == "int8_ef_f32":
            fn, nbytes = (lambda: ccgpu.all_reduce_int8_ef(g, e, r)), N * M * 16
        elif name == "int8_quant_f32":
            fn, nbytes = (lambda: ccgpu.quantize_ef(g, e, q, sc)), N * M * 13 + N * (M // 128) * 4
        else:
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
    else:
        raise SystemExit(f"unknown profile section {name}")
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return nbytes


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
    ap.add_argument("--cpu-sample", type=int, default=67_108_864)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bf16 twin, the alpha-beta calibration and the other workloads")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="before timing, run a plain device copy of this many bytes 3 times "
                         "(a known-size kernel for scaling HBM counters)")
    ap.add_argument("--profile-section", default="",
                    help="run only this kernel of the next-row schedules --steps times (for rocprofv3): "
                         "hier_2x2x2, hier_8x8, dbt_n8, int8_ef_f32, int8_quant_f32, int8_dequant_f32, "
                         "moe_padded_c125")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the N logical ranks live in one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from ring_allreduce_reduction_02_amd import ccgpu, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ccgpu.load()
    dev = "cuda:0"
    if args.profile_section:
        if args.copy_probe_bytes:
            a = torch.empty(args.copy_probe_bytes, dtype=torch.uint8, device=dev).fill_(1)
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        nbytes = profile_section(args.profile_section, dev, args.steps, args.warmup, args.pad_bytes)
        print(json.dumps({"profile_section": args.profile_section, "alg_bytes_per_call": nbytes}), flush=True)
        return
    N, M = args.ranks, args.count
    tdt = torch.float32 if args.dtype == "f32" else torch.bfloat16
    es = 4 if args.dtype == "f32" else 2
    log(f"generating {N} x {M} {args.dtype} synthetic gradients")
    xs = synth.gradient_inputs(N, M, args.dtype)
    send = rank_tensor(N, M, tdt, args.pad_bytes, dev)
    recv = rank_tensor(N, M, tdt, args.pad_bytes, dev)
    upload(xs, send)
    del xs
    ws = ccgpu.make_workspace("all_reduce", N, M, args.dtype, args.algo, args.fuse_depth, dev)
    if args.copy_probe_bytes:
        a = torch.empty(args.copy_probe_bytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step():
        ccgpu.all_reduce(send, recv, op="sum", algo=args.algo, fuse_depth=args.fuse_depth, workspace=ws,
                         blocks_per_cu=args.blocks_per_cu)

    log("timing")
    # the K timed steps run back to back; the per-launch durations behind the
    # roofline come from a second, instrumented pass of K launches (an event
    # pair around every launch adds about 5 us per step to the first)
    res = time_steps(step, args.steps, args.warmup)
    ms_per_step = res["total_ms"] / args.steps
    alg_bytes = 2 * N * M * es
    value = alg_bytes / (ms_per_step / 1e3) / 1e9
    per = time_launches(step, args.steps, 2)["per_launch_ms"]
    avg_launch_ms = sum(per) / len(per)
    achieved = alg_bytes / (avg_launch_ms / 1e3) / 1e9
    busbw = (M * es) / (ms_per_step / 1e3) * 2 * (N - 1) / N / 1e9
    traffic, traffic_src = traffic_from_profile(alg_bytes)
    kname = {"ring": "k_ring_fused", "hd": "k_tree_fused", "butterfly": "k_tree_fused"}[args.algo]
    if args.fuse_depth:
        kname = "stepwise schedule (several kernels per step)"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
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
            "blocks_per_cu": args.blocks_per_cu,
            "rank_stride_bytes": send.stride(0) * es,
            "values": "Gaussian, sigma=1e-3" + (" (bf16 rounding of the fp32 samples)" if args.dtype == "bf16" else ""),
            "parallelism": f"{N} logical ranks in one GPU's HBM",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "busbw_GBps": round(busbw, 2),
        "algorithmic_bytes_per_step": alg_bytes,
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "traffic_over_algorithmic": round(traffic / alg_bytes, 4) if traffic else None,
            "avg_launch_ms": round(avg_launch_ms, 5),
            "median_launch_ms": round(sorted(per)[len(per) // 2], 5),
            "min_launch_ms": round(min(per), 5),
        },
    }
    if not args.no_extras and args.dtype == "f32" and args.algo == "ring" and args.fuse_depth == 0:
        log("rank-stride pad sweep")
        out["pad_sweep"] = pad_sweep(send, N, M, dev)
        log("bf16 twin")
        xb = synth.gradient_inputs(N, M, "bf16")
        sb = rank_tensor(N, M, torch.bfloat16, args.pad_bytes, dev)
        rb = rank_tensor(N, M, torch.bfloat16, args.pad_bytes, dev)
        upload(xb, sb)
        del xb
        rb16 = time_steps(lambda: ccgpu.all_reduce(sb, rb, algo="ring", fuse_depth=0), args.steps, args.warmup)
        ms16 = rb16["total_ms"] / args.steps
        out["bf16_twin"] = {"ms_per_step": round(ms16, 5),
                            "GBps": round(2 * N * M * 2 / (ms16 / 1e3) / 1e9, 2),
                            "pct_of_peak": round(100 * 2 * N * M * 2 / (ms16 / 1e3) / 1e9 / PEAK_HBM_GBPS, 2)}
        del sb, rb
        torch.cuda.empty_cache()
        del send, recv, ws
        torch.cuda.empty_cache()
        log("alpha-beta calibration")
        out["alpha_beta"] = alpha_beta(dev)
        log("other workloads")
        out["workloads"] = workloads(dev)
        log("schedules")
        out["schedules"] = schedules(dev, args.pad_bytes)
        log("hierarchical")
        out["hierarchical"] = hierarchical(dev, args.pad_bytes)
        log("alltoall variants")
        out["alltoall_variants"] = alltoall_variants(dev)
        log("int8 error feedback")
        out["int8_ef"] = int8_ef(dev)
    if not args.no_cpu_baseline:
        log("oracle on the host")
        out["cpu_baseline"] = cpu_baseline(N, min(args.cpu_sample, M))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
