"""Seeded synthetic inputs for the collective workloads.

This module only draws random numbers and lays them out; it holds none of the
reduction, scheduling or rounding arithmetic.  Both the tests (for the oracle
and for the HIP library) and the benchmark take their inputs from here.  Every
generator is keyed by numpy.random.default_rng([SEED, workload_id, rank]).

bf16 inputs are produced by drawing float32 samples and converting them with
torch's CPU cast; they are returned as uint16 bit patterns.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

SEED = 20261202

# workload ids (used only to key the random streams)
W_INT_RING = 1        # ring AllReduce SUM, N=4, M=1,048,576 int32
W_GRAD_RING = 2       # ring AllReduce SUM, N=8, M=67,108,864 fp32 (and a bf16 twin)
W_BUCKETS = 3         # bucketed gradient sync, N=8, 120 bf16 tensors
W_ZERO3 = 4           # standalone RS then AG, N=16, M=33,554,432 fp32; int32 MAX/PROD
W_MOE = 5             # MoE AllToAll(v), N=8, 4096 tokens, hidden 7168, top-8 of 64
W_SMALL_RING = 6      # ring AllReduce SUM, N=4, M=131,072 bf16 (small-message case)


def rng(workload: int, rank: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, workload, rank, sub])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 samples -> bf16 bit patterns via torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def uniform_int32(workload: int, N: int, M: int, lo: int = -1000, hi: int = 1000,
                  sub: int = 0) -> List[np.ndarray]:
    """Integers uniform in [lo, hi] inclusive, one array per rank."""
    return [rng(workload, r, sub).integers(lo, hi + 1, size=M, dtype=np.int32) for r in range(N)]


def choice_int32(workload: int, N: int, M: int, values, sub: int = 0) -> List[np.ndarray]:
    vals = np.asarray(values, dtype=np.int32)
    return [vals[rng(workload, r, sub).integers(0, len(vals), size=M)] for r in range(N)]


def gaussian_f32(workload: int, N: int, M: int, sigma: float, sub: int = 0) -> List[np.ndarray]:
    """i.i.d. N(0, sigma^2) float32 samples (sigma is the standard deviation)."""
    out = []
    for r in range(N):
        x = rng(workload, r, sub).standard_normal(M, dtype=np.float32)
        x *= np.float32(sigma)
        out.append(x)
    return out


def uniform_f32(workload: int, N: int, M: int, lo: float = -1.0, hi: float = 1.0,
                sub: int = 0) -> List[np.ndarray]:
    out = []
    for r in range(N):
        x = rng(workload, r, sub).random(M, dtype=np.float32)
        x *= np.float32(hi - lo)
        x += np.float32(lo)
        out.append(x)
    return out


def gradient_inputs(N: int, M: int, dtype: str = "f32", sigma: float = 1e-3,
                    workload: int = W_GRAD_RING) -> List[np.ndarray]:
    """Synthetic gradients: Gaussian float32, or their bf16 rounding."""
    xs = gaussian_f32(workload, N, M, sigma)
    if dtype == "bf16":
        return [to_bf16_bits(x) for x in xs]
    return xs


def tensor_sizes_log_uniform(n: int = 120, lo: int = 4096, hi: int = 16_777_216,
                             workload: int = W_BUCKETS) -> List[int]:
    """floor(exp(U(ln lo, ln hi))) element counts for n tensors."""
    u = rng(workload, 0, 1).uniform(math.log(lo), math.log(hi), size=n)
    return [int(math.floor(math.exp(v))) for v in u]


def bucket_tensors(N: int, sizes: List[int], sigma: float = 1e-2,
                   workload: int = W_BUCKETS) -> List[List[np.ndarray]]:
    """Per rank, per tensor: bf16 bits of N(0, sigma^2) samples."""
    out = []
    for r in range(N):
        g = rng(workload, r, 2)
        row = []
        for n in sizes:
            x = g.standard_normal(n, dtype=np.float32)
            x *= np.float32(sigma)
            row.append(to_bf16_bits(x))
        out.append(row)
    return out


# --------------------------------------------------------------------------
# MoE routing for the AllToAll(v) workload
# --------------------------------------------------------------------------

def moe_routing(N: int = 8, tokens: int = 4096, experts: int = 64, topk: int = 8,
                zipf_s: float = 1.2, workload: int = W_MOE) -> List[np.ndarray]:
    """Per source rank, an int array [tokens, topk] of chosen experts.

    Expert popularity is proportional to (e+1)^-zipf_s; top-k without
    replacement is drawn by adding Gumbel noise to the log-popularities and
    taking the k largest.
    """
    logp = -zipf_s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    out = []
    for r in range(N):
        g = rng(workload, r, 0).gumbel(size=(tokens, experts))
        score = logp[None, :] + g
        top = np.argsort(-score, axis=1, kind="stable")[:, :topk]
        out.append(top.astype(np.int64))
    return out


def moe_send_layout(choice: np.ndarray, N: int, experts: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows of one source rank sorted by (dest rank, local expert, token).

    Returns (rows, counts): rows[k] = (token, slot, expert) of send row k, and
    counts[j] = number of rows for destination rank j.  Expert e lives on rank
    e // (experts // N).
    """
    per_rank = experts // N
    tok = np.repeat(np.arange(choice.shape[0]), choice.shape[1])
    slot = np.tile(np.arange(choice.shape[1]), choice.shape[0])
    exp = choice.reshape(-1)
    dest = exp // per_rank
    order = np.lexsort((tok, exp % per_rank, dest))
    rows = np.stack([tok[order], slot[order], exp[order]], axis=1)
    counts = np.bincount(dest, minlength=N).astype(np.int64)
    return rows, counts


def moe_counts(N: int = 8, tokens: int = 4096, experts: int = 64, topk: int = 8,
               zipf_s: float = 1.2) -> np.ndarray:
    """counts[i][j]: rows source rank i sends to rank j."""
    ch = moe_routing(N, tokens, experts, topk, zipf_s)
    C = np.zeros((N, N), dtype=np.int64)
    for i in range(N):
        _, c = moe_send_layout(ch[i], N, experts)
        C[i] = c
    return C


def moe_payload_rows(src: int, nrows: int, hidden: int, seed_sub: int = 3) -> np.ndarray:
    """bf16 N(0,1) payload, [nrows, hidden] uint16; element 0..2 of each row carry
    a tag (source rank, row index low/high 16 bits) so every row is self-identifying."""
    x = rng(W_MOE, src, seed_sub).standard_normal((nrows, hidden), dtype=np.float32)
    bits = to_bf16_bits(x.reshape(-1)).reshape(nrows, hidden)
    idx = np.arange(nrows, dtype=np.int64)
    bits[:, 0] = np.uint16(src)
    bits[:, 1] = (idx & 0xFFFF).astype(np.uint16)
    bits[:, 2] = ((idx >> 16) & 0xFFFF).astype(np.uint16)
    return bits
