"""alpha-beta calibration of a schedule on this GPU.

The pages model a step as a fixed cost plus a per-byte cost and ask that the
model be fitted on the same collective, dtype, rank count and algorithm that
is being predicted (textbook ch. 6 "集合通信", section "绘制地形图：网络性能建模";
lesson 3, "理论通信量与网络延迟模型", where beta is seconds per byte).  Here a
"step" is one ring step of the stepwise schedule and a "byte" is one byte a
rank sends on the simulated ring, so

    T = alpha * steps + beta * bytes_sent_per_rank

is fitted by non-negative least squares.  n* = alpha / beta is the message
size (bytes per rank and step) at which the two terms are equal.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np


def fit_alpha_beta(steps: Sequence[float], bytes_sent: Sequence[float], seconds: Sequence[float]) -> Dict[str, float]:
    from scipy.optimize import nnls

    A = np.stack([np.asarray(steps, dtype=np.float64), np.asarray(bytes_sent, dtype=np.float64)], axis=1)
    t = np.asarray(seconds, dtype=np.float64)
    # weight each point by 1/t so small and large messages count alike
    w = 1.0 / t
    sol, _ = nnls(A * w[:, None], t * w)
    alpha, beta = float(sol[0]), float(sol[1])
    pred = A @ sol
    return {
        "alpha_us_per_step": alpha * 1e6,
        "beta_ps_per_byte": beta * 1e12,
        "link_GBps": (1.0 / beta / 1e9) if beta > 0 else float("inf"),
        "n_star_bytes": alpha / beta if beta > 0 else float("inf"),
        "max_rel_residual": float(np.max(np.abs(pred - t) / t)),
    }


def fit_fixed_plus_bandwidth(bytes_moved: Sequence[float], seconds: Sequence[float]) -> Dict[str, float]:
    """T = t0 + bytes / BW for a fused launch (least squares, 1/t weights)."""
    from scipy.optimize import nnls

    b = np.asarray(bytes_moved, dtype=np.float64)
    t = np.asarray(seconds, dtype=np.float64)
    A = np.stack([np.ones_like(b), b], axis=1)
    w = 1.0 / t
    sol, _ = nnls(A * w[:, None], t * w)
    return {"t0_us": float(sol[0]) * 1e6, "bw_GBps": (1.0 / sol[1] / 1e9) if sol[1] > 0 else float("inf")}


def fit_launch_alpha_beta(steps: Sequence[float], bytes_sent: Sequence[float],
                          seconds: Sequence[float]) -> Dict[str, float]:
    """T = t0 + alpha * steps + beta * bytes_sent_per_rank: the same model with a
    per-call constant (the launch of a schedule that runs all its steps in
    one kernel).  t0 and alpha separate only when the points span several
    step counts (several rank counts N)."""
    from scipy.optimize import nnls

    n = np.asarray(steps, dtype=np.float64)
    b = np.asarray(bytes_sent, dtype=np.float64)
    t = np.asarray(seconds, dtype=np.float64)
    A = np.stack([np.ones_like(n), n, b], axis=1)
    w = 1.0 / t
    sol, _ = nnls(A * w[:, None], t * w)
    t0, alpha, beta = (float(v) for v in sol)
    pred = A @ sol
    return {
        "t0_us": t0 * 1e6,
        "alpha_us_per_step": alpha * 1e6,
        "beta_ps_per_byte": beta * 1e12,
        "link_GBps": (1.0 / beta / 1e9) if beta > 0 else float("inf"),
        "n_star_bytes": alpha / beta if beta > 0 else float("inf"),
        "max_rel_residual": float(np.max(np.abs(pred - t) / t)),
    }


def ring_tree_crossover(N: int, alpha: float, beta_s_per_byte: float) -> Dict[str, float]:
    """Per-rank message size (bytes) at which the ring and the tree AllReduce
    models take equal time (textbook ch. 6, "算法切换点"):
    2(N-1) a + 2 (N-1)/N M b = 2 log2(N) a + 2 log2(N) M b solved for M
    ('exact'), and the large-N forms N a / (b log2 N) ('log') and N a / b
    ('rough') the passage simplifies it to."""
    import math
    lg = math.log2(N)
    den = (2 * lg - 2.0 * (N - 1) / N) * beta_s_per_byte
    exact = (2 * (N - 1) - 2 * lg) * alpha / den if den > 0 else float("inf")
    return {"exact": exact, "log": N * alpha / beta_s_per_byte / lg, "rough": N * alpha / beta_s_per_byte}


def multidim_time(M_bytes: float, dims: Sequence[int], alphas: Sequence[float],
                  betas: Sequence[float]) -> List[float]:
    """Per-level time of the hierarchical AllReduce (AllReduce notes, 算法五,
    BlueConnect cost): level i runs 2 (p_i - 1) steps of latency alpha_i and
    sends 2 (p_i - 1) / p_i of the M / (p_0 ... p_(i-1)) bytes it works on at
    beta_i seconds per byte.  The flat ring is the one-level case."""
    out, shard = [], float(M_bytes)
    for p, a, b in zip(dims, alphas, betas):
        out.append(2 * (p - 1) * a + 2 * (p - 1) / p * shard * b)
        shard /= p
    return out


def pairwise_time(step_max_bytes: Sequence[float], alpha: float, beta: float) -> float:
    """Pairwise AllToAll time (blog, Pairwise performance model): steps
    k = 1..N-1 each cost alpha + beta * (largest block of the step);
    step_max_bytes[k] is that block for k = 0..N-1 (step 0, the local block,
    is not a transfer)."""
    return sum(alpha + beta * float(b) for b in list(step_max_bytes)[1:])
