"""compress -- plain CPU reference of block-wise INT8 gradient compression with
error feedback, and of the AllReduce of the compressed contributions.

TEST INFRASTRUCTURE ONLY.  Like oracle/ccsim.py, this module is what the HIP
library is checked against: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does,
and it imports nothing from the product (it builds on oracle/ccsim.py alone).

Page key: [MLSys-6] = MLSys textbook vol. 2, ch. 6 "集合通信" (gptbert.com),
sections "量化：降低精度" (INT8: s = max|g| / 127, g_int8 = round(g / s),
reconstruction g_int8 * s), "梯度通信的分块量化" (one scale per block of
b_block elements, message d + 4 d / b_block bytes, ratio 4 b / (b + 4) = 3.88
at 128, error at most s_b / 2), and "错误反馈与残差累积" (e_(t+1) = g_t + e_t -
v_t, Definition 1.4, the telescoping sum, Tables 3 and 4).

Arithmetic is float32 throughout, one IEEE operation at a time:
  u = g + e;  m = max over the block of |u|;  s = m / 127;
  q = round_half_even(u / s) clamped to [-127, 127] (q = 0 when s = 0);
  v = q * s;  e_next = u - v.
bf16 gradients are widened exactly to float32 first.  Readings (the passages
do not fix them): round() is round-half-to-even; blocks run from element 0 of
each rank's vector, the last one possibly short; an all-zero block has scale
0 and sends zeros.

Pins: tests/test_oracle_compress.py.
"""
from __future__ import annotations

from typing import Callable, List, Sequence, Tuple

import numpy as np

from oracle import ccsim as cs

QMAX = 127


def block_scales(u: np.ndarray, block: int) -> np.ndarray:
    """s_b = max_{i in b} |u_i| / 127 in float32, one per block of `block`
    elements ([MLSys-6] 分块量化)."""
    u = np.asarray(u, dtype=np.float32)
    nb = -(-u.size // block)
    out = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        seg = u[b * block:(b + 1) * block]
        m = np.float32(np.max(np.abs(seg))) if seg.size else np.float32(0)
        out[b] = np.float32(m) / np.float32(QMAX)
    return out


def quantize(u: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """q_i = round(u_i / s_b) as int8 ([MLSys-6] 量化: g_int8 = round(g / s))."""
    u = np.asarray(u, dtype=np.float32)
    s = np.repeat(np.asarray(scales, dtype=np.float32), block)[:u.size]
    q = np.zeros(u.size, dtype=np.float32)
    nz = s != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q[nz] = np.rint(u[nz] / s[nz])
    return np.clip(q, -QMAX, QMAX).astype(np.int8)


def dequantize(q: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """The receiver's reconstruction g_hat = g_int8 * s (float32)."""
    s = np.repeat(np.asarray(scales, dtype=np.float32), block)[:np.asarray(q).size]
    return (np.asarray(q).astype(np.float32) * s).astype(np.float32)


def ef_compress(g: np.ndarray, e: np.ndarray, block: int, dtype: str = "f32"
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """One error-feedback compression ([MLSys-6] Definition 1.4,
    e_(t+1) = g_t + e_t - v_t): returns (q, scales, v, e_next)."""
    gf = cs.to_acc(g, dtype) if dtype == "bf16" else np.asarray(g, dtype=np.float32)
    u = (gf + np.asarray(e, dtype=np.float32)).astype(np.float32)
    s = block_scales(u, block)
    q = quantize(u, s, block)
    v = dequantize(q, s, block)
    return q, s, v, (u - v).astype(np.float32)


def compressed_all_reduce(gs: Sequence[np.ndarray], es: Sequence[np.ndarray], block: int = 128,
                          dtype: str = "f32") -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """AllReduce (SUM) of the compressed contributions: every rank compresses
    g_r + e_r with its own error feedback, and the dequantized contributions
    v_r are summed in the ring AllReduce's fold order in float32
    (ccsim.ring_all_reduce); a bf16 result is rounded once at the end.
    Returns (outputs, next error accumulators)."""
    vs, enext = [], []
    for g, e in zip(gs, es):
        _, _, v, en = ef_compress(g, e, block, dtype)
        vs.append(v)
        enext.append(en)
    out = cs.ring_all_reduce(vs, "sum", "f32")
    if dtype == "bf16":
        out = [cs.f32_to_bf16_bits(o) for o in out]
    return out, enext


def all_reduce_of_messages(qs: Sequence[np.ndarray], ss: Sequence[np.ndarray], block: int = 128,
                           dtype: str = "f32") -> List[np.ndarray]:
    """The reduction side alone: dequantize every rank's message and sum in the
    ring AllReduce's order."""
    vs = [dequantize(q, s, block) for q, s in zip(qs, ss)]
    out = cs.ring_all_reduce(vs, "sum", "f32")
    if dtype == "bf16":
        out = [cs.f32_to_bf16_bits(o) for o in out]
    return out


def message_bytes(d: int, block: int) -> int:
    """INT8 values plus one float32 scale per block: d + 4 ceil(d / b)."""
    return d + 4 * (-(-d // block))


def compression_ratio(block: int) -> float:
    """4 d / (d + 4 d / b) = 4 b / (b + 4) against float32 ([MLSys-6] 分块量化)."""
    return 4.0 * block / (block + 4)


def threshold_compressor(x: float, thr: float = 0.5) -> float:
    """The greedy 1-bit compressor of [MLSys-6] Tables 3 and 4: sends 1 when
    the value reaches the threshold, else 0."""
    return 1.0 if x >= thr else 0.0


def ef_trace(gs: Sequence[float], compressor: Callable[[float], float], feedback: bool = True
             ) -> List[Tuple[float, float, float, float, float, float]]:
    """Rows (g_t, e_t, g_t + e_t, v_t, e_(t+1), cumulative v) of the scalar
    trace of [MLSys-6] Table 4 (feedback) or Table 3 (feedback=False: e stays
    0 and the compressor sees g_t alone)."""
    rows, e, cum = [], 0.0, 0.0
    for g in gs:
        x = g + e if feedback else g
        v = compressor(x)
        en = x - v if feedback else 0.0
        cum += v
        rows.append((g, e, x, v, en, cum))
        e = en
    return rows
