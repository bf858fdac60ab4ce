"""ccsim -- a plain, slow, step-by-step CPU simulator of the collective schedules.

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP library is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path (the C-ABI library and its
Python binding) never does, and this module imports nothing from the product.
It shares no code, table or constant generator with the HIP path.

Every function below follows a passage of the source pages, cited by page
title and section.  Page keys used in the comments:

  [MLSys-6]  MLSys textbook vol. 2, ch. 6 "集合通信" (gptbert.com)
  [Slides]   "集合通信与分片矩阵乘法" slide deck (hs-black.github.io)
  [AR-notes] "AllReduce" algorithm notes (t6page.pages.dev)
  [Lesson3]  "第 3 课：分布式通信原语" course lesson (hsthanb4.github.io)
  [Blog]     "分布式大模型集合通信" blog post (bowenei.github.io)

Conventions (see each function for the passage it follows):

* N logical ranks; each rank r holds a 1-D array x_r of M elements.
* Chunk c of a rank's vector is [b_c, b_{c+1}) with b_c = floor(c*M/N).  The
  pages split evenly and require N | M ([Lesson3], simulator exercise); floor
  boundaries are the plain generalisation and agree with the even split
  whenever N divides M.
* Element types: "int32" (two's-complement wrap for SUM and PROD), "f32",
  and "bf16" carried as uint16 bit patterns.  bf16 inputs are widened exactly
  to float32, every partial result stays float32 across all steps, and the
  final value is rounded once to bf16 (round to nearest, ties to even).
* A step that combines data does  acc_local = op(acc_local, incoming)  with a
  snapshot of everything sent in that step taken before any rank updates
  ([Lesson3], reference answer: the sends of one step are copied first so
  that no rank reads data another rank already updated in the same step).
* Float MAX is the IEEE-754-2019 "maximum": NaN if either operand is NaN,
  +0 counts as larger than -0.  It is commutative and associative, so every
  schedule reaches the same bits; SUM and PROD are not associative in floating
  point ([MLSys-6], "六种核心原语": different schedules change the low bits),
  which is why this simulator performs the steps themselves.

Parity is pinned by tests/test_oracle_*.py against the worked examples the
pages print, their step tables, closed forms, brute force on tiny inputs and an
fp64 error bound; nothing in this module is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

DTYPES = ("int32", "f32", "bf16")
OPS = ("sum", "max", "prod")


# --------------------------------------------------------------------------
# bf16 <-> f32 by definition
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly.

    bf16 is the upper half of an IEEE binary32 word, so the widening appends
    sixteen zero bits; no rounding is involved.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_value_f64(hi16: np.ndarray) -> np.ndarray:
    """Numeric value (float64) of bf16 patterns, with the all-ones-exponent
    finite continuation 2**128 used for the overflow candidate."""
    hi16 = hi16.astype(np.uint32)
    mag = hi16 & 0x7FFF
    sign = np.where(hi16 & 0x8000, -1.0, 1.0)
    out = (mag.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # the pattern just above the largest finite bf16 is +inf; for rounding
    # decisions it stands for the value 2**128 (unbounded exponent range)
    out = np.where(mag == 0x7F80, 2.0 ** 128, out)
    return sign * np.abs(out)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) by definition.

    For each finite x, take the two bf16 neighbours that bracket it (the
    truncation toward zero and the next value away from zero), measure both
    distances exactly in float64 and keep the nearer one; on a tie keep the one
    whose last mantissa bit is 0.  A value that rounds to 2**128 or beyond is an
    overflow and becomes +-inf.  NaN maps to a quiet NaN with the same sign.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    with np.errstate(invalid="ignore", over="ignore"):
        return _f32_to_bf16_bits(x)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)          # truncation toward zero
    hi = lo + np.uint32(1)                                # next bf16 away from zero
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - _bf16_value_f64(lo))
    d_hi = np.abs(_bf16_value_f64(hi) - xv)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    r = np.where(take_hi, hi, lo).astype(np.uint32)
    # exact bf16 values (low half zero) are returned unchanged
    r = np.where((u & 0xFFFF) == 0, lo, r)
    nan = np.isnan(x)
    r = np.where(nan, (lo | 0x0040), r)
    inf = np.isinf(x)
    r = np.where(inf, lo, r)
    return (r & 0xFFFF).astype(np.uint16)


# --------------------------------------------------------------------------
# element types and the combine operator
# --------------------------------------------------------------------------

def to_acc(x: np.ndarray, dtype: str) -> np.ndarray:
    """Input buffer -> accumulator array (int32, or float32 for f32/bf16)."""
    if dtype == "int32":
        return np.array(x, dtype=np.int32, copy=True)
    if dtype == "f32":
        return np.array(x, dtype=np.float32, copy=True)
    if dtype == "bf16":
        return bf16_bits_to_f32(np.asarray(x, dtype=np.uint16)).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def from_acc(a: np.ndarray, dtype: str) -> np.ndarray:
    """Accumulator -> output buffer type (bf16 rounds once, here)."""
    if dtype == "int32":
        return np.array(a, dtype=np.int32, copy=True)
    if dtype == "f32":
        return np.array(a, dtype=np.float32, copy=True)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def _fmax_ieee(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    out = np.where(a > b, a, b)
    both_zero = (a == 0) & (b == 0)
    z = (a.view(np.uint32) & b.view(np.uint32)).view(np.float32)
    out = np.where(both_zero, z, out)
    nan = np.isnan(a) | np.isnan(b)
    return np.where(nan, np.float32(np.nan), out).astype(np.float32)


def combine(op: str, local: np.ndarray, incoming: np.ndarray) -> np.ndarray:
    """The elementwise reduction operator: local (+) incoming.

    SUM, MAX and PROD are the operators the pages name ([Lesson3], "核心概念"
    item 1; [Blog], "Reduce & All Reduce").  Integer SUM and PROD wrap modulo
    2**32 (NumPy int32 array arithmetic wraps).
    """
    if local.dtype == np.int32:
        if op == "sum":
            return np.add(local, incoming, dtype=np.int32)
        if op == "prod":
            return np.multiply(local, incoming, dtype=np.int32)
        if op == "max":
            return np.maximum(local, incoming)
    else:
        local = local.astype(np.float32, copy=False)
        incoming = incoming.astype(np.float32, copy=False)
        if op == "sum":
            return np.add(local, incoming, dtype=np.float32)
        if op == "prod":
            return np.multiply(local, incoming, dtype=np.float32)
        if op == "max":
            return _fmax_ieee(local, incoming)
    raise ValueError(f"unknown op {op!r}")


# --------------------------------------------------------------------------
# chunking
# --------------------------------------------------------------------------

def chunk_bounds(M: int, N: int) -> List[int]:
    """b_c = floor(c*M/N) for c = 0..N: N contiguous chunks, possibly empty
    when M < N ([Lesson3], simulator: each rank views its tensor as N blocks)."""
    return [(c * M) // N for c in range(N + 1)]


def chunk_of(idx: np.ndarray, M: int, N: int) -> np.ndarray:
    """Chunk index of each element index (the chunk c with b_c <= e < b_{c+1})."""
    b = np.asarray(chunk_bounds(M, N), dtype=np.int64)
    return np.searchsorted(b, np.asarray(idx, dtype=np.int64), side="right") - 1


# --------------------------------------------------------------------------
# step trace / accounting record
# --------------------------------------------------------------------------

@dataclass
class Trace:
    """What a simulated schedule did: per step, the (src, dst, what, count)
    transfers, and per rank the number of values sent."""
    steps: List[List[Tuple[int, int, object, int]]] = field(default_factory=list)
    sent: List[int] = field(default_factory=list)

    @property
    def nsteps(self) -> int:
        return len(self.steps)


# --------------------------------------------------------------------------
# ring schedule
# --------------------------------------------------------------------------

def _ring_transfers(N: int, s: int, first: Sequence[int]) -> List[Tuple[int, int, int]]:
    """The transfers of ring step s as (sender, receiver, chunk), one per
    receiver in rank order: every rank receives from its left neighbour
    i = (r - 1) mod N, which passes on chunk (first[i] - s) mod N -- the
    chunk it passed on at step 0, moved back by one per step ([AR-notes],
    "算法一：Ring AllReduce": at step s rank i sends chunk (i - s) mod N)."""
    return [((r - 1) % N, r, (first[(r - 1) % N] - s) % N) for r in range(N)]


def _synchronous_step(acc: List[np.ndarray], b: List[int], transfers, deliver, tr: Trace) -> None:
    """One step of the schedule: every message is read off its sender before
    any receiver changes, then each is handed to deliver(receiver row, lo, hi,
    payload) ([Lesson3], reference answer: a step's sends are copied first, so
    that no rank reads data already updated in the same step)."""
    wire = [(src, dst, c, acc[src][b[c]:b[c + 1]].copy()) for src, dst, c in transfers]
    for src, dst, c, payload in wire:
        deliver(acc[dst], b[c], b[c + 1], payload)
        tr.sent[src] += b[c + 1] - b[c]
    tr.steps.append([(src, dst, c, b[c + 1] - b[c]) for src, dst, c, _ in wire])


def _ring_rs_phase(acc: List[np.ndarray], b: List[int], op: str, off: int,
                   tr: Trace) -> None:
    """Ring ReduceScatter phase, N-1 steps.

    At step s rank r sends its chunk (r - s + off) mod N to rank r+1, which
    folds it into its own copy as op(own, incoming) ([AR-notes], "算法一：Ring
    AllReduce", 阶段 1; [Slides], "环形 ReduceScatter").  off = 0 is the
    pages' formula, used inside AllReduce: rank r ends owning chunk (r+1) mod N.
    off = -1 is the standalone ReduceScatter, whose contract puts chunk r on
    rank r ([Slides], primitives table and the 3-rank example).
    """
    N = len(acc)
    first = [(r + off) % N for r in range(N)]

    def fold(row, lo, hi, payload):
        row[lo:hi] = combine(op, row[lo:hi], payload)

    for s in range(N - 1):
        _synchronous_step(acc, b, _ring_transfers(N, s, first), fold, tr)


def _ring_ag_phase(acc: List[np.ndarray], b: List[int], own: List[int],
                   tr: Trace) -> None:
    """Ring AllGather phase, N-1 steps: each rank forwards what it received in
    the previous step ([Slides], "环形 AllGather").  own[r] is the chunk rank r
    holds complete at the start: at step s it sends chunk (own[r] - s) mod N,
    which its right neighbour stores."""
    N = len(acc)

    def store(row, lo, hi, payload):
        row[lo:hi] = payload

    for s in range(N - 1):
        _synchronous_step(acc, b, _ring_transfers(N, s, own), store, tr)


def ring_all_reduce(xs: Sequence[np.ndarray], op: str = "sum", dtype: str = "f32",
                    trace: Optional[Trace] = None) -> List[np.ndarray]:
    """Ring AllReduce = ring ReduceScatter then ring AllGather, 2(N-1) steps
    ([MLSys-6], "Ring AllReduce", Algorithm 1; [AR-notes], "语义与分解" and
    "算法一"; [Slides], "2(N−1)/N 是怎么来的").  Returns each rank's output."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    b = chunk_bounds(M, N)
    _ring_rs_phase(acc, b, op, 0, tr)
    _ring_ag_phase(acc, b, [(r + 1) % N for r in range(N)], tr)
    return [from_acc(a, dtype) for a in acc]


def ring_reduce_scatter(xs: Sequence[np.ndarray], op: str = "sum", dtype: str = "f32",
                        trace: Optional[Trace] = None) -> List[np.ndarray]:
    """Standalone ring ReduceScatter: rank r returns the reduced chunk r
    (recvcount = M/N; the pages' send buffer is N chunks of equal size,
    [Slides], "环形 ReduceScatter": V is the per-rank output times N)."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    b = chunk_bounds(M, N)
    _ring_rs_phase(acc, b, op, -1, tr)
    return [from_acc(acc[r][b[r]:b[r + 1]], dtype) for r in range(N)]


def ring_all_gather(shards: Sequence[np.ndarray], dtype: str = "f32",
                    trace: Optional[Trace] = None) -> List[np.ndarray]:
    """Standalone ring AllGather: rank r's shard lands in slot r of every
    rank's output ([Slides], "环形 AllGather" and the primitives table)."""
    N = len(shards)
    S = int(np.asarray(shards[0]).shape[0])
    M = N * S
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    b = chunk_bounds(M, N)
    acc = []
    for r in range(N):
        a = np.zeros(M, dtype=np.asarray(shards[r]).dtype)
        a[b[r]:b[r + 1]] = shards[r]
        acc.append(a)
    _ring_ag_phase(acc, b, list(range(N)), tr)
    return [a.copy() for a in acc]


def ring_fold_elements(vals: np.ndarray, idx: np.ndarray, M: int, op: str,
                       dtype: str, standalone_rs: bool = False) -> np.ndarray:
    """Closed form of the ring's fold for a sample of element indices.

    vals[r, k] is rank r's input at element idx[k].  Following one chunk c
    through the ReduceScatter steps above, its partial starts at rank c (c+1
    for the standalone ReduceScatter) and each step folds in the next rank's
    value as op(next_rank_value, partial), N-1 times.  This is the same
    arithmetic as ring_all_reduce, written without steps, so that full-size
    outputs can be checked at sampled positions.
    """
    vals = np.asarray(vals)
    N = vals.shape[0]
    c = chunk_of(idx, M, N)
    start = (c + (1 if standalone_rs else 0)) % N
    cols = np.arange(vals.shape[1])
    acc = to_acc(vals[start, cols], dtype)
    for j in range(1, N):
        acc = combine(op, to_acc(vals[(start + j) % N, cols], dtype), acc)
    return from_acc(acc, dtype)


# --------------------------------------------------------------------------
# recursive halving-doubling (N = 2**k)
# --------------------------------------------------------------------------

def _is_pow2(n: int) -> bool:
    return n >= 1 and (n & (n - 1)) == 0


def _blk_elems(b: List[int], lo: int, hi: int) -> Tuple[int, int]:
    return b[lo], b[hi]


def _hd_rs_phase(acc: List[np.ndarray], b: List[int], op: str, tr: Trace) -> None:
    """Recursive halving ReduceScatter: at the step with distance d = N/2, N/4,
    ..., 1, rank i exchanges with i XOR d ([AR-notes], "算法二：Recursive
    Halving-Doubling", table tbl-cc-ar-hd-trace: pairs (0,4)(1,5)... first,
    moving M/2, then M/4, M/8).  Each rank's current block range of chunks is
    halved: the rank whose bit d is 0 keeps the lower half, the other the upper
    half, and it combines the partner's copy of the half it keeps.  After the
    phase rank i holds chunk i."""
    N = len(acc)
    rng = [(0, N)] * N
    d = N // 2
    while d >= 1:
        keep, send = [], []
        for i in range(N):
            lo, hi = rng[i]
            mid = (lo + hi) // 2
            if i & d == 0:
                keep.append((lo, mid)); send.append((mid, hi))
            else:
                keep.append((mid, hi)); send.append((lo, mid))
        snap = []
        for i in range(N):
            e0, e1 = _blk_elems(b, *send[i])
            snap.append(acc[i][e0:e1].copy())
        step = []
        for i in range(N):
            p = i ^ d
            assert send[p] == keep[i]
            e0, e1 = _blk_elems(b, *keep[i])
            acc[i][e0:e1] = combine(op, acc[i][e0:e1], snap[p])
            tr.sent[p] += e1 - e0
            step.append((p, i, keep[i], e1 - e0))
            rng[i] = keep[i]
        tr.steps.append(step)
        d //= 2


def _hd_ag_phase(acc: List[np.ndarray], b: List[int], tr: Trace) -> None:
    """Recursive doubling AllGather, the reverse of the halving phase: at
    distance d = 1, 2, ..., N/2 partners swap their block ranges and the held
    range doubles ([AR-notes], "算法二", 阶段 2)."""
    N = len(acc)
    rng = [(i, i + 1) for i in range(N)]
    d = 1
    while d < N:
        snap = []
        for i in range(N):
            e0, e1 = _blk_elems(b, *rng[i])
            snap.append(acc[i][e0:e1].copy())
        step = []
        new = list(rng)
        for i in range(N):
            p = i ^ d
            e0, e1 = _blk_elems(b, *rng[p])
            acc[i][e0:e1] = snap[p]
            tr.sent[p] += e1 - e0
            step.append((p, i, rng[p], e1 - e0))
            new[i] = (min(rng[i][0], rng[p][0]), max(rng[i][1], rng[p][1]))
        rng = new
        tr.steps.append(step)
        d *= 2


def _hd_core(acc: List[np.ndarray], op: str, tr: Trace) -> None:
    M = int(acc[0].shape[0])
    b = chunk_bounds(M, len(acc))
    _hd_rs_phase(acc, b, op, tr)
    _hd_ag_phase(acc, b, tr)


def hd_all_reduce(xs, op="sum", dtype="f32", trace=None):
    """Halving-doubling AllReduce: 2*log2(N) steps ([AR-notes], "算法二";
    [Blog], "Recursive Halving-Doubling").  For N not a power of two the
    first 2r ranks are folded in pairs before and restored after
    (_with_pair_fold), r = N - 2**floor(log2 N)."""
    N = len(xs)
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    if _is_pow2(N):
        _hd_core(acc, op, tr)
    else:
        _with_pair_fold(acc, op, tr, _hd_core)
    return [from_acc(a, dtype) for a in acc]


def hd_reduce_scatter(xs, op="sum", dtype="f32", trace=None):
    N = len(xs)
    if not _is_pow2(N):
        raise ValueError("halving-doubling needs N = 2**k")
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    b = chunk_bounds(M, N)
    _hd_rs_phase(acc, b, op, tr)
    return [from_acc(acc[r][b[r]:b[r + 1]], dtype) for r in range(N)]


def hd_all_gather(shards, dtype="f32", trace=None):
    N = len(shards)
    if not _is_pow2(N):
        raise ValueError("halving-doubling needs N = 2**k")
    S = int(np.asarray(shards[0]).shape[0])
    M = N * S
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    b = chunk_bounds(M, N)
    acc = []
    for r in range(N):
        a = np.zeros(M, dtype=np.asarray(shards[r]).dtype)
        a[b[r]:b[r + 1]] = shards[r]
        acc.append(a)
    _hd_ag_phase(acc, b, tr)
    return [a.copy() for a in acc]


def hd_fold_elements(vals: np.ndarray, idx: np.ndarray, M: int, op: str,
                     dtype: str) -> np.ndarray:
    """Closed form of the halving phase for sampled elements of chunk c:
    S_N(j) = x_j and S_d(j) = op(S_2d(j), S_2d(j XOR d)) for d = N/2 .. 1;
    the result for chunk c is S_1(c).  For N not a power of two the sequence
    starts from the pair-folded values w_v (see _pair_folded_values) over the
    m = 2**floor(log2 N) remaining ranks, whose vector is cut into m chunks."""
    vals = np.asarray(vals)
    N = vals.shape[0]
    S = _pair_folded_values(vals, op, dtype)
    m = len(S)
    c = chunk_of(idx, M, m)
    cols = np.arange(vals.shape[1])
    d = m // 2
    while d >= 1:
        S = [combine(op, S[j], S[j ^ d]) for j in range(m)]
        d //= 2
    stacked = np.stack(S)
    return from_acc(stacked[c, cols], dtype)


# --------------------------------------------------------------------------
# butterfly (recursive doubling with full exchange), N = 2**k
# --------------------------------------------------------------------------

def _butterfly_core(v: List[np.ndarray], op: str, tr: Trace) -> None:
    N = len(v)
    M = int(v[0].shape[0])
    k = 1
    while k < N:
        snap = [a.copy() for a in v]
        step = []
        for i in range(N):
            p = i ^ k
            v[i] = combine(op, v[i], snap[p])
            tr.sent[p] += M
            step.append((p, i, "all", M))
        tr.steps.append(step)
        k *= 2


def butterfly_all_reduce(xs, op="sum", dtype="f32", trace=None):
    """Butterfly AllReduce: log2(N) steps; at step k rank i pairs with
    i XOR 2**k, both exchange the full vector and combine it ([AR-notes],
    "算法四：Butterfly (Recursive Doubling)": distance 1, then 2, then 4).
    For N not a power of two the first 2r ranks are folded in pairs before
    and restored after, as for halving-doubling ([AR-notes], 算法四,
    "非 2^k 处理")."""
    N = len(xs)
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    v = [to_acc(x, dtype) for x in xs]
    if _is_pow2(N):
        _butterfly_core(v, op, tr)
    else:
        _with_pair_fold(v, op, tr, _butterfly_core)
    return [from_acc(a, dtype) for a in v]


def butterfly_fold_elements(vals: np.ndarray, rank: int, op: str, dtype: str) -> np.ndarray:
    """Closed form of butterfly's result on one rank: a pairwise tree over the
    sequence x_{rank XOR t}, t = 0..N-1, nearest pairs combined first.  For N
    not a power of two the tree runs over the pair-folded values w_v of the
    m remaining ranks, taken from the virtual rank that `rank` belongs to
    (rank // 2 for the first 2r ranks, rank - r after them)."""
    vals = np.asarray(vals)
    N = vals.shape[0]
    w = _pair_folded_values(vals, op, dtype)
    m = len(w)
    r = N - m
    v = rank // 2 if rank < 2 * r else rank - r
    seq = [w[v ^ t] for t in range(m)]
    while len(seq) > 1:
        seq = [combine(op, seq[2 * i], seq[2 * i + 1]) for i in range(len(seq) // 2)]
    return from_acc(seq[0], dtype)


# --------------------------------------------------------------------------
# N not a power of two: fold pairs first, restore them last
# --------------------------------------------------------------------------

def _pair_fold_layout(N: int) -> Tuple[int, List[int]]:
    """r = N - 2**floor(log2 N) and the ranks that take part in the
    power-of-two schedule: 0, 2, ..., 2r-2 (each holding its pair's fold),
    then 2r .. N-1 ([Blog], RHD "非 2 的整数次幂场景": the 2r ranks of part1 are
    reduced pairwise into r ranks, the block of p' = 2**floor(log2 p) ranks
    runs halving-doubling, and the folded ranks get the result back)."""
    m = 1 << (N.bit_length() - 1)
    r = N - m
    return r, [2 * v for v in range(r)] + list(range(2 * r, N))


def _with_pair_fold(acc: List[np.ndarray], op: str, tr: Trace,
                    core: Callable[[List[np.ndarray], str, Trace], None]) -> None:
    """Pre-step: rank 2i+1 (i < r) sends its vector to rank 2i, which combines
    it, op(own, incoming).  The m = N - r active ranks run `core` as virtual
    ranks 0..m-1.  Post-step: rank 2i sends the result to rank 2i+1.  The two
    extra steps cost 2 alpha + 2 M beta ([AR-notes], "拓扑要求与非 2^k 处理")."""
    N = len(acc)
    M = int(acc[0].shape[0])
    r, active = _pair_fold_layout(N)
    snap = {2 * i + 1: acc[2 * i + 1].copy() for i in range(r)}
    step = []
    for i in range(r):
        acc[2 * i] = combine(op, acc[2 * i], snap[2 * i + 1])
        tr.sent[2 * i + 1] += M
        step.append((2 * i + 1, 2 * i, "all", M))
    tr.steps.append(step)
    sub = Trace()
    sub.sent = [0] * len(active)
    vacc = [acc[a] for a in active]
    core(vacc, op, sub)
    for v, a in enumerate(active):
        acc[a] = vacc[v]
        tr.sent[a] += sub.sent[v]
    for st in sub.steps:
        tr.steps.append([(active[s], active[d], what, n) for (s, d, what, n) in st])
    step = []
    for i in range(r):
        acc[2 * i + 1] = acc[2 * i].copy()
        tr.sent[2 * i] += M
        step.append((2 * i, 2 * i + 1, "all", M))
    tr.steps.append(step)


def _pair_folded_values(vals: np.ndarray, op: str, dtype: str) -> List[np.ndarray]:
    """w_v = op(x_{2v}, x_{2v+1}) for v < r, x_{v+r} otherwise (accumulator
    type): the values the m active ranks start the power-of-two schedule with."""
    N = vals.shape[0]
    m = 1 << (N.bit_length() - 1)
    r = N - m
    return [combine(op, to_acc(vals[2 * v], dtype), to_acc(vals[2 * v + 1], dtype)) if v < r
            else to_acc(vals[v + r], dtype) for v in range(m)]


# --------------------------------------------------------------------------
# binary tree AllReduce (reduce up, broadcast down), any N
# --------------------------------------------------------------------------

def tree_all_reduce(xs, op="sum", dtype="f32", trace=None):
    """Tree AllReduce ([MLSys-6], "Tree AllReduce"): in the reduce phase the
    leaves send to their parents and every parent combines what it receives
    and passes it up, reaching the root after log2(N) steps; the broadcast
    phase sends the root's result back down in as many steps.  The tree is
    the one whose link use the passage counts -- N/2 senders at the leaf
    level, N/4 at the next, two nodes at the root: at distance d = 1, 2, 4,
    ... rank i with i mod 2d = d sends its partial to rank i - d, which
    combines op(own, incoming).  The broadcast doubles the holders from rank 0
    (distance D/2, ..., 1 with D the power of two at or above N).  For N not
    a power of two the ranks from N up are absent.  The root rounds bf16 once
    and the broadcast copies the rounded result."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    d = 1
    while d < N:
        senders = list(range(d, N, 2 * d))
        snap = {i: acc[i].copy() for i in senders}
        step = []
        for i in senders:
            acc[i - d] = combine(op, acc[i - d], snap[i])
            tr.sent[i] += M
            step.append((i, i - d, "all", M))
        tr.steps.append(step)
        d *= 2
    out: List[Optional[np.ndarray]] = [None] * N
    out[0] = from_acc(acc[0], dtype)
    d //= 2
    while d >= 1:
        step = []
        for i in range(0, N, 2 * d):
            if i + d < N:
                out[i + d] = out[i].copy()
                tr.sent[i] += M
                step.append((i, i + d, "all", M))
        tr.steps.append(step)
        d //= 2
    return out


def tree_fold_elements(vals: np.ndarray, op: str, dtype: str) -> np.ndarray:
    """Closed form of the tree's result: T(lo, n) over the ranks lo..lo+n-1
    is x_lo for n = 1, else op(T(lo, h), T(lo + h, n - h)) with h the largest
    power of two below n -- the subtree that rank lo gathers before its
    partner at distance h sends the rest."""
    vals = np.asarray(vals)

    def T(lo: int, n: int) -> np.ndarray:
        if n == 1:
            return to_acc(vals[lo], dtype)
        h = 1 << ((n - 1).bit_length() - 1)
        return combine(op, T(lo, h), T(lo + h, n - h))

    return from_acc(T(0, vals.shape[0]), dtype)


# --------------------------------------------------------------------------
# double binary tree
# --------------------------------------------------------------------------

def dbt_trees(N: int) -> Tuple[Dict[int, List[int]], int, Dict[int, List[int]], int]:
    """The two complementary trees ([AR-notes], "算法三：Double Binary Tree":
    T1 and T2 complementary, the leaves of one are internal nodes of the
    other; [MLSys-6], "双二叉树").  The pages fix only that property; the
    construction read here: T1 is the in-order binary tree over ranks
    1..N-1 -- rank x whose lowest set bit is b has the left child x - b/2 and
    the right child x + c, c the largest of b/2, b/4, ... with x + c < N (no
    right child if there is none) -- rooted at the largest power of two below
    N, with rank 0 on top of that root as its parent.  T2 is T1 with every
    rank x renamed (x + 1) mod N.  For N = 2**k the leaves of T1 are the odd
    ranks and those of T2 the even ranks.  Returns (children, top) of T1 and
    of T2; children lists are left first."""
    ch1: Dict[int, List[int]] = {x: [] for x in range(N)}
    if N >= 2:
        root = 1 << ((N - 1).bit_length() - 1)
        ch1[0] = [root]
        for x in range(1, N):
            bl = x & -x
            if bl >= 2:
                ch1[x].append(x - bl // 2)
                c = bl // 2
                while c >= 1 and x + c >= N:
                    c //= 2
                if c >= 1:
                    ch1[x].append(x + c)
    ch2 = {(x + 1) % N: [(y + 1) % N for y in ys] for x, ys in ch1.items()}
    return ch1, 0, ch2, 1 % N


def _tree_heights(ch: Dict[int, List[int]], top: int) -> Dict[int, int]:
    h: Dict[int, int] = {}

    def H(x: int) -> int:
        if x not in h:
            h[x] = 1 + max((H(y) for y in ch[x]), default=-1)
        return h[x]

    H(top)
    return h


def _tree_depths(ch: Dict[int, List[int]], top: int) -> Dict[int, int]:
    dep = {top: 0}
    todo = [top]
    while todo:
        x = todo.pop()
        for y in ch[x]:
            dep[y] = dep[x] + 1
            todo.append(y)
    return dep


def double_tree_all_reduce(xs, op="sum", dtype="f32", trace=None):
    """Double binary tree AllReduce ([AR-notes], "算法三": the message is cut
    in two halves, each half does a Reduce and a Broadcast on one of the two
    trees, both trees at once).  Elements [0, M//2) use T1 and [M//2, M) T2.
    Reduce: at step t every node of height t sends its partial up; a node's
    partial is op(op(own, partial of left child), partial of right child),
    children folded left first once both have arrived.  Broadcast: at step t
    the nodes of depth t send the top's result (bf16 rounded once at the top)
    to their children.  The two trees share the step counter."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    out = [np.empty(M, dtype=np.uint16 if dtype == "bf16" else acc[0].dtype) for _ in range(N)]
    if N == 1:
        return [from_acc(acc[0], dtype)]
    ch1, top1, ch2, top2 = dbt_trees(N)
    h = M // 2
    trees = [(ch1, top1, 0, h), (ch2, top2, h, M)]
    hts = [_tree_heights(c, t) for c, t, _, _ in trees]
    deps = [_tree_depths(c, t) for c, t, _, _ in trees]
    H = max(hts[0][trees[0][1]], hts[1][trees[1][1]])
    parents = [{y: x for x, ys in c.items() for y in ys} for c, _, _, _ in trees]
    inbox: List[Dict[int, np.ndarray]] = [dict(), dict()]
    for t in range(H):
        step = []
        for k, (ch, top, lo, hi) in enumerate(trees):
            for x in sorted(x for x in ch if hts[k][x] == t and x != top):
                part = acc[x][lo:hi].copy()
                for y in ch[x]:
                    part = combine(op, part, inbox[k][y])
                inbox[k][x] = part
                tr.sent[x] += hi - lo
                step.append((x, parents[k][x], (lo, hi), hi - lo))
        tr.steps.append(step)
    for k, (ch, top, lo, hi) in enumerate(trees):
        part = acc[top][lo:hi].copy()
        for y in ch[top]:
            part = combine(op, part, inbox[k][y])
        out[top][lo:hi] = from_acc(part, dtype)
    for t in range(H):
        step = []
        for k, (ch, top, lo, hi) in enumerate(trees):
            for x in sorted(x for x in ch if deps[k][x] == t):
                for y in ch[x]:
                    out[y][lo:hi] = out[x][lo:hi]
                    tr.sent[x] += hi - lo
                    step.append((x, y, (lo, hi), hi - lo))
        tr.steps.append(step)
    return out


def dbt_fold_elements(vals: np.ndarray, idx: np.ndarray, M: int, op: str, dtype: str) -> np.ndarray:
    """Closed form of the double tree's result at sampled elements: the
    recursive subtree fold F(x) = op(op(x_x, F(left)), F(right)) of T1 for
    idx < M//2 and of T2 otherwise, evaluated at the top."""
    vals = np.asarray(vals)
    N = vals.shape[0]
    idx = np.asarray(idx)
    if N == 1:
        return from_acc(to_acc(vals[0], dtype), dtype)
    ch1, top1, ch2, top2 = dbt_trees(N)

    def F(ch, x, cols):
        a = to_acc(vals[x, cols], dtype)
        for y in ch[x]:
            a = combine(op, a, F(ch, y, cols))
        return a

    out = np.empty(len(idx), dtype=np.uint16 if dtype == "bf16" else to_acc(vals[0, :1], dtype).dtype)
    first = idx < M // 2
    cols = np.arange(len(idx))
    if first.any():
        out[first] = from_acc(F(ch1, top1, cols[first]), dtype)
    if (~first).any():
        out[~first] = from_acc(F(ch2, top2, cols[~first]), dtype)
    return out


# --------------------------------------------------------------------------
# 2-port ring
# --------------------------------------------------------------------------

def ring2_chain_lengths(N: int) -> Tuple[int, int]:
    """(a, b): the clockwise chain of a chunk covers the a ranks before its
    owner, the counter-clockwise chain the b ranks after it; a + b = N - 1."""
    return (N - 1 + 1) // 2, (N - 1) // 2


def ring2_all_reduce(xs, op="sum", dtype="f32", trace=None):
    """2-port ring AllReduce ([AR-notes], "2-port Ring 优化": with two DMA
    engines the chunks go round the ring in both directions and the number of
    steps halves).  Reading: chunk c is owned by rank c.  Its ReduceScatter
    runs two chains toward the owner at once: a clockwise one that starts at
    rank c-a and moves +1 per step, and a counter-clockwise one that starts
    at rank c+b and moves -1 per step (a = ceil((N-1)/2), b = floor((N-1)/2));
    a rank folds its own value into the partial it receives, op(own,
    partial); the owner folds its own value into the clockwise partial,
    keeps the counter-clockwise partial until then, and ends with
    op(op(x_c, P_cw), P_ccw).  The AllGather sends the finished chunk a ranks
    clockwise and b ranks counter-clockwise.  Each step a rank sends one
    chunk on each port."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    own = [a.copy() for a in acc]
    bnd = chunk_bounds(M, N)
    a, b = ring2_chain_lengths(N)
    held_ccw: Dict[int, np.ndarray] = {}
    for s in range(a):
        snap = []
        for c in range(N):
            lo, hi = bnd[c], bnd[c + 1]
            # clockwise: the partial at rank c-a+s moves to c-a+s+1
            src = (c - a + s) % N
            snap.append(("cw", c, src, (src + 1) % N, acc[src][lo:hi].copy()))
            if s < b:
                src = (c + b - s) % N
                snap.append(("ccw", c, src, (src - 1) % N, acc[src][lo:hi].copy()))
        step = []
        for kind, c, src, dst, part in snap:
            lo, hi = bnd[c], bnd[c + 1]
            if dst == c and kind == "ccw":
                held_ccw[c] = part
            elif dst == c:
                acc[c][lo:hi] = combine(op, own[c][lo:hi], part)
            else:
                acc[dst][lo:hi] = combine(op, own[dst][lo:hi], part)
            tr.sent[src] += hi - lo
            step.append((src, dst, (kind, c), hi - lo))
        tr.steps.append(step)
    res = [None] * N
    for c in range(N):
        lo, hi = bnd[c], bnd[c + 1]
        if c in held_ccw:
            acc[c][lo:hi] = combine(op, acc[c][lo:hi], held_ccw[c])
    out = [np.empty(M, dtype=np.uint16 if dtype == "bf16" else acc[0].dtype) for _ in range(N)]
    for c in range(N):
        lo, hi = bnd[c], bnd[c + 1]
        out[c][lo:hi] = from_acc(acc[c][lo:hi], dtype)
    for s in range(a):
        snap = []
        for c in range(N):
            lo, hi = bnd[c], bnd[c + 1]
            src = (c + s) % N
            snap.append(("cw", c, src, (src + 1) % N, out[src][lo:hi].copy()))
            if s < b:
                src = (c - s) % N
                snap.append(("ccw", c, src, (src - 1) % N, out[src][lo:hi].copy()))
        step = []
        for kind, c, src, dst, v in snap:
            lo, hi = bnd[c], bnd[c + 1]
            out[dst][lo:hi] = v
            tr.sent[src] += hi - lo
            step.append((src, dst, (kind, c), hi - lo))
        tr.steps.append(step)
    return out


def ring2_port(entry) -> int:
    """Port of a 2-port ring transfer in a Trace: 0 clockwise, 1 the other way."""
    return 0 if entry[2][0] == "cw" else 1


def ring2_fold_elements(vals: np.ndarray, idx: np.ndarray, M: int, op: str, dtype: str) -> np.ndarray:
    """Closed form of the 2-port ring at sampled elements of chunk c:
    P_cw folds x_{c-a}, then x_{c-a+1} ... x_{c-1} as op(next, partial);
    P_ccw folds x_{c+b}, then x_{c+b-1} ... x_{c+1}; out = op(op(x_c, P_cw),
    P_ccw) (without P_ccw when b = 0)."""
    vals = np.asarray(vals)
    N = vals.shape[0]
    c = chunk_of(idx, M, N)
    cols = np.arange(vals.shape[1])
    a, b = ring2_chain_lengths(N)
    if N == 1:
        return from_acc(to_acc(vals[0, cols], dtype), dtype)
    pcw = to_acc(vals[(c - a) % N, cols], dtype)
    for j in range(a - 1, 0, -1):
        pcw = combine(op, to_acc(vals[(c - j) % N, cols], dtype), pcw)
    out = combine(op, to_acc(vals[c, cols], dtype), pcw)
    if b > 0:
        pccw = to_acc(vals[(c + b) % N, cols], dtype)
        for j in range(b - 1, 0, -1):
            pccw = combine(op, to_acc(vals[(c + j) % N, cols], dtype), pccw)
        out = combine(op, out, pccw)
    return from_acc(out, dtype)


# --------------------------------------------------------------------------
# hierarchical (multi-dimensional) AllReduce
# --------------------------------------------------------------------------

def hier_coords(r: int, dims: Sequence[int]) -> List[int]:
    """Coordinates of rank r, level 0 (the innermost, fastest network level)
    varying fastest: r = r_0 + p_0 (r_1 + p_1 (r_2 + ...))."""
    out = []
    for p in dims:
        out.append(r % p)
        r //= p
    return out


def hier_groups(dims: Sequence[int], level: int) -> List[List[int]]:
    """The groups of level `level`: ranks that agree on every coordinate but
    that level's, each listed by its coordinate at the level."""
    N = int(np.prod(dims))
    step = int(np.prod(dims[:level])) if level else 1
    groups = []
    for r in range(N):
        if hier_coords(r, dims)[level] == 0:
            groups.append([r + k * step for k in range(dims[level])])
    return groups


def hierarchical_all_reduce(xs, dims: Sequence[int], op: str = "sum", dtype: str = "f32",
                            trace: Optional[Trace] = None):
    """Multi-dimensional AllReduce ([AR-notes], "算法五：多维分层 AllReduce":
    N = prod p_i, a ReduceScatter per level from the innermost out, then the
    AllGathers in reverse order; [MLSys-6], "分层全归约": ReduceScatter inside
    the node, AllReduce among the ranks holding the same shard across nodes,
    AllGather inside the node).  Reading: levels 0 .. d-2 run standalone ring
    ReduceScatters within their groups (the member with coordinate c keeps
    chunk c of the group's current range, the fold starting one member after
    it); the outermost level runs a ring AllReduce on that shard; the levels
    then run ring AllGathers back to the full vector.  Partials stay in the
    accumulator type throughout; bf16 rounds once at the end."""
    dims = [int(p) for p in dims]
    N = int(np.prod(dims))
    if len(xs) != N:
        raise ValueError("len(xs) must be prod(dims)")
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    acc = [to_acc(x, dtype) for x in xs]
    rng = [(0, M)] * N
    d = len(dims)

    def run(members, fn):
        lo, hi = rng[members[0]]
        assert all(rng[m] == (lo, hi) for m in members)
        views = [acc[m][lo:hi] for m in members]
        sub = Trace()
        sub.sent = [0] * len(members)
        fn(views, sub)
        return lo, hi, sub

    def merge_steps(per_group):
        # groups of one level run side by side: their k-th steps are one step
        depth = max((len(sub.steps) for _, sub in per_group), default=0)
        for k in range(depth):
            step = []
            for members, sub in per_group:
                if k < len(sub.steps):
                    step.extend((members[s], members[t], w, n) for (s, t, w, n) in sub.steps[k])
            tr.steps.append(step)
        for members, sub in per_group:
            for j, m in enumerate(members):
                tr.sent[m] += sub.sent[j]

    for i in range(d - 1):
        per = []
        for members in hier_groups(dims, i):
            lo, hi, sub = run(members, lambda v, t: _ring_rs_phase(v, chunk_bounds(len(v[0]), len(v)), op, -1, t))
            b = chunk_bounds(hi - lo, len(members))
            for c, m in enumerate(members):
                rng[m] = (lo + b[c], lo + b[c + 1])
            per.append((members, sub))
        merge_steps(per)
    per = []
    for members in hier_groups(dims, d - 1):
        def ar(v, t):
            p = len(v)
            b = chunk_bounds(len(v[0]), p)
            _ring_rs_phase(v, b, op, 0, t)
            _ring_ag_phase(v, b, [(r + 1) % p for r in range(p)], t)
        _, _, sub = run(members, ar)
        per.append((members, sub))
    merge_steps(per)
    for i in range(d - 2, -1, -1):
        per = []
        for members in hier_groups(dims, i):
            # the group's parent range is the union of its members' chunks
            lo = min(rng[m][0] for m in members)
            hi = max(rng[m][1] for m in members)
            for m in members:
                rng[m] = (lo, hi)
            _, _, sub = run(members, lambda v, t: _ring_ag_phase(v, chunk_bounds(len(v[0]), len(v)),
                                                                  list(range(len(v))), t))
            per.append((members, sub))
        merge_steps(per)
    return [from_acc(a, dtype) for a in acc]


def hier_fold_elements(vals: np.ndarray, idx: np.ndarray, M: int, dims: Sequence[int], op: str,
                       dtype: str) -> np.ndarray:
    """Closed form of the hierarchical AllReduce at sampled elements: the
    element's chunk c_i at every level (splitting the range it is in p_i
    ways, level by level), then nested ring chains -- the outermost over its
    coordinate starting at c_(d-1) (AllReduce order), each inner one over its
    coordinate starting at c_i + 1 (standalone ReduceScatter order), every
    chain folding op(next, partial)."""
    vals = np.asarray(vals)
    dims = [int(p) for p in dims]
    d = len(dims)
    strides = [int(np.prod(dims[:i])) for i in range(d)]
    out = []
    for k, e in enumerate(np.asarray(idx)):
        lo, hi = 0, M
        cs = []
        for p in dims:
            b = chunk_bounds(hi - lo, p)
            c = int(np.searchsorted(np.asarray(b), e - lo, side="right") - 1)
            cs.append(c)
            lo, hi = lo + b[c], lo + b[c + 1]

        def F(level, base):
            p = dims[level]
            start = (cs[level] + (0 if level == d - 1 else 1)) % p

            def leaf(coord):
                r = base + coord * strides[level]
                return to_acc(vals[r:r + 1, k], dtype) if level == 0 else F(level - 1, r)

            a = leaf(start)
            for j in range(1, p):
                a = combine(op, leaf((start + j) % p), a)
            return a

        out.append(F(d - 1, 0))
    return from_acc(np.concatenate(out) if out else np.zeros(0, np.float32 if dtype != "int32" else np.int32), dtype)


def multidim_time_model(M_bytes: float, dims: Sequence[int], alphas: Sequence[float],
                        betas_s_per_byte: Sequence[float]) -> List[float]:
    """Per-level times of the multi-dimensional AllReduce ([AR-notes], eq.
    cc-ar-multidim, BlueConnect): level i costs 2(p_i - 1) alpha_i +
    2 (p_i - 1)/p_i * M / P_(i-1) * beta_i, P_(i-1) the product of the inner
    levels' sizes; the total is their sum."""
    out, P = [], 1
    for p, a, b in zip(dims, alphas, betas_s_per_byte):
        out.append(2 * (p - 1) * a + 2.0 * (p - 1) / p * M_bytes / P * b)
        P *= p
    return out


# --------------------------------------------------------------------------
# broadcast
# --------------------------------------------------------------------------

def broadcast(xs, root: int, schedule: str = "ring", trace=None):
    """Broadcast: every rank ends with the root's buffer ([Slides], "Broadcast：
    一份数据发给所有人").  schedule "ring" forwards along the chain root,
    root+1, ...; "binomial" doubles the holders each step, the pattern of the
    rank-0 example in [Blog], "Recursive Halving-Doubling"."""
    N = len(xs)
    M = int(np.asarray(xs[0]).shape[0])
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    have = {root: np.array(xs[root], copy=True)}
    out = [np.array(x, copy=True) for x in xs]
    if schedule == "ring":
        for s in range(N - 1):
            src, dst = (root + s) % N, (root + s + 1) % N
            have[dst] = have[src].copy()
            tr.sent[src] += M
            tr.steps.append([(src, dst, "all", M)])
    elif schedule == "binomial":
        k = 1
        while k < N:
            step = []
            for rel in range(k):
                if rel + k < N:
                    src, dst = (root + rel) % N, (root + rel + k) % N
                    have[dst] = have[src].copy()
                    tr.sent[src] += M
                    step.append((src, dst, "all", M))
            tr.steps.append(step)
            k *= 2
    else:
        raise ValueError(schedule)
    for r in range(N):
        out[r] = have[r]
    return out


# --------------------------------------------------------------------------
# AllToAll(v)
# --------------------------------------------------------------------------

def all_to_all(sends: Sequence[np.ndarray], counts: np.ndarray, row: int = 1,
               pairwise: bool = False, trace=None) -> List[np.ndarray]:
    """AllToAll(v): rank i's send buffer holds N consecutive blocks, block j
    (counts[i][j] rows of `row` elements) destined for rank j; rank j's receive
    buffer holds the blocks from ranks 0..N-1 in source order.  No arithmetic,
    no duplication: a blocked transpose ([Slides], "AllToAll：分布式的转置";
    [Blog], "All to All").

    pairwise=True performs the schedule of [Blog], "Pairwise（成对）算法": at
    step k rank i sends to (i+k) mod N and receives from (i-k) mod N; step 0
    is the local block.  The trace records, per step, the largest block moved
    (the max term of that section's time formula)."""
    N = len(sends)
    C = np.asarray(counts, dtype=np.int64).reshape(N, N)
    tr = trace if trace is not None else Trace()
    tr.sent = [0] * N
    sd = np.zeros((N, N + 1), dtype=np.int64)
    sd[:, 1:] = np.cumsum(C, axis=1)                  # send displacement of block j on rank i
    rd = np.zeros((N + 1, N), dtype=np.int64)
    rd[1:, :] = np.cumsum(C, axis=0)                  # recv displacement of block from i on rank j
    recv = [np.zeros(int(rd[N, j]) * row, dtype=np.asarray(sends[0]).dtype) for j in range(N)]

    def move(i, j):
        n = int(C[i, j])
        s0 = int(sd[i, j]) * row
        r0 = int(rd[i, j]) * row
        recv[j][r0:r0 + n * row] = np.asarray(sends[i])[s0:s0 + n * row]
        if i != j:
            tr.sent[i] += n * row
        return n

    if pairwise:
        for k in range(N):
            step = []
            for i in range(N):
                j = (i + k) % N
                n = move(i, j)
                step.append((i, j, "block", n * row))
            tr.steps.append(step)
    else:
        for i in range(N):
            for j in range(N):
                move(i, j)
    return recv


def pairwise_time_model(counts: np.ndarray, alpha: float, beta: float) -> float:
    """T = (N-1) alpha + beta * sum_{k=1..N-1} max_i n_{i,(i+k) mod N}
    ([Blog], "Pairwise（成对）算法", performance model)."""
    C = np.asarray(counts)
    N = C.shape[0]
    t = 0.0
    for k in range(1, N):
        t += alpha + beta * max(C[i, (i + k) % N] for i in range(N))
    return t


# --------------------------------------------------------------------------
# DDP-style gradient buckets
# --------------------------------------------------------------------------

def bucket_pack(sizes_elems: Sequence[int], elem_bytes: int, cap_bytes: int) -> List[List[int]]:
    """Group tensors into buckets in reverse order of the list, closing a
    bucket when the next tensor would push it past the cap; a tensor larger
    than the cap gets a bucket of its own ([MLSys-6], "Bucket fusion": buckets
    of about 25 MB, parameters in reverse forward order)."""
    buckets: List[List[int]] = []
    cur: List[int] = []
    cur_bytes = 0
    for t in reversed(range(len(sizes_elems))):
        nb = int(sizes_elems[t]) * elem_bytes
        if cur and cur_bytes + nb > cap_bytes:
            buckets.append(cur)
            cur, cur_bytes = [], 0
        cur.append(t)
        cur_bytes += nb
    if cur:
        buckets.append(cur)
    return buckets


def bucketed_all_reduce(tensors_per_rank: Sequence[Sequence[np.ndarray]], buckets: List[List[int]],
                        algo: str = "ring", op: str = "sum", dtype: str = "bf16"):
    """All-reduce every bucket as one flat vector (the bucket's tensors laid out
    back to back in bucket order), then split the result back into tensors."""
    N = len(tensors_per_rank)
    fn = {"ring": ring_all_reduce, "hd": hd_all_reduce, "butterfly": butterfly_all_reduce}[algo]
    out = [[None] * len(tensors_per_rank[0]) for _ in range(N)]
    for bk in buckets:
        flat = [np.concatenate([np.asarray(tensors_per_rank[r][t]) for t in bk]) for r in range(N)]
        red = fn(flat, op, dtype)
        for r in range(N):
            pos = 0
            for t in bk:
                n = np.asarray(tensors_per_rank[r][t]).shape[0]
                out[r][t] = red[r][pos:pos + n]
                pos += n
    return out


# --------------------------------------------------------------------------
# closed forms: plain results and accounting
# --------------------------------------------------------------------------

def plain_reduce(xs: Sequence[np.ndarray], op: str, dtype: str) -> np.ndarray:
    """The plain definition B = (+)_j A_j ([AR-notes], "语义与分解", eq.
    cc-ar-semantic), computed order-free where the operator allows: integers in
    int64 then wrapped to int32, float MAX elementwise.  For float SUM the
    order-free reference is the float64 sum (not rounded)."""
    if dtype == "int32":
        a = np.stack([np.asarray(x, dtype=np.int64) for x in xs])
        if op == "sum":
            r = a.sum(axis=0)
            return ((r + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)
        if op == "max":
            return a.max(axis=0).astype(np.int32)
        if op == "prod":
            r = np.ones(a.shape[1], dtype=np.int64)
            for row in a:
                r = ((r * row) + 2 ** 31) % 2 ** 32 - 2 ** 31
            return r.astype(np.int32)
    if op == "max":
        # maximum never rounds: reduce in the accumulator type, exact in any order
        m = to_acc(xs[0], dtype)
        for x in xs[1:]:
            m = _fmax_ieee(m, to_acc(x, dtype))
        return from_acc(m, dtype)
    f = np.stack([to_acc(x, dtype).astype(np.float64) for x in xs])
    if op == "sum":
        return f.sum(axis=0)
    if op == "prod":
        return np.prod(f, axis=0)
    raise ValueError(op)


def ring_values_sent_per_rank(M: int, N: int, coll: str = "all_reduce") -> List[int]:
    """Values each rank sends under the ring schedule, counted chunk by chunk
    ([Lesson3], simulator: bytes_sent_per_rank; equals 2(N-1)M/N when N | M)."""
    b = chunk_bounds(M, N)
    size = [b[c + 1] - b[c] for c in range(N)]
    out = []
    for r in range(N):
        rs = sum(size[(r - s) % N] for s in range(N - 1))
        rs_sa = sum(size[(r - s - 1) % N] for s in range(N - 1))
        ag = sum(size[(r + 1 - s) % N] for s in range(N - 1))
        ag_sa = sum(size[(r - s) % N] for s in range(N - 1))
        out.append({"all_reduce": rs + ag, "reduce_scatter": rs_sa, "all_gather": ag_sa}[coll])
    return out


BUSBW_FACTOR = {
    "all_reduce": lambda n: 2.0 * (n - 1) / n,
    "reduce_scatter": lambda n: (n - 1) / n,
    "all_gather": lambda n: (n - 1) / n,
    "all_to_all": lambda n: (n - 1) / n,
    "broadcast": lambda n: 1.0,
}


def busbw(coll: str, size_bytes: float, seconds: float, n: int) -> float:
    """busbw = (S / t) * factor ([Slides], "algbw 与 busbw"; [AR-notes],
    eq. cc-ar-busbw), in bytes per second."""
    return size_bytes / seconds * BUSBW_FACTOR[coll](n)


def ring_time_model(M_bytes: float, N: int, alpha: float, beta_s_per_byte: float) -> float:
    """T = 2(N-1) alpha + 2 (N-1)/N * M * beta ([Lesson3], "理论通信量与网络
    延迟模型", beta in seconds per byte)."""
    return 2 * (N - 1) * alpha + 2.0 * (N - 1) / N * M_bytes * beta_s_per_byte


def step_time_model(tr: Trace, elem_bytes: float, alpha: float, beta_s_per_byte: float,
                    port_of: Optional[Callable[[tuple], int]] = None) -> float:
    """Time of a simulated schedule under the alpha-beta model, one step after
    the other: each step costs alpha plus beta times the largest number of
    bytes one rank sends through one port in it ([Lesson3], "理论通信量与网络
    延迟模型"; one port per rank unless port_of assigns transfers to ports, as
    for the 2-port ring whose two DMA engines send one chunk each per step,
    [AR-notes], "2-port Ring 优化")."""
    T = 0.0
    for st in tr.steps:
        per: Dict[Tuple[int, int], int] = {}
        for e in st:
            key = (e[0], port_of(e) if port_of else 0)
            per[key] = per.get(key, 0) + e[3]
        worst = max(per.values(), default=0)
        T += alpha + worst * elem_bytes * beta_s_per_byte
    return T


def ring_tree_crossover(N: int, alpha: float, beta_s_per_byte: float) -> Dict[str, float]:
    """Message size (bytes) at which ring and tree AllReduce take the same
    time ([MLSys-6], "算法切换点"): 'exact' solves
    2(N-1)a + 2(N-1)/N M b = 2 log2(N) a + 2 log2(N) M b, 'log' is the
    passage's large-N form N a / (b log2 N) with beta as a rate, and 'rough'
    drops the logarithm (N a / b)."""
    lg = math.log2(N)
    exact = (2 * (N - 1) - 2 * lg) * alpha / ((2 * lg - 2.0 * (N - 1) / N) * beta_s_per_byte)
    return {"exact": exact, "log": N * alpha / beta_s_per_byte / lg, "rough": N * alpha / beta_s_per_byte}


def norm_rel_error(y: np.ndarray, ref64: np.ndarray) -> float:
    """||y - ref||_2 / ||ref||_2 in float64."""
    y = np.asarray(y, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    den = np.linalg.norm(ref64)
    return float(np.linalg.norm(y - ref64) / den) if den > 0 else float(np.linalg.norm(y - ref64))
