"""alltoall -- plain CPU reference of the AllToAll variants around MoE routing.

TEST INFRASTRUCTURE ONLY.  Like oracle/ccsim.py, this module is what the HIP
library is checked against: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does,
and it imports nothing from the product.

Page keys as in oracle/ccsim.py:

  [MLSys-6]  MLSys textbook vol. 2, ch. 6 "集合通信" (gptbert.com)
  [Blog]     "分布式大模型集合通信" blog post (bowenei.github.io)

What is here:

* expert capacity and the capacity-padded dispatch / combine ([MLSys-6],
  "容量因子与有界分配"): fixed-size expert buffers, rows beyond capacity
  dropped, free slots filled with zero rows so the exchange is uniform;
* the hierarchical (node-aggregated) AllToAll ([MLSys-6], "分层 MoE 交换"):
  aggregate inside the source node, one exchange per ordered node pair,
  distribute inside the destination node;
* the AllToAll cost bounds of [MLSys-6] "Napkin Math 1.4" and "二分饱和与慢节点
  尾部" (injection, hottest receiver, bisection).

The pairwise schedule and its time model live in ccsim.all_to_all and
ccsim.pairwise_time_model.  Pins: tests/test_oracle_alltoall.py.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# capacity factor
# --------------------------------------------------------------------------

def expert_capacity(P: int, T: int, k: int, E: int, C) -> int:
    """Capacity_e = ceil(P T k / E * C): P ranks of T tokens, top-k routing
    over E experts, capacity factor C ([MLSys-6], "容量因子与有界分配").
    Exact rational arithmetic, C given as a decimal (1.25 -> 5/4)."""
    c = Fraction(str(C))
    return math.ceil(Fraction(P * T * k, E) * c)


def source_capacity(T: int, k: int, E: int, C) -> int:
    """Rows one source rank may send to one expert: the capacity formula
    applied to that source's own batch, ceil(T k / E * C) (reading: the
    expert buffer is split evenly among the P sources, so that every
    (source, expert) block of the exchange has the same size)."""
    return expert_capacity(1, T, k, E, C)


def padded_dispatch(sends: Sequence[np.ndarray], counts_e: np.ndarray, capacity: int, row: int
                    ) -> Tuple[List[np.ndarray], np.ndarray]:
    """Capacity-padded MoE dispatch.

    sends[i]: rank i's rows sorted by expert, counts_e[i][e] rows of `row`
    elements for expert e = 0..E-1 (E a multiple of N; expert e lives on
    rank e // (E/N) as local expert e % (E/N)).
    Rank j receives, for source i = 0..N-1 and then local expert
    l = 0..E/N-1, a block of `capacity` rows: the first
    min(counts_e[i][e], capacity) rows of source i's expert-e block (e =
    j E/N + l), in order, then zero rows.  Rows beyond the capacity are
    dropped ([MLSys-6], "容量因子与有界分配": C = 1.0 drops the excess; C > 1
    pads every buffer with dummy rows so the collective stays uniform).
    Returns (recv, kept) with kept[i][e] the rows of block (i, e) delivered."""
    N = len(sends)
    Ce = np.asarray(counts_e, dtype=np.int64)
    E = Ce.shape[1]
    if Ce.shape[0] != N or E % N:
        raise ValueError("counts_e must be [N, E] with E a multiple of N")
    epr = E // N
    kept = np.minimum(Ce, capacity)
    disp = np.zeros((N, E + 1), dtype=np.int64)
    disp[:, 1:] = np.cumsum(Ce, axis=1)
    dt = np.asarray(sends[0]).dtype
    recv = []
    for j in range(N):
        out = np.zeros(N * epr * capacity * row, dtype=dt)
        for i in range(N):
            for l in range(epr):
                e = j * epr + l
                n = int(kept[i, e])
                dst = ((i * epr + l) * capacity) * row
                src = int(disp[i, e]) * row
                out[dst:dst + n * row] = np.asarray(sends[i])[src:src + n * row]
        recv.append(out)
    return recv, kept


def padded_combine(expert_bufs: Sequence[np.ndarray], counts_e: np.ndarray, capacity: int, row: int
                   ) -> List[np.ndarray]:
    """The combine exchange, the transpose of padded_dispatch: rank i gets
    back, in its own send order (expert-sorted, counts_e[i][e] rows per
    expert), the rows the expert ranks hold in the slots its rows were
    dispatched to; a dropped row comes back as zeros (reading: the expert
    never saw it; the residual connection that carries such a token is not
    part of the exchange).  expert_bufs[j] has padded_dispatch's receive
    layout."""
    N = len(expert_bufs)
    Ce = np.asarray(counts_e, dtype=np.int64)
    E = Ce.shape[1]
    epr = E // N
    kept = np.minimum(Ce, capacity)
    dt = np.asarray(expert_bufs[0]).dtype
    out = []
    for i in range(N):
        buf = np.zeros(int(Ce[i].sum()) * row, dtype=dt)
        at = 0
        for e in range(E):
            j, l = divmod(e, epr)
            n = int(kept[i, e])
            src = ((i * epr + l) * capacity) * row
            buf[at * row:(at + n) * row] = np.asarray(expert_bufs[j])[src:src + n * row]
            at += int(Ce[i, e])
        out.append(buf)
    return out


def padded_volume(counts_e: np.ndarray, capacity: int) -> Dict[str, int]:
    """Rows the padded exchange moves (every (source, expert) block is
    `capacity` rows), rows a dropless AllToAllv would move, and rows
    dropped.  With balanced routing the padded volume is C times the
    dropless one ([MLSys-6], "容量因子与有界分配")."""
    Ce = np.asarray(counts_e, dtype=np.int64)
    return {"padded_rows": int(Ce.size * capacity), "dropless_rows": int(Ce.sum()),
            "dropped_rows": int(np.maximum(Ce - capacity, 0).sum())}


# --------------------------------------------------------------------------
# hierarchical (node-aggregated) AllToAll
# --------------------------------------------------------------------------

def hier_all_to_all(sends: Sequence[np.ndarray], counts: np.ndarray, row: int, L: int
                    ) -> Tuple[List[np.ndarray], Dict[str, list]]:
    """Two-level AllToAll(v) ([MLSys-6], "分层 MoE 交换"): P = G L ranks,
    rank r on node r // L with local index r % L.  Reading of the three
    phases, with one inter-node flow per ordered node pair (the passage's
    P(P-1) -> N_nodes(N_nodes-1)):

    1. aggregate: rank (n, l) copies its blocks for the ranks of every other
       node n' to the aggregator (n, n' mod L) of its own node, whose payload
       for n' holds the blocks ordered by source local index, then
       destination local index; blocks for ranks of its own node go
       straight to their destination;
    2. exchange: aggregator (n, n' mod L) sends the payload to the receiver
       (n', n mod L);
    3. distribute: the receiver copies every block to its destination rank,
       at the place the flat AllToAll(v) puts it.

    Returns (recv, flows): recv equals ccsim.all_to_all(sends, counts, row);
    flows[phase] lists (src_rank, dst_rank, rows) of every transfer between
    different ranks."""
    P = len(sends)
    C = np.asarray(counts, dtype=np.int64).reshape(P, P)
    if L < 1 or P % L:
        raise ValueError("L must divide the number of ranks")
    G = P // L
    node = lambda r: r // L
    sd = np.zeros((P, P + 1), dtype=np.int64)
    sd[:, 1:] = np.cumsum(C, axis=1)
    rd = np.zeros((P + 1, P), dtype=np.int64)
    rd[1:, :] = np.cumsum(C, axis=0)
    dt = np.asarray(sends[0]).dtype
    recv = [np.zeros(int(rd[P, j]) * row, dtype=dt) for j in range(P)]
    flows: Dict[str, list] = {"aggregate": [], "exchange": [], "distribute": []}

    def block(i, j):
        return np.asarray(sends[i])[int(sd[i, j]) * row:int(sd[i, j] + C[i, j]) * row]

    # phase 1: intra-node blocks delivered, remote blocks gathered per node pair
    payload: Dict[Tuple[int, int], List[Tuple[int, int, np.ndarray]]] = {}
    for n in range(G):
        for n2 in range(G):
            if n2 != n:
                payload[(n, n2)] = []
    for i in range(P):
        for j in range(P):
            if node(i) == node(j):
                recv[j][int(rd[i, j]) * row:int(rd[i, j] + C[i, j]) * row] = block(i, j)
                if i != j and C[i, j]:
                    flows["aggregate"].append((i, j, int(C[i, j])))
    for n in range(G):
        for n2 in range(G):
            if n2 == n:
                continue
            agg = n * L + n2 % L
            for l in range(L):
                i = n * L + l
                rows = 0
                for l2 in range(L):
                    j = n2 * L + l2
                    payload[(n, n2)].append((i, j, block(i, j).copy()))
                    rows += int(C[i, j])
                if i != agg and rows:
                    flows["aggregate"].append((i, agg, rows))
    # phase 2: one transfer per ordered node pair
    landed = {}
    for (n, n2), blocks in payload.items():
        rows = sum(b.size for _, _, b in blocks) // row if row else 0
        src, dst = n * L + n2 % L, n2 * L + n % L
        landed[(n, n2)] = [(i, j, b.copy()) for i, j, b in blocks]
        if rows:
            flows["exchange"].append((src, dst, rows))
    # phase 3: the receiver scatters inside its node
    for (n, n2), blocks in landed.items():
        rcv = n2 * L + n % L
        for i, j, b in blocks:
            recv[j][int(rd[i, j]) * row:int(rd[i, j] + C[i, j]) * row] = b
            if j != rcv and C[i, j]:
                flows["distribute"].append((rcv, j, int(C[i, j])))
    return recv, flows


def flat_inter_node_flows(counts: np.ndarray, L: int) -> int:
    """Transfers of a flat AllToAll that cross nodes (non-empty blocks
    between ranks of different nodes)."""
    C = np.asarray(counts)
    P = C.shape[0]
    return int(sum(1 for i in range(P) for j in range(P) if i // L != j // L and C[i, j] > 0))


# --------------------------------------------------------------------------
# cost bounds
# --------------------------------------------------------------------------

def injection_bound(bytes_matrix: np.ndarray, alpha: float, beta: float) -> float:
    """Lower bound of a concurrent AllToAll on one injection port per rank:
    alpha + (bytes a rank sends to other ranks) * beta, for the busiest
    sender ([MLSys-6], "Napkin Math 1.4": all 7 transfers share the port)."""
    B = np.asarray(bytes_matrix, dtype=np.float64)
    off = B - np.diag(np.diag(B))
    return alpha + float(off.sum(axis=1).max()) * beta


def receive_bound(bytes_matrix: np.ndarray, rx_bytes_per_s: float) -> float:
    """T_dispatch >= (bytes the hottest receiver takes) / BW_rx ([MLSys-6],
    "二分饱和与慢节点尾部", M_max term)."""
    B = np.asarray(bytes_matrix, dtype=np.float64)
    off = B - np.diag(np.diag(B))
    return float(off.sum(axis=0).max()) / rx_bytes_per_s


def bisection_bound(cut_bytes: float, P: int, inject_bytes_per_s: float, oversub: float) -> float:
    """T >= V_cut / BW_bisect with BW_bisect = P BW_inject / (2 R) ([MLSys-6],
    "二分饱和与慢节点尾部")."""
    return cut_bytes / (P * inject_bytes_per_s / (2.0 * oversub))


def uniform_moe_exchange(P: int, tokens_per_rank: int, token_bytes: int) -> Dict[str, float]:
    """[MLSys-6] "Napkin Math 1.4": uniform routing, one expert per token,
    every rank sends an equal share of its tokens to every rank (its own
    share stays local)."""
    per_pair = tokens_per_rank // P
    pair_bytes = per_pair * token_bytes
    return {"tokens_per_pair": per_pair, "bytes_per_pair": pair_bytes,
            "bytes_sent_per_rank": (P - 1) * pair_bytes}


def dispatch_counts_by_expert(choice: np.ndarray, E: int) -> np.ndarray:
    """Rows per expert for one source: its [tokens, k] expert choices counted
    (one row per (token, expert) assignment)."""
    return np.bincount(np.asarray(choice).reshape(-1), minlength=E).astype(np.int64)
