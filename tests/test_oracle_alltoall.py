"""Pins for oracle/alltoall.py: the capacity formula, the capacity-padded
dispatch and combine (brute force on tagged rows, the dropless limit, the
C-fold volume under balanced routing), the hierarchical AllToAll (equal to the
flat one for any counts, one exchange per node pair, the flat forms for one
node or one rank per node) and the cost bounds of the textbook's
Napkin Math 1.4 (tests/golden/moe_alltoall_napkin.json)."""
import json
import os

import numpy as np
import pytest

from oracle import alltoall as aa
from oracle import ccsim as cs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "moe_alltoall_napkin.json")


def test_capacity_formula():
    """[MLSys-6] 容量因子与有界分配: Capacity_e = ceil(P T k / E * C)."""
    assert aa.expert_capacity(8, 512, 1, 64, 1.0) == 64          # Napkin Math 1.4's 64 tokens per expert
    assert aa.expert_capacity(8, 512, 1, 64, 1.25) == 80
    assert aa.expert_capacity(8, 512, 1, 64, 1.5) == 96
    assert aa.expert_capacity(8, 4096, 8, 64, 1.25) == 5120
    assert aa.expert_capacity(1, 100, 1, 64, 1.25) == 2          # 1.953 rounds up
    assert aa.expert_capacity(3, 7, 2, 5, 1.1) == 10             # 42/5 * 11/10 = 9.24 -> 10, exact rationals
    assert aa.source_capacity(4096, 8, 64, 1.25) == 640


def _tagged(counts_e, row, seed):
    """Rows whose first element is a unique tag (source, row index)."""
    N = counts_e.shape[0]
    g = np.random.default_rng(seed)
    out = []
    for i in range(N):
        n = int(counts_e[i].sum())
        x = g.integers(1, 1000, size=(n, row)).astype(np.int32)
        x[:, 0] = i * 100000 + np.arange(n) + 1
        out.append(x.reshape(-1))
    return out


@pytest.mark.parametrize("N,E,cap", [(2, 2, 3), (4, 8, 2), (4, 8, 5), (8, 64, 1), (3, 6, 4), (8, 16, 0)])
def test_padded_dispatch_brute_force(N, E, cap):
    g = np.random.default_rng([N, E, cap])
    Ce = g.integers(0, 7, size=(N, E))
    row = 3
    sends = _tagged(Ce, row, 5)
    recv, kept = aa.padded_dispatch(sends, Ce, cap, row)
    epr = E // N
    assert np.array_equal(kept, np.minimum(Ce, cap))
    for j in range(N):
        r = recv[j].reshape(N, epr, cap, row)
        for i in range(N):
            rows_i = sends[i].reshape(-1, row)
            start = np.concatenate([[0], np.cumsum(Ce[i])])
            for l in range(epr):
                e = j * epr + l
                n = min(int(Ce[i, e]), cap)
                assert np.array_equal(r[i, l, :n], rows_i[start[e]:start[e] + n])   # the first rows, in order
                assert not r[i, l, n:].any()                                          # zero padding


def test_padded_dispatch_dropless_limit_is_the_alltoallv():
    """With a capacity no block exceeds, dropping the padding leaves exactly
    the AllToAll(v) of the expert-sorted rows (ccsim.all_to_all with the
    per-rank counts)."""
    N, E, row = 4, 8, 2
    g = np.random.default_rng(7)
    Ce = g.integers(0, 6, size=(N, E))
    sends = _tagged(Ce, row, 8)
    cap = int(Ce.max())
    recv, _ = aa.padded_dispatch(sends, Ce, cap, row)
    C = Ce.reshape(N, N, E // N).sum(axis=2)
    flat = cs.all_to_all(sends, C, row)
    for j in range(N):
        r = recv[j].reshape(N, E // N, cap, row)
        parts = [r[i, l, :Ce[i, j * (E // N) + l]] for i in range(N) for l in range(E // N)]
        assert np.array_equal(np.concatenate(parts).reshape(-1), flat[j])


def test_padded_volume_is_c_times_dropless_under_balanced_routing():
    """[MLSys-6]: padding to capacity multiplies the bytes on the wire by C."""
    N, E, T, k = 8, 64, 512, 1
    Ce = np.full((N, E), T * k // E)                 # 8 rows per (source, expert)
    cap = aa.source_capacity(T, k, E, 1.25)
    assert cap == 10
    v = aa.padded_volume(Ce, cap)
    assert v["padded_rows"] / v["dropless_rows"] == pytest.approx(1.25)
    assert v["dropped_rows"] == 0
    v1 = aa.padded_volume(Ce, aa.source_capacity(T, k, E, 1.0))
    assert v1["padded_rows"] == v1["dropless_rows"] and v1["dropped_rows"] == 0
    skew = Ce.copy()
    skew[:, 0] += 5
    skew[:, 1] -= 5
    assert aa.padded_volume(skew, 8)["dropped_rows"] == N * 5   # C = 1.0 drops the excess of the hot expert


@pytest.mark.parametrize("cap", [0, 2, 4, 9])
def test_combine_is_the_transpose_of_dispatch(cap):
    N, E, row = 4, 8, 3
    Ce = np.random.default_rng(cap).integers(0, 7, size=(N, E))
    sends = _tagged(Ce, row, 9)
    recv, kept = aa.padded_dispatch(sends, Ce, cap, row)
    back = aa.padded_combine(recv, Ce, cap, row)
    for i in range(N):
        rows = sends[i].reshape(-1, row)
        got = back[i].reshape(-1, row)
        start = np.concatenate([[0], np.cumsum(Ce[i])])
        for e in range(E):
            n = int(kept[i, e])
            assert np.array_equal(got[start[e]:start[e] + n], rows[start[e]:start[e] + n])
            assert not got[start[e] + n:start[e + 1]].any()            # dropped rows come back as zeros


@pytest.mark.parametrize("P,L", [(8, 2), (8, 4), (6, 3), (6, 2), (4, 1), (4, 4), (12, 3), (16, 4)])
def test_hierarchical_equals_flat(P, L):
    g = np.random.default_rng([P, L])
    for trial in range(3):
        C = g.integers(0, 5, size=(P, P))
        if trial == 2:
            C[g.random((P, P)) < 0.4] = 0
        row = 2
        sends = [g.integers(-99, 99, size=int(C[i].sum()) * row).astype(np.int32) for i in range(P)]
        flat = cs.all_to_all(sends, C, row)
        hier, flows = aa.hier_all_to_all(sends, C, row, L)
        for j in range(P):
            assert np.array_equal(hier[j], flat[j]), (P, L, trial, j)
        # every block's rows are carried exactly once across nodes
        inter = sum(int(C[i, j]) for i in range(P) for j in range(P) if i // L != j // L)
        assert sum(n for _, _, n in flows["exchange"]) == inter


@pytest.mark.parametrize("P,L", [(8, 2), (8, 4), (16, 4), (64, 8)])
def test_exchange_flows_per_node_pair(P, L):
    """[MLSys-6] 分层 MoE 交换: inter-node flows fall from P(P-1) to
    N_nodes(N_nodes-1) when every pair has data."""
    G = P // L
    C = np.ones((P, P), dtype=np.int64)
    _, flows = aa.hier_all_to_all([np.arange(P, dtype=np.int32)] * P, C, 1, L)
    assert len(flows["exchange"]) == G * (G - 1)
    pairs = {(s // L, d // L) for s, d, _ in flows["exchange"]}
    assert len(pairs) == G * (G - 1)                      # one transfer per ordered node pair
    assert aa.flat_inter_node_flows(C, L) == P * (P - 1) - G * L * (L - 1)
    assert all(s // L != d // L for s, d, _ in flows["exchange"])
    assert all(s // L == d // L for ph in ("aggregate", "distribute") for s, d, _ in flows[ph])


def test_one_rank_per_node_and_one_node():
    P = 6
    C = np.random.default_rng(3).integers(1, 4, size=(P, P))
    sends = [np.arange(int(C[i].sum()), dtype=np.int32) + 100 * i for i in range(P)]
    _, f1 = aa.hier_all_to_all(sends, C, 1, 1)            # L = 1: the flat exchange
    assert not f1["aggregate"] and not f1["distribute"] and len(f1["exchange"]) == P * (P - 1)
    _, fP = aa.hier_all_to_all(sends, C, 1, P)            # one node: only intra-node copies
    assert not fP["exchange"] and len(fP["aggregate"]) == P * (P - 1)


def test_napkin_math_1_4():
    """[MLSys-6] Napkin Math 1.4: 8 GPUs, 512 tokens each, 4.096 KB tokens,
    uniform routing to 64 experts; 262.144 KB per pair, 1.84 MB per GPU,
    8 us per transfer at alpha = 3 us, beta = 50 GB/s, 56 us serial, and the
    39.7 us injection bound."""
    gd = json.load(open(GOLD))
    u = aa.uniform_moe_exchange(gd["ranks"], gd["tokens_per_rank"], gd["token_bytes"])
    assert u["tokens_per_pair"] == gd["tokens_per_pair"]
    assert u["bytes_per_pair"] == gd["bytes_per_pair"]
    assert round(u["bytes_sent_per_rank"] / 1e6, 2) == gd["bytes_sent_per_rank_MB"]
    a, b = gd["alpha_s"], 1 / gd["beta_bytes_per_s"]
    per = a + u["bytes_per_pair"] * b
    assert round(a * 1e6) + round(u["bytes_per_pair"] * b * 1e6) == gd["transfer_time_us_rounded"]
    assert 7 * gd["transfer_time_us_rounded"] == gd["serial_time_us"]
    B = np.full((8, 8), u["bytes_per_pair"])
    assert aa.injection_bound(B, a, b) * 1e6 == pytest.approx(gd["injection_bound_us"], abs=0.05)
    # the pairwise schedule of the same exchange: 7 steps of alpha + n beta
    assert cs.pairwise_time_model(B, a, b) == pytest.approx(7 * per)
    assert aa.dispatch_counts_by_expert(np.arange(512) % 64, 64).tolist() == [8] * 64


def test_receive_and_bisection_bounds():
    """[MLSys-6] 二分饱和与慢节点尾部: the hottest receiver and the bisection."""
    B = np.array([[5, 1, 2], [3, 7, 4], [6, 0, 9]], dtype=np.float64)
    # receivers take 3+6, 1+0, 2+4 bytes from others -> 9
    assert aa.receive_bound(B, 3.0) == pytest.approx(3.0)
    assert aa.injection_bound(B, 1.0, 0.5) == pytest.approx(1.0 + 0.5 * 7)
    # BW_bisect = P BW / (2R): 8 ranks at 50 B/s, 2:1 -> 100 B/s
    assert aa.bisection_bound(1000.0, 8, 50.0, 2.0) == pytest.approx(10.0)
