"""Closed forms of the accounting: values sent per rank, busbw factors,
bandwidth efficiency, halving sizes, bucket packing, the pairwise time model."""
import math

import numpy as np
import pytest

from oracle import ccsim as cs


def test_lesson_main_case_192_values(golden):
    g = golden("ring_traffic.json")["main_case"]
    N = g["N"]
    K = int(np.prod(g["shape"]))
    tr = cs.Trace()
    cs.ring_all_reduce([np.zeros(K, dtype=np.float32)] * N, "sum", "f32", tr)
    assert tr.sent == [g["values_sent_per_rank"]] * N
    assert cs.ring_values_sent_per_rank(K, N) == tr.sent


@pytest.mark.parametrize("N", [2, 3, 4, 5, 7])
def test_values_sent_match_theory(golden, N):
    assert N in golden("ring_traffic.json")["matched_for_N"]
    K = N * 12
    tr = cs.Trace()
    cs.ring_all_reduce([np.zeros(K, dtype=np.int32)] * N, "sum", "int32", tr)
    assert tr.sent == [2 * (N - 1) * K // N] * N
    t_rs = cs.Trace(); cs.ring_reduce_scatter([np.zeros(K, dtype=np.int32)] * N, "sum", "int32", t_rs)
    t_ag = cs.Trace(); cs.ring_all_gather([np.zeros(K // N, dtype=np.int32)] * N, "int32", t_ag)
    # ReduceScatter and AllGather each carry half of AllReduce's traffic
    assert [2 * v for v in t_rs.sent] == tr.sent
    assert [2 * v for v in t_ag.sent] == tr.sent


def test_values_sent_ragged_sums_chunk_sizes():
    for N, M in ((3, 7), (4, 10), (8, 3), (5, 0)):
        tr = cs.Trace()
        cs.ring_all_reduce([np.zeros(M, dtype=np.int32)] * N, "sum", "int32", tr)
        assert tr.sent == cs.ring_values_sent_per_rank(M, N)
        b = cs.chunk_bounds(M, N)
        assert sum(b[c + 1] - b[c] for c in range(N)) == M


def test_volume_factor_table(golden):
    table = golden("ring_traffic.json")["volume_factor_per_K"]
    K = 1024 * 1024
    for n, f in table.items():
        N = int(n)
        assert sum(cs.ring_values_sent_per_rank(K, N)) / N / K == pytest.approx(f)


def test_busbw_factors(golden):
    g = golden("busbw_factors.json")["factors"]
    for coll, formula in g.items():
        for n in (2, 3, 8, 16):
            expect = eval(formula.replace("2(", "2*("), {"__builtins__": {}}, {"n": n})
            assert cs.busbw(coll, 1.0, 1.0, n) == pytest.approx(expect)


def test_ring_busbw_equals_link_rate_from_traffic():
    """busbw for the ring AllReduce is exactly the per-rank values sent divided
    by the time: the factor 2(N-1)/N is the ring's per-rank traffic over M."""
    for N in (2, 4, 8, 16):
        M = 64 * N
        per_rank = cs.ring_values_sent_per_rank(M, N)[0]
        assert cs.busbw("all_reduce", M, 1.0, N) == pytest.approx(per_rank)


def test_butterfly_bandwidth_efficiency(golden):
    eff = golden("butterfly_pairs_n8.json")["bandwidth_efficiency"]
    for N, key in ((8, "N8_approx"), (64, "N64_approx"), (1024, "N1024_approx")):
        M = N * 4
        ring = cs.ring_values_sent_per_rank(M, N)[0]
        if N <= 64:
            tr = cs.Trace()
            cs.butterfly_all_reduce([np.zeros(M, dtype=np.int32)] * N, "sum", "int32", tr)
            bfly = tr.sent[0]
        else:
            bfly = int(math.log2(N)) * M
        assert ring / bfly == pytest.approx(eff[key], abs=0.01)


def test_hd_sizes_halve_and_sum():
    for N in (2, 4, 8, 16):
        M = 16 * N
        tr = cs.Trace()
        cs.hd_all_reduce([np.zeros(M, dtype=np.int32)] * N, "sum", "int32", tr)
        k = int(math.log2(N))
        sizes = [tr.steps[j][0][3] for j in range(k)]
        assert sizes == [M >> (j + 1) for j in range(k)]
        assert sum(sizes) == (N - 1) * M // N
        assert tr.sent == [2 * (N - 1) * M // N] * N     # bandwidth-optimal like the ring


def test_ring_time_model_lesson_numbers():
    """The lesson's model for its main case: 2(N-1)*10 us + bytes/(25 GB/s)."""
    t = cs.ring_time_model(128 * 4, 4, 10e-6, 1 / 25e9)
    assert t == pytest.approx(2 * 3 * 10e-6 + 192 * 4 / 25e9)


def test_pairwise_time_model():
    C = np.array([[0, 5, 1], [2, 0, 7], [3, 4, 0]])
    # k=1: n01=5, n12=7, n20=3 -> 7 ; k=2: n02=1, n10=2, n21=4 -> 4
    assert cs.pairwise_time_model(C, 1.0, 0.5) == pytest.approx(2 * 1.0 + 0.5 * (7 + 4))


def test_bucket_pack_rules():
    g = np.random.default_rng(0)
    sizes = [int(math.floor(math.exp(v))) for v in g.uniform(math.log(4096), math.log(16_777_216), 120)]
    cap = 25 * 1024 * 1024
    bk = cs.bucket_pack(sizes, 2, cap)
    flat = [t for b in bk for t in b]
    assert flat == list(reversed(range(len(sizes))))
    for i, b in enumerate(bk):
        nbytes = sum(sizes[t] * 2 for t in b)
        assert nbytes <= cap or len(b) == 1
        if i + 1 < len(bk):
            nxt = bk[i + 1][0]
            assert nbytes + sizes[nxt] * 2 > cap       # greedy: the next tensor did not fit


def test_bucketed_all_reduce_matches_per_bucket_ring():
    N = 4
    sizes = [3, 10, 1, 7, 2]
    g = np.random.default_rng(1)
    ten = [[g.integers(-9, 9, size=n, dtype=np.int32) for n in sizes] for _ in range(N)]
    bk = cs.bucket_pack(sizes, 4, 40)
    out = cs.bucketed_all_reduce(ten, bk, "ring", "sum", "int32")
    for t, n in enumerate(sizes):
        expect = sum(ten[r][t].astype(np.int64) for r in range(N))
        for r in range(N):
            assert np.array_equal(out[r][t], expect.astype(np.int32))


def test_ring_time_model_70b_budgets(golden):
    """The textbook's 70B gradient budgets: the ring's bandwidth term
    2(N-1)/N * bytes / link bandwidth at the printed N and link speeds
    (tests/golden/ring_70b_budget.json)."""
    g = golden("ring_70b_budget.json")
    for c in g["cases"]:
        t = cs.ring_time_model(g["gradient_bytes"], c["N"], 0.0, 1 / (c["link_GBps"] * 1e9))
        assert t == pytest.approx(c["seconds"], rel=c["printed_rel_precision"]), c
        if "factor" in c:
            sent = cs.ring_values_sent_per_rank(c["N"] * 1000, c["N"])
            assert sent[0] / (c["N"] * 1000) == c["factor"]
    # a dropped (N-1)/N or a single phase would miss the 64-GPU figure by 1.6% or 2x
    assert cs.ring_time_model(140e9, 64, 0.0, 1 / 50e9) != pytest.approx(2 * 140 / 50, rel=1e-3)
    ctx = g["context_not_a_pin"]
    assert ctx["rs_us"] + ctx["ag_us"] + ctx["sync_us"] == pytest.approx(ctx["total_us"], abs=1e-9)
