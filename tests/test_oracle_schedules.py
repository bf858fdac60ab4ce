"""The oracle's schedules against the step tables and pairing rules the pages print."""
import numpy as np
import pytest

from oracle import ccsim as cs


def test_ring_step_table_n4(golden):
    g = golden("ring_step_table_n4.json")
    letters = "ABCD"
    tr = cs.Trace()
    cs.ring_all_reduce([np.zeros(4, dtype=np.int32) for _ in range(4)], "sum", "int32", tr)
    rs_steps = tr.steps[:3]
    for s, expect in enumerate(g["steps"]):
        got = {f"{src}->{dst}": letters[chunk] for (src, dst, chunk, n) in rs_steps[s]}
        assert got == expect, (s, got)


@pytest.mark.parametrize("N", [2, 3, 4, 5, 8, 16])
def test_ring_owner_after_reduce_scatter_phase(N):
    """Rank i owns chunk (i+1) mod N after the in-AllReduce phase (off=0) and
    chunk i after the standalone ReduceScatter (off=-1)."""
    M = 3 * N
    full = (1 << N) - 1
    for off, owner in ((0, lambda i: (i + 1) % N), (-1, lambda i: i)):
        acc = [np.full(M, 1 << r, dtype=np.int32) for r in range(N)]
        tr = cs.Trace(); tr.sent = [0] * N
        b = cs.chunk_bounds(M, N)
        cs._ring_rs_phase(acc, b, "sum", off, tr)
        for i in range(N):
            c = owner(i)
            assert np.all(acc[i][b[c]:b[c + 1]] == full), (off, i)
            # and no other chunk on rank i is complete
            for c2 in range(N):
                if c2 != c:
                    assert not np.any(acc[i][b[c2]:b[c2 + 1]] == full)


def test_ring_send_rule_matches_slides():
    """At step k rank i sends chunk (i-k) mod N (the ReduceScatter slide)."""
    for N in (3, 5, 8):
        tr = cs.Trace()
        cs.ring_all_reduce([np.zeros(2 * N, dtype=np.int32)] * N, "sum", "int32", tr)
        for k in range(N - 1):
            for (src, dst, chunk, n) in tr.steps[k]:
                assert dst == (src + 1) % N
                assert chunk == (src - k) % N
        # AllGather phase: at step s rank i sends (i+1-s) mod N (lesson simulator)
        for s in range(N - 1):
            for (src, dst, chunk, n) in tr.steps[N - 1 + s]:
                assert chunk == (src + 1 - s) % N


def test_hd_trace_n8(golden):
    g = golden("hd_trace_n8.json")
    M = 64
    tr = cs.Trace()
    cs.hd_reduce_scatter([np.zeros(M, dtype=np.int32)] * 8, "sum", "int32", tr)
    assert tr.nsteps == 3
    for s, expect in enumerate(g["steps"]):
        pairs = {tuple(sorted((src, dst))) for (src, dst, blk, n) in tr.steps[s]}
        assert pairs == {tuple(p) for p in expect["pairs"]}
        for (src, dst, blk, n) in tr.steps[s]:
            assert n == int(M * expect["size_fraction"])


def test_hd_owner_is_rank_index():
    for N in (2, 4, 8, 16):
        M = 2 * N + 1
        xs = [np.full(M, 1 << r, dtype=np.int32) for r in range(N)]
        out = cs.hd_reduce_scatter(xs, "sum", "int32")
        b = cs.chunk_bounds(M, N)
        for r in range(N):
            assert out[r].shape[0] == b[r + 1] - b[r]
            assert np.all(out[r] == (1 << N) - 1)


def test_butterfly_pairs_n8(golden):
    g = golden("butterfly_pairs_n8.json")
    tr = cs.Trace()
    cs.butterfly_all_reduce([np.zeros(5, dtype=np.int32)] * 8, "sum", "int32", tr)
    assert tr.nsteps == 3
    for s, expect in enumerate(g["steps"]):
        pairs = {tuple(sorted((src, dst))) for (src, dst, what, n) in tr.steps[s]}
        assert pairs == {tuple(p) for p in expect["pairs"]}
        for (src, dst, what, n) in tr.steps[s]:
            assert abs(src - dst) == expect["distance"] and n == 5


def test_binomial_broadcast_n8(golden):
    g = golden("binomial_broadcast_n8.json")
    tr = cs.Trace()
    cs.broadcast([np.arange(3, dtype=np.int32)] * 8, g["root"], "binomial", tr)
    got = [[[s, d] for (s, d, w, n) in step] for step in tr.steps]
    assert got == g["steps"]


def test_ring_broadcast_chain():
    tr = cs.Trace()
    cs.broadcast([np.arange(3, dtype=np.int32)] * 5, 2, "ring", tr)
    assert [[(s, d) for (s, d, w, n) in st] for st in tr.steps] == [[(2, 3)], [(3, 4)], [(4, 0)], [(0, 1)]]


def test_pairwise_alltoall_rule():
    N = 5
    C = np.arange(N * N).reshape(N, N) % 3 + 1
    sends = [np.arange(C[i].sum(), dtype=np.int32) + 100 * i for i in range(N)]
    tr = cs.Trace()
    out_pw = cs.all_to_all(sends, C, 1, pairwise=True, trace=tr)
    out_direct = cs.all_to_all(sends, C, 1, pairwise=False)
    for j in range(N):
        assert np.array_equal(out_pw[j], out_direct[j])
    assert tr.nsteps == N
    for k, step in enumerate(tr.steps):
        for (i, j, what, n) in step:
            assert j == (i + k) % N
            assert i == (j - k + N) % N


def test_step_counts():
    for N in (2, 4, 8, 16):
        M = 4 * N
        xs = [np.zeros(M, dtype=np.int32)] * N
        t = cs.Trace(); cs.ring_all_reduce(xs, "sum", "int32", t); assert t.nsteps == 2 * (N - 1)
        t = cs.Trace(); cs.ring_reduce_scatter(xs, "sum", "int32", t); assert t.nsteps == N - 1
        t = cs.Trace(); cs.hd_all_reduce(xs, "sum", "int32", t); assert t.nsteps == 2 * int(np.log2(N))
        t = cs.Trace(); cs.butterfly_all_reduce(xs, "sum", "int32", t); assert t.nsteps == int(np.log2(N))


def test_pow2_schedules_reject_other_n():
    """Halving-doubling ReduceScatter / AllGather need N = 2^k; the AllReduces
    take any N by folding the first 2r ranks in pairs (tests/test_oracle_f1.py)."""
    xs = [np.zeros(6, dtype=np.int32)] * 3
    with pytest.raises(ValueError):
        cs.hd_reduce_scatter(xs, "sum", "int32")
    with pytest.raises(ValueError):
        cs.hd_all_gather([np.zeros(2, dtype=np.int32)] * 3, "int32")
