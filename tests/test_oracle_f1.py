"""Pins for the tree, double binary tree, 2-port ring and the non-power-of-two
halving-doubling / butterfly schedules of the oracle: brute force against
Python-integer reductions, the step simulators against their loop-free
closed forms, the pages' step counts, tree shapes and time formulas, and the
printed ring/tree crossover example."""
import math

import numpy as np
import pytest

from oracle import ccsim as cs
from tests.test_oracle_bruteforce import _inputs, _py_reduce

NEW = {"tree": cs.tree_all_reduce, "dbt": cs.double_tree_all_reduce, "ring2": cs.ring2_all_reduce,
       "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce}
NS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 13, 16, 17]


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_new_schedules_reach_the_plain_reduction(N, op):
    for M in list(range(0, 2 * N + 3)) + [41]:
        xs = _inputs(N, M, op, 3)
        expect = [_py_reduce([int(xs[r][e]) for r in range(N)], op) for e in range(M)]
        for name, fn in NEW.items():
            out = fn(xs, op, "int32")
            for r in range(N):
                assert [int(v) for v in out[r]] == expect, (name, N, M, r)


def _floats(N, M, dtype, seed=0):
    g = np.random.default_rng([19, N, M, seed])
    xs = [(g.standard_normal(M) * (1e-3 if seed % 2 else 1.0)).astype(np.float32) for _ in range(N)]
    return [cs.f32_to_bf16_bits(x) for x in xs] if dtype == "bf16" else xs


@pytest.mark.parametrize("N", [2, 3, 5, 6, 7, 8, 11, 12, 16, 17])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_step_simulators_equal_closed_forms(N, dtype, op):
    """Each step simulator agrees bit for bit with its fold written without
    steps (float SUM and PROD depend on the association)."""
    M = 3 * N + 7
    xs = _floats(N, M, dtype, seed=N)
    vals = np.stack(xs)
    idx = np.arange(M)
    b = lambda a: np.asarray(a).view(np.uint8)
    out = cs.tree_all_reduce(xs, op, dtype)
    exp = cs.tree_fold_elements(vals, op, dtype)
    assert all(np.array_equal(b(out[r]), b(exp)) for r in range(N)), "tree"
    out = cs.double_tree_all_reduce(xs, op, dtype)
    exp = cs.dbt_fold_elements(vals, idx, M, op, dtype)
    assert all(np.array_equal(b(out[r]), b(exp)) for r in range(N)), "dbt"
    out = cs.ring2_all_reduce(xs, op, dtype)
    exp = cs.ring2_fold_elements(vals, idx, M, op, dtype)
    assert all(np.array_equal(b(out[r]), b(exp)) for r in range(N)), "ring2"
    out = cs.hd_all_reduce(xs, op, dtype)
    exp = cs.hd_fold_elements(vals, idx, M, op, dtype)
    assert all(np.array_equal(b(out[r]), b(exp)) for r in range(N)), "hd"
    out = cs.butterfly_all_reduce(xs, op, dtype)
    for r in range(N):
        assert np.array_equal(b(out[r]), b(cs.butterfly_fold_elements(vals, r, op, dtype))), ("butterfly", r)


@pytest.mark.parametrize("N", [2, 4, 8, 16])
def test_tree_equals_butterfly_for_powers_of_two(N):
    """Rank 0's binomial reduce and the butterfly's distance-1-first exchange
    build the same pairwise tree in rank order: same bits."""
    xs = _floats(N, 301, "f32", seed=5)
    t = cs.tree_all_reduce(xs, "sum", "f32")
    bf = cs.butterfly_all_reduce(xs, "sum", "f32")
    assert np.array_equal(t[0].view(np.uint32), bf[0].view(np.uint32))


def test_tree_pairs_and_step_counts():
    """[MLSys-6] "Tree AllReduce": log2 N reduce steps with N/2, N/4, ... 1
    senders (two nodes at the root), the same number of broadcast steps; an
    8-GPU group takes 2*log2(8) = 6 steps against the ring's 2*(8-1) = 14."""
    for N in (2, 4, 8, 16, 32):
        tr = cs.Trace()
        cs.tree_all_reduce([np.zeros(4, np.int32)] * N, "sum", "int32", trace=tr)
        k = int(math.log2(N))
        assert tr.nsteps == 2 * k
        assert [len(s) for s in tr.steps[:k]] == [N >> (j + 1) for j in range(k)]
        assert tr.steps[k - 1] == [(N // 2, 0, "all", 4)]
    ring, tree = cs.Trace(), cs.Trace()
    cs.ring_all_reduce([np.zeros(8, np.int32)] * 8, "sum", "int32", trace=ring)
    cs.tree_all_reduce([np.zeros(8, np.int32)] * 8, "sum", "int32", trace=tree)
    assert (ring.nsteps, tree.nsteps) == (14, 6)


@pytest.mark.parametrize("N", [2, 3, 4, 5, 6, 7, 8, 11, 16, 17, 32])
def test_double_tree_shape(N):
    """Both trees span all N ranks once, rank 0 (resp. 1) on top; for N = 2^k
    the leaves of one are the internal nodes of the other ([AR-notes],
    "算法三") and each tree has log2 N levels below its top."""
    ch1, top1, ch2, top2 = cs.dbt_trees(N)
    for ch, top in ((ch1, top1), (ch2, top2)):
        seen, todo = set(), [top]
        while todo:
            x = todo.pop()
            assert x not in seen
            seen.add(x)
            todo.extend(ch[x])
            assert len(ch[x]) <= 2 and all(0 <= y < N for y in ch[x])
        assert seen == set(range(N))
    if N & (N - 1) == 0:
        leaves1 = {x for x in range(N) if not ch1[x]}
        leaves2 = {x for x in range(N) if not ch2[x]}
        assert leaves1 == set(range(N)) - leaves2
        assert leaves1 == {x for x in range(N) if x % 2 == 1}
        dep = cs._tree_depths(ch1, top1)
        assert max(dep.values()) == int(math.log2(N))


def test_ring2_step_counts_and_time_formula():
    """[AR-notes] "2-port Ring 优化": each phase takes ceil(N/2) steps for
    even N, and with one chunk per port and step the time is
    2 ceil(N/2) (alpha + (M/N) beta) exactly when N divides M."""
    alpha, beta = 3e-6, 1e-9
    for N in (2, 4, 6, 8, 16):
        M = 4 * N
        tr = cs.Trace()
        cs.ring2_all_reduce([np.zeros(M, np.int32)] * N, "sum", "int32", trace=tr)
        assert tr.nsteps == 2 * math.ceil(N / 2)
        for st in tr.steps:                        # at most one chunk per port per rank
            ports = [(e[0], cs.ring2_port(e)) for e in st]
            assert len(ports) == len(set(ports))
        T = cs.step_time_model(tr, 4, alpha, beta, port_of=cs.ring2_port)
        assert T == pytest.approx(2 * math.ceil(N / 2) * alpha + 2 * math.ceil(N / 2) * (M * 4 / N) * beta)
    for N in (3, 5, 7):                            # odd N: (N-1)/2 steps per phase
        tr = cs.Trace()
        cs.ring2_all_reduce([np.zeros(N, np.int32)] * N, "sum", "int32", trace=tr)
        assert tr.nsteps == N - 1


@pytest.mark.parametrize("N", [3, 5, 6, 7, 12, 13])
def test_non_power_of_two_halving_doubling_cost(N):
    """[Blog] RHD, "非 2 的整数次幂场景": 2 floor(log2 p) + 2 steps and
    T = (2 floor(log2 p) + 2) alpha + (2 (p'-1)/p' + 2) n beta (no gamma term:
    the reduction arithmetic is not timed by the model)."""
    pp = 1 << (N.bit_length() - 1)
    M = 8 * pp
    tr = cs.Trace()
    cs.hd_all_reduce([np.zeros(M, np.int32)] * N, "sum", "int32", trace=tr)
    assert tr.nsteps == 2 * int(math.log2(pp)) + 2
    alpha, beta = 2e-6, 3e-10
    n = M * 4
    T = cs.step_time_model(tr, 4, alpha, beta)
    assert T == pytest.approx((2 * int(math.log2(pp)) + 2) * alpha + (2 * (pp - 1) / pp + 2) * n * beta)
    # the butterfly's variant: log2 p' full exchanges plus the two extra steps
    tb = cs.Trace()
    cs.butterfly_all_reduce([np.zeros(M, np.int32)] * N, "sum", "int32", trace=tb)
    assert tb.nsteps == int(math.log2(pp)) + 2


def test_pair_fold_uses_the_first_2r_ranks():
    """The first 2r ranks pair up (2i, 2i+1) and the rest run the power-of-two
    schedule ([AR-notes], 算法四 "非 2^k 处理"; [Blog], part1 of 2r ranks)."""
    r, active = cs._pair_fold_layout(11)
    assert r == 3 and active == [0, 2, 4, 6, 7, 8, 9, 10]
    tr = cs.Trace()
    cs.hd_all_reduce([np.zeros(16, np.int32)] * 11, "sum", "int32", trace=tr)
    assert tr.steps[0] == [(1, 0, "all", 16), (3, 2, "all", 16), (5, 4, "all", 16)]
    assert tr.steps[-1] == [(0, 1, "all", 16), (2, 3, "all", 16), (4, 5, "all", 16)]


def test_ring_tree_crossover_example():
    """[MLSys-6] "算法切换点": alpha = 5 us, beta = 50 GB/s, N = 100 give about
    3.8 MB with the log-aware form; the exact solution of T_ring = T_tree is
    of the same size, and ring/tree times cross there."""
    c = cs.ring_tree_crossover(100, 5e-6, 1 / 50e9)
    assert c["log"] / 1e6 == pytest.approx(3.76, abs=0.01)
    assert c["rough"] == pytest.approx(100 * 5e-6 * 50e9)
    a, b, N = 5e-6, 1 / 50e9, 100
    Tr = lambda M: 2 * (N - 1) * a + 2 * (N - 1) / N * M * b
    Tt = lambda M: 2 * math.log2(N) * a + 2 * math.log2(N) * M * b
    assert Tr(c["exact"]) == pytest.approx(Tt(c["exact"]))
    assert Tr(c["exact"] / 2) > Tt(c["exact"] / 2) and Tr(c["exact"] * 2) < Tt(c["exact"] * 2)
    assert 0.9 < c["exact"] / c["log"] < 1.2          # 4.08 MB exact against 3.76 MB


def test_tree_time_matches_the_tree_like_formula():
    """Step-synchronous cost of the binomial tree: 2 log2 N alpha +
    2 log2 N M beta, the pages' tree-like model ([MLSys-6], eq. T_tree-like)."""
    for N in (2, 4, 8, 16):
        M = 64
        tr = cs.Trace()
        cs.tree_all_reduce([np.zeros(M, np.int32)] * N, "sum", "int32", trace=tr)
        k = math.log2(N)
        assert cs.step_time_model(tr, 4, 1e-6, 1e-9) == pytest.approx(2 * k * 1e-6 + 2 * k * M * 4 * 1e-9)
