"""Pins for the hierarchical (multi-dimensional) AllReduce of the oracle:
brute force against Python-integer reductions, the step simulator against
its closed form, reductions to the flat ring, the pages' two- and three-level
examples (group counts, per-level data volumes, the 8 x 8 GPU time budget and
the flat-ring time of the 32-rank comparison)."""
import math

import numpy as np
import pytest

from oracle import ccsim as cs
from tests.test_oracle_bruteforce import _inputs, _py_reduce

DIMS = [(2,), (5,), (2, 2), (3, 2), (2, 3), (4, 2), (3, 2, 2), (2, 2, 2), (1, 4), (4, 1), (2, 1, 3)]


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_hierarchical_reaches_the_plain_reduction(dims, op):
    N = math.prod(dims)
    for M in list(range(0, 2 * N + 3)) + [29]:
        xs = _inputs(N, M, op, 11)
        expect = [_py_reduce([int(xs[r][e]) for r in range(N)], op) for e in range(M)]
        out = cs.hierarchical_all_reduce(xs, dims, op, "int32")
        for r in range(N):
            assert [int(v) for v in out[r]] == expect, (dims, M, r)


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_step_simulator_equals_closed_form(dims, dtype, op):
    N = math.prod(dims)
    M = 5 * N + 3
    g = np.random.default_rng([3, N, M])
    xs = [(1 + 0.1 * g.standard_normal(M) if op == "prod" else g.standard_normal(M)).astype(np.float32)
          for _ in range(N)]
    if dtype == "bf16":
        xs = [cs.f32_to_bf16_bits(x) for x in xs]
    out = cs.hierarchical_all_reduce(xs, dims, op, dtype)
    cf = cs.hier_fold_elements(np.stack(xs), np.arange(M), M, dims, op, dtype)
    for r in range(N):
        assert np.array_equal(np.asarray(out[r]).view(np.uint8), np.asarray(cf).view(np.uint8)), (dims, r)


@pytest.mark.parametrize("N", [2, 3, 5, 8])
def test_one_level_is_the_flat_ring(N):
    """One level (or every other level of size 1) is the ring AllReduce; a
    single inner level under a trivial outer one is the standalone ring
    ReduceScatter followed by the ring AllGather."""
    M = 4 * N + 1
    xs = [np.random.default_rng([N, r]).standard_normal(M).astype(np.float32) for r in range(N)]
    ring = cs.ring_all_reduce(xs, "sum", "f32")
    for dims in ((N,), (1, N), (1, 1, N)):
        out = cs.hierarchical_all_reduce(xs, dims, "sum", "f32")
        assert all(np.array_equal(out[r].view(np.uint32), ring[r].view(np.uint32)) for r in range(N)), dims
    xs = [x[:4 * N] for x in xs]
    rsag = cs.ring_all_gather(cs.ring_reduce_scatter(xs, "sum", "f32"), "f32")
    for dims in ((N, 1), (1, N, 1)):          # the N-rank level is an inner one
        out = cs.hierarchical_all_reduce(xs, dims, "sum", "f32")
        assert all(np.array_equal(out[r].view(np.uint32), rsag[r].view(np.uint32)) for r in range(N)), dims


def test_blueconnect_twelve_gpu_example():
    """[AR-notes] BlueConnect, 12 GPUs as p = (3, 2, 2): 4, 6 and 6 parallel
    groups; the ReduceScatters shrink a rank's data M -> M/3 -> M/6 -> M/12
    and the AllGathers restore it in reverse order."""
    dims = (3, 2, 2)
    assert [len(cs.hier_groups(dims, i)) for i in range(3)] == [4, 6, 6]
    M = 1200
    tr = cs.Trace()
    cs.hierarchical_all_reduce([np.zeros(M, np.int32)] * 12, dims, "sum", "int32", trace=tr)
    # steps: level 0 RS (2), level 1 RS (1), top AllReduce (1 + 1), level 1 AG (1), level 0 AG (2)
    assert tr.nsteps == 2 + 1 + 2 + 1 + 2
    sizes = [{n for (_, _, _, n) in st} for st in tr.steps]
    assert sizes == [{M // 3}, {M // 3}, {M // 6}, {M // 12}, {M // 12}, {M // 6}, {M // 3}, {M // 3}]
    # the outermost level's AllReduce sends 2 x M/12 = M/6 per rank: the payload compressed 6-fold
    assert sum(n for st in tr.steps[3:5] for (s, _, _, n) in st if s == 0) == 2 * (M // 12)


def test_two_level_napkin_math():
    """[MLSys-6] Napkin Math 1.6: 8 nodes x 8 GPUs, a 1 GB gradient, 450 GB/s
    inside the node, 50 GB/s across: about 1.94 ms of ReduceScatter and as much
    AllGather inside, 4.4 ms of AllReduce across (4.375 ms without latency),
    8.3 ms in all against about 40 ms for the flat ring: a 4.8x speed-up."""
    M = 1e9
    lv = cs.multidim_time_model(M, (8, 8), (0.0, 0.0), (1 / 450e9, 1 / 50e9))
    assert lv[0] / 2 == pytest.approx(1.944e-3, abs=1e-6)
    assert lv[1] == pytest.approx(4.375e-3)
    assert sum(lv) == pytest.approx(8.26e-3, abs=0.01e-3)
    flat = cs.ring_time_model(M, 64, 0.0, 1 / 50e9)
    assert flat == pytest.approx(39.4e-3, abs=0.05e-3)
    assert flat / sum(lv) == pytest.approx(4.8, abs=0.05)


def test_two_level_formula_is_the_multidim_instance():
    """[AR-notes] eq. cc-ar-2level (G groups of L) equals the BlueConnect sum
    for dims (L, G)."""
    G, L, M = 4, 8, 100e6
    ai, ae, bi, be = 2e-6, 7e-6, 1 / 450e9, 1 / 25e9
    two = 2 * (L - 1) * ai + 2 * (L - 1) * M / L * bi + 2 * (G - 1) * ae + 2 * (G - 1) * M / (G * L) * be
    assert sum(cs.multidim_time_model(M, (L, G), (ai, ae), (bi, be))) == pytest.approx(two)


def test_flat_ring_of_the_32_rank_comparison():
    """[AR-notes] 算法五 numerical comparison: the flat ring over N = 32 for
    M = 100 MB at 25 GB/s is about 8060 us, which fixes alpha = 5 us (the
    hierarchical 1586 us needs latencies the passage does not state)."""
    assert cs.ring_time_model(100e6, 32, 5e-6, 1 / 25e9) == pytest.approx(8060e-6)


def test_top_level_traffic_is_compressed():
    """Per rank, the outermost level moves 2 (p-1)/p of M / P_(d-2): the
    payload crossing the slow level shrinks by the product of the inner
    levels ([MLSys-6], "分层全归约": M/G instead of M per GPU)."""
    dims = (4, 3)
    M = 1200
    tr = cs.Trace()
    cs.hierarchical_all_reduce([np.zeros(M, np.int32)] * 12, dims, "sum", "int32", trace=tr)
    top = tr.steps[3:3 + 2 * (3 - 1)]
    sent0 = sum(n for st in top for (s, _, _, n) in st if s == 0)
    assert sent0 == 2 * (3 - 1) * (M // 4) // 3
