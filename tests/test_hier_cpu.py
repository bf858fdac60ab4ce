"""Host logic of the hierarchical AllReduce, without a GPU: the records
cc_hierarchical_plan returns -- the operations the stepwise kernels perform --
replayed with NumPy must give the oracle's bits for every rank grid; no record
of a step touches what another writes; per-level traffic equals what the
oracle's trace counts per level and the BlueConnect per-level volumes;
argument checks and workspace sizes."""
import ctypes
import math

import numpy as np
import pytest

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.test_plan_cpu import _inputs, _touches, replay

DIMS = [(2, 2), (3, 2), (2, 3), (4, 2), (2, 4), (3, 3), (3, 2, 2), (2, 2, 2), (2, 3, 2), (2, 2, 2, 2),
        (4, 4), (8, 2), (2, 8), (8, 8), (4, 1), (1, 4), (2, 1, 3), (3, 1), (1, 3, 1), (5,), (1, 2, 1, 3)]


@pytest.mark.parametrize("dims", DIMS)
def test_hier_plan_replay_matches_oracle(dims):
    N = math.prod(dims)
    for M in (1, N - 1, N + 1, 3 * N + 5, 97):
        recs = ccgpu.hierarchical_plan(dims, M)
        for dtype, op, modes in (("int32", "sum", ("recv", "in_place")), ("int32", "prod", ("recv",)),
                                 ("f32", "sum", ("recv", "in_place")), ("f32", "max", ("recv",)),
                                 ("bf16", "sum", ("staged",)), ("bf16", "prod", ("staged",))):
            xs = _inputs(N, M, dtype, op, M)
            expect = cs.hierarchical_all_reduce(xs, dims, op, dtype)
            for mode in modes:
                got = replay(recs, xs, op, dtype, mode)
                for r in range(N):
                    assert np.array_equal(np.asarray(got[r]).view(np.uint8), np.asarray(expect[r]).view(np.uint8)), \
                        (dims, M, dtype, op, mode, r)


@pytest.mark.parametrize("dims", DIMS)
def test_hier_plan_steps_are_race_free(dims):
    N = math.prod(dims)
    for M in (1, N + 1, 4 * N + 3):
        recs = ccgpu.hierarchical_plan(dims, M)
        steps = {}
        for r in recs:
            assert r["lo"] + r["len"] <= M and r["len"] > 0, r
            assert 0 <= r["dst"] < N and 0 <= r["in1"] < N and 0 <= r["in2"] < N, r
            steps.setdefault(r["step"], []).append(_touches(r))
        for s, ops in steps.items():
            for i, (ri, wi) in enumerate(ops):
                for j, (rj, wj) in enumerate(ops):
                    if i == j:
                        continue
                    for (x, a0, a1) in wi:
                        for (y, b0, b1) in rj + wj:
                            assert not (x == y and a0 < b1 and b0 < a1), (dims, M, s, i, j)


def _oracle_level_traffic(dims, M):
    """Largest per-rank element count sent at each level, from the oracle's
    trace: inner levels' ReduceScatter steps first (p - 1 each), the
    outermost level's AllReduce (2 (p - 1)), then the AllGathers in reverse
    order; levels of size 1 take no step."""
    N = math.prod(dims)
    tr = cs.Trace()
    cs.hierarchical_all_reduce([np.zeros(M, np.int32)] * N, dims, "sum", "int32", trace=tr)
    d = len(dims)
    order = [(i, dims[i] - 1) for i in range(d - 1)] + [(d - 1, 2 * (dims[-1] - 1))] + \
        [(i, dims[i] - 1) for i in range(d - 2, -1, -1)]
    sent = [[0] * N for _ in range(d)]
    k = 0
    for lvl, n in order:
        for st in tr.steps[k:k + n]:
            for (src, _, _, cnt) in st:
                sent[lvl][src] += cnt
        k += n
    assert k == len(tr.steps)
    return [max(v) for v in sent]


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("dtype", ["int32", "bf16"])
def test_level_traffic_matches_oracle_trace(dims, dtype):
    for M in (64, 3 * math.prod(dims) + 1, 1000):
        got = ccgpu.hierarchical_traffic(dims, M, dtype)
        want = _oracle_level_traffic(dims, M)
        assert [b for b, _ in got] == [w * ccgpu.ESIZE[dtype] for w in want], (dims, M)
        assert [s for _, s in got] == [2 * (p - 1) for p in dims]


def test_blueconnect_per_level_volumes():
    """AllReduce notes, BlueConnect: level i moves 2 (p_i - 1) / p_i of the
    M / P_(i-1) elements it works on; (3, 2, 2) on 1200 elements gives 1600,
    400 and 200 elements per rank."""
    got = ccgpu.hierarchical_traffic((3, 2, 2), 1200, "f32")
    assert got == [(1600 * 4, 4), (400 * 4, 2), (200 * 4, 2)]
    # compare with the oracle's time model at alpha = 0, beta = 1 s/byte
    lv = cs.multidim_time_model(1200 * 4, (3, 2, 2), (0.0, 0.0, 0.0), (1.0, 1.0, 1.0))
    assert [b for b, _ in got] == pytest.approx(lv)


def test_one_outermost_level_is_the_ring_plan():
    """A lone outermost level is the flat ring AllReduce: its plan records
    reach the oracle's ring AllReduce."""
    for dims in ((6,), (1, 6), (1, 1, 6)):
        xs = _inputs(6, 41, "f32", "sum", 1)
        got = replay(ccgpu.hierarchical_plan(dims, 41), xs, "sum", "f32", "recv")
        ring = cs.ring_all_reduce(xs, "sum", "f32")
        assert all(np.array_equal(got[r].view(np.uint32), ring[r].view(np.uint32)) for r in range(6))


def _ws(dims, fd, M, dtype):
    return ccgpu.hierarchical_workspace_size(dims, M, dtype, fd)


def test_workspace_sizes():
    M = 1000
    assert _ws((4, 2), 0, M, "bf16") == 0
    assert _ws((4, 2), 1, M, "f32") == 0 and _ws((4, 2), 1, M, "int32") == 0
    assert _ws((4, 2), 1, M, "bf16") == 8 * 4096          # fp32 partials per rank, 256-byte rows
    assert _ws((2, 2, 2), 3, 1 << 20, "bf16") == 8 * (4 << 20)
    # a lone outermost level sizes as the ring AllReduce
    assert _ws((1, 8), 1, M, "bf16") == ccgpu.workspace_size("all_reduce", 8, M, "bf16", "ring", 1)
    assert _ws((1, 8), 7, M, "bf16") == ccgpu.workspace_size("all_reduce", 8, M, "bf16", "ring", 7) == 0
    # a lone inner level runs descriptor steps
    assert _ws((8, 1), 1, M, "bf16") == 8 * 4096
    assert _ws((1,), 1, M, "bf16") == 0


def _call(dims, count=100, dtype=1, op=0, cfg=None, send=None, recv=None):
    L = ccgpu.load()
    nd = len(dims)
    arr = (ctypes.c_int * max(nd, 1))(*dims)
    N = max(1, math.prod(dims)) if dims else 1
    s = send or ccgpu.RankBuf(1 << 20, 1 << 16)
    r = recv or ccgpu.RankBuf(1 << 30, 1 << 16)
    return L.cc_all_reduce_hierarchical(s, r, count, dtype, op, nd, arr if nd else None,
                                        ctypes.byref(cfg) if cfg else None, None)


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-device status")
def test_argument_checks():
    E = ccgpu
    assert _call((4, 2)) == E.CC_ERR_NO_DEVICE
    assert _call((4, 2), send=ccgpu.RankBuf(1 << 20, 1 << 16), recv=ccgpu.RankBuf(1 << 20, 1 << 16)) == \
        E.CC_ERR_NO_DEVICE                                   # in place
    assert _call(()) == E.CC_ERR_INVALID_ARG                 # ndims 0
    assert _call((1,) * 9) == E.CC_ERR_INVALID_ARG           # ndims 9
    assert _call((4, 0)) == E.CC_ERR_INVALID_ARG
    assert _call((4, -1)) == E.CC_ERR_INVALID_ARG
    assert _call((8, 9)) == E.CC_ERR_INVALID_ARG             # 72 ranks
    assert _call((2, 2, 2, 2, 2)) == E.CC_ERR_UNSUPPORTED    # five levels of size > 1
    assert _call((2, 2, 1, 2, 2, 1)) == E.CC_ERR_NO_DEVICE   # four of them
    assert _call((4, 2), dtype=3) == E.CC_ERR_INVALID_ARG
    assert _call((4, 2), op=3) == E.CC_ERR_INVALID_ARG
    assert _call((4, 2), cfg=E.Config(1, 0, None, 0, 0, 0)) == E.CC_ERR_UNSUPPORTED   # halving-doubling
    assert _call((4, 2), cfg=E.Config(0, 1, None, 0, 0, 1)) == E.CC_ERR_UNSUPPORTED   # grid_sync
    assert _call((4, 2), cfg=E.Config(0, 1, None, 0, 0, 0), dtype=2) == E.CC_ERR_INVALID_ARG  # no bf16 workspace
    assert _call((4, 2), count=0) == E.CC_OK
    # overlapping rank buffers, recv rows too short
    assert _call((4, 2), send=ccgpu.RankBuf(1 << 20, 1 << 16), recv=ccgpu.RankBuf((1 << 20) + 64, 1 << 16)) == \
        E.CC_ERR_INVALID_ARG
    assert _call((4, 2), count=1 << 16, recv=ccgpu.RankBuf(1 << 30, 1 << 10)) == E.CC_ERR_INVALID_ARG


def test_plan_and_traffic_checks():
    L = ccgpu.load()
    n = ctypes.c_size_t(0)
    one = (ctypes.c_int * 2)(1, 1)
    assert L.cc_hierarchical_plan(2, one, 10, None, 0, ctypes.byref(n)) == ccgpu.CC_ERR_UNSUPPORTED
    d = (ctypes.c_int * 2)(4, 2)
    assert L.cc_hierarchical_plan(2, d, 10, None, 0, ctypes.byref(n)) == ccgpu.CC_OK and n.value > 0
    few = (ccgpu.PlanOp * 1)()
    assert L.cc_hierarchical_plan(2, d, 10, few, 1, ctypes.byref(n)) == ccgpu.CC_ERR_INVALID_ARG
    b = (ctypes.c_uint64 * 2)()
    s = (ctypes.c_int * 2)()
    assert L.cc_hierarchical_traffic(2, one, 10, 1, b, s) == ccgpu.CC_OK and list(b) == [0, 0]
    assert L.cc_hierarchical_traffic(2, d, 10, 5, b, s) == ccgpu.CC_ERR_INVALID_ARG
    assert L.cc_hierarchical_traffic(2, d, 10, 1, None, s) == ccgpu.CC_ERR_INVALID_ARG


def test_plan_step_count():
    """Every level of size p takes 2 (p - 1) steps."""
    for dims in DIMS:
        recs = ccgpu.hierarchical_plan(dims, 10 * math.prod(dims))
        assert max(r["step"] for r in recs) + 1 == sum(2 * (p - 1) for p in dims), dims
