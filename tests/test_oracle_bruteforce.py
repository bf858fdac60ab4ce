"""Brute force on tiny inputs: every schedule of the oracle reaches the plain
definition B_i = (+)_j A_j for operators that are exact (integer SUM/PROD with
wrap, integer and float MAX), computed here with Python integers and loops."""
import itertools

import numpy as np
import pytest

from oracle import ccsim as cs

NS = [2, 3, 4, 5, 6, 7, 8, 16]


def _wrap32(v):
    return (v + 2 ** 31) % 2 ** 32 - 2 ** 31


def _py_reduce(cols, op):
    if op == "sum":
        return _wrap32(sum(cols))
    if op == "max":
        return max(cols)
    acc = 1
    for v in cols:
        acc = _wrap32(acc * v)
    return acc


def _inputs(N, M, op, seed):
    g = np.random.default_rng([7, N, M, seed])
    if op == "prod":
        return [g.integers(-40000, 40000, size=M, dtype=np.int32) for _ in range(N)]
    return [g.integers(-2 ** 31, 2 ** 31 - 1, size=M, dtype=np.int64).astype(np.int32) for _ in range(N)]


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_all_reduce_all_schedules_exact(N, op):
    algos = [cs.ring_all_reduce]
    if N & (N - 1) == 0:
        algos += [cs.hd_all_reduce, cs.butterfly_all_reduce]
    for M in range(0, 3 * N + 3):
        xs = _inputs(N, M, op, 0)
        expect = [_py_reduce([int(xs[r][e]) for r in range(N)], op) for e in range(M)]
        for fn in algos:
            out = fn(xs, op, "int32")
            for r in range(N):
                assert out[r].dtype == np.int32
                assert [int(v) for v in out[r]] == expect, (fn.__name__, N, M, r)


@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_reduce_scatter_exact_and_rs_then_ag_is_ar(N, op):
    rs_fns = [cs.ring_reduce_scatter] + ([cs.hd_reduce_scatter] if N & (N - 1) == 0 else [])
    ag_fns = [cs.ring_all_gather] + ([cs.hd_all_gather] if N & (N - 1) == 0 else [])
    for S in range(0, 4):
        M = N * S
        xs = _inputs(N, M, op, 1)
        expect = [_py_reduce([int(xs[r][e]) for r in range(N)], op) for e in range(M)]
        for rs in rs_fns:
            shards = rs(xs, op, "int32")
            for r in range(N):
                assert [int(v) for v in shards[r]] == expect[r * S:(r + 1) * S]
            for ag in ag_fns:
                full = ag(shards, "int32")
                ar = cs.ring_all_reduce(xs, op, "int32")
                for r in range(N):
                    assert np.array_equal(full[r], ar[r])


@pytest.mark.parametrize("N", [2, 3, 4, 7, 8])
def test_all_gather_adjoint_of_reduce_scatter(N):
    """<AG x, y> = <x, RS y> for the SUM ReduceScatter (the two maps are
    adjoint; a wrong chunk-to-rank assignment in either breaks it)."""
    g = np.random.default_rng(11)
    for S in (1, 2, 5):
        x = [g.integers(-50, 50, size=S, dtype=np.int32) for _ in range(N)]
        y = [g.integers(-50, 50, size=N * S, dtype=np.int32) for _ in range(N)]
        agx = cs.ring_all_gather(x, "int32")
        rsy = cs.ring_reduce_scatter(y, "sum", "int32")
        lhs = sum(int(np.dot(agx[r].astype(np.int64), y[r].astype(np.int64))) for r in range(N))
        rhs = sum(int(np.dot(x[r].astype(np.int64), rsy[r].astype(np.int64))) for r in range(N))
        assert lhs == rhs


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
def test_all_to_all_blocked_transpose_and_round_trip(N):
    g = np.random.default_rng([3, N])
    for row in (1, 3):
        C = g.integers(0, 4, size=(N, N))
        sends = [g.integers(-1000, 1000, size=int(C[i].sum()) * row, dtype=np.int32) for i in range(N)]
        recv = cs.all_to_all(sends, C, row)
        # brute force: walk the send buffers block by block
        for j in range(N):
            expect = []
            for i in range(N):
                start = int(C[i, :j].sum()) * row
                expect += list(sends[i][start:start + int(C[i, j]) * row])
            assert list(recv[j]) == expect
        back = cs.all_to_all(recv, C.T, row)
        for i in range(N):
            assert np.array_equal(back[i], sends[i])


def test_float_max_every_schedule_equals_plain():
    g = np.random.default_rng(5)
    for N in (2, 4, 8):
        for M in (1, 7, 33):
            xs = [g.standard_normal(M).astype(np.float32) for _ in range(N)]
            xs[0][0] = np.nan if M > 3 else xs[0][0]
            plain = cs.plain_reduce(xs, "max", "f32")
            for fn in (cs.ring_all_reduce, cs.hd_all_reduce, cs.butterfly_all_reduce):
                out = fn(xs, "max", "f32")
                for r in range(N):
                    assert np.array_equal(out[r].view(np.uint32), plain.view(np.uint32))


def test_broadcast_every_root():
    for N in (1, 2, 3, 6, 8):
        xs = [np.arange(4, dtype=np.int32) + 10 * r for r in range(N)]
        for root in range(N):
            for sch in ("ring", "binomial"):
                out = cs.broadcast(xs, root, sch)
                for r in range(N):
                    assert np.array_equal(out[r], xs[root])
