"""GPU parity of the split forms of the fused AllReduce against the oracle's
step simulators, every element of every rank bit for bit.  The ring: a
ReduceScatter launch that stores each chunk's fold to its owner, then an
AllGather launch from the owners (from 32 ranks of 16 MiB on).  The hierarchical AllReduce: the
nested fold stored once, to the owner of the element's flat ring chunk, then
the same AllGather (from 32 ranks of 4 MiB on).  Both sides of the size and
rank thresholds, ragged chunks and segments, unaligned and in-place buffers,
every operator."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import alloc_ranks, bits, download, upload

pytestmark = pytest.mark.gpu

F32_MIN = (16 << 20) // 4       # elements per rank where the ring splits: 4-byte elements
BF16_MIN = (16 << 20) // 2      # and bf16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(N, M, dtype, op, seed):
    g = np.random.default_rng([61, N, M, seed, len(dtype), len(op)])
    if dtype == "int32":
        lo, hi = (-2, 3) if op == "prod" else (-1000, 1001)
        return [g.integers(lo, hi, size=M, dtype=np.int32) for _ in range(N)]
    x = [(g.standard_normal(M) * 1e-2).astype(np.float32) for _ in range(N)]
    if op == "prod":
        x = [(1.0 + v).astype(np.float32) for v in x]
    return [cs.f32_to_bf16_bits(v) for v in x] if dtype == "bf16" else x


def check(N, M, dtype, op="sum", offset=0, pad=0, in_place=False, seed=0):
    say(f"split ring all_reduce {dtype} N={N} M={M} {op} offset={offset} pad={pad} in_place={in_place}")
    xs = inputs(N, M, dtype, op, seed)
    send = upload(xs, dtype, pad, offset)
    recv = send if in_place else alloc_ranks(N, M, dtype, pad, offset)
    ccgpu.all_reduce(send, recv, op=op)
    torch.cuda.synchronize()
    got = download(recv, dtype)
    del send, recv
    torch.cuda.empty_cache()
    want = cs.ring_all_reduce(xs, op, dtype)
    for r in range(N):
        assert np.array_equal(bits(got[r]), bits(want[r])), (N, M, dtype, op, offset, in_place, r)


@pytest.mark.parametrize("case", [
    (32, F32_MIN, "sum", 0, 0, False),            # the threshold: split
    (32, F32_MIN - 1, "sum", 0, 0, False),        # one element below: one launch, ragged
    (31, F32_MIN + 31 * 3, "sum", 0, 8, False),   # 31 ranks: one launch
    (64, F32_MIN + 1000, "sum", 0, 8, False),     # ragged chunks
    (33, F32_MIN + 33 * 5, "max", 1, 0, False),   # unaligned: element-wise tiles
    (40, F32_MIN + 3, "prod", 0, 4, False),
    (48, F32_MIN, "sum", 0, 0, True),             # in place
])
def test_split_ring_f32(case):
    N, M, op, offset, pad, in_place = case
    check(N, M, "f32", op, offset, pad, in_place)


@pytest.mark.parametrize("case", [
    (32, F32_MIN, "prod"),
    (47, F32_MIN + 11, "max"),
    (64, F32_MIN, "sum"),
])
def test_split_ring_int32(case):
    N, M, op = case
    check(N, M, "int32", op)


@pytest.mark.parametrize("case", [
    (32, BF16_MIN, "sum", 0, False),              # the threshold: split
    (32, BF16_MIN - 8, "sum", 0, False),          # below: one launch
    (36, BF16_MIN + 7, "sum", 0, False),          # ragged
    (33, BF16_MIN + 64, "max", 1, True),          # unaligned, in place
])
def test_split_ring_bf16(case):
    N, M, op, offset, in_place = case
    check(N, M, "bf16", op, offset, 0, in_place)


HIER_MIN = (4 << 20) // 4       # fp32 elements per rank where the hierarchical form splits


@pytest.mark.parametrize("case", [
    ((8, 8), "f32", HIER_MIN, "sum", 0, 0, False),          # the threshold: split
    ((8, 8), "f32", HIER_MIN - 1, "sum", 0, 0, False),      # below: one launch
    ((4, 4, 2), "f32", HIER_MIN + 999, "sum", 0, 8, False),  # ragged segments
    ((3, 11), "f32", HIER_MIN + 33, "prod", 0, 0, False),   # 33 ranks, odd levels
    ((2, 16), "int32", HIER_MIN, "prod", 0, 0, False),
    ((4, 8), "bf16", 2 * HIER_MIN, "max", 1, 0, False),     # bf16 at 4 MiB, unaligned
    ((2, 2, 8), "f32", HIER_MIN + 5, "sum", 0, 0, True),    # in place
    ((4, 4, 4), "f32", HIER_MIN - 64, "sum", 0, 0, False),  # below: one launch, compile-time grid
    ((4, 4, 4), "bf16", 2 * HIER_MIN, "sum", 0, 0, False),  # split, compile-time grid
    ((8, 8), "bf16", 2 * HIER_MIN - 8, "prod", 0, 0, False),
])
def test_split_hierarchical(case):
    dims, dtype, M, op, offset, pad, in_place = case
    N = math.prod(dims)
    say(f"split hierarchical all_reduce {dtype} dims={dims} M={M} {op} offset={offset} pad={pad} in_place={in_place}")
    xs = inputs(N, M, dtype, op, 7)
    send = upload(xs, dtype, pad, offset)
    recv = send if in_place else alloc_ranks(N, M, dtype, pad, offset)
    ccgpu.all_reduce_hierarchical(send, recv, dims, op=op)
    torch.cuda.synchronize()
    got = download(recv, dtype)
    del send, recv
    torch.cuda.empty_cache()
    want = cs.hierarchical_all_reduce(xs, dims, op, dtype)
    for r in range(N):
        assert np.array_equal(bits(got[r]), bits(want[r])), (dims, M, dtype, op, offset, in_place, r)


def test_split_forms_graph_replays():
    """Both launches of the split forms captured into one HIP graph: every
    replay, with eager work between them, equals the eager result."""
    gen = torch.Generator(device="cuda:0").manual_seed(62)
    x = torch.randn(32, F32_MIN + 5, generator=gen, device="cuda:0")
    h = torch.randn(64, HIER_MIN, generator=gen, device="cuda:0")
    ex, eh = torch.empty_like(x), torch.empty_like(h)
    ccgpu.all_reduce(x, ex)
    ccgpu.all_reduce_hierarchical(h, eh, (8, 8))
    y, z = torch.empty_like(x), torch.empty_like(h)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ccgpu.all_reduce(x, y)
        ccgpu.all_reduce_hierarchical(h, z, (8, 8))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ccgpu.all_reduce(x, y)
        ccgpu.all_reduce_hierarchical(h, z, (8, 8))
    for t in range(3):
        say(f"split forms graph replay {t}")
        y.fill_(3)
        z.fill_(5)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ex.view(torch.int32))
        assert torch.equal(z.view(torch.int32), eh.view(torch.int32))


def test_split_ring_seeded_sweep():
    """Seeded draws around the ring's thresholds: rank counts 28-64, element
    counts a few elements either side of 16 MiB per rank, every type and
    operator, aligned or not, against the step simulator."""
    g = np.random.default_rng(63)
    for case in range(6):
        dtype = ["f32", "bf16", "int32"][case % 3]
        es = 2 if dtype == "bf16" else 4
        N = int(g.integers(28, 65))
        M = (16 << 20) // es + int(g.integers(-40, 41))
        op = ["sum", "max", "prod"][int(g.integers(0, 3))]
        check(N, M, dtype, op, offset=int(g.integers(0, 2)), pad=int(g.integers(0, 3)) * 8, seed=case)


def test_split_hierarchical_seeded_sweep():
    """Seeded grids of 24-64 ranks in two to four levels, a few elements
    either side of 4 MiB per rank, every type and operator."""
    g = np.random.default_rng(64)
    grids = [(4, 8), (8, 4), (2, 16), (4, 4, 2), (2, 2, 2, 4), (8, 8), (4, 4, 4), (3, 8), (2, 3, 5), (6, 6)]
    for case in range(5):
        dims = grids[int(g.integers(0, len(grids)))]
        dtype = ["f32", "bf16", "int32"][case % 3]
        es = 2 if dtype == "bf16" else 4
        N, M = math.prod(dims), (4 << 20) // es + int(g.integers(-40, 41))
        op = ["sum", "max", "prod"][int(g.integers(0, 3))]
        offset = int(g.integers(0, 2))
        say(f"seeded split hierarchical {dims} {dtype} M={M} {op} offset={offset}")
        xs = inputs(N, M, dtype, op, 100 + case)
        send = upload(xs, dtype, 0, offset)
        recv = alloc_ranks(N, M, dtype, 0, offset)
        ccgpu.all_reduce_hierarchical(send, recv, dims, op=op)
        torch.cuda.synchronize()
        got = download(recv, dtype)
        del send, recv
        torch.cuda.empty_cache()
        want = cs.hierarchical_all_reduce(xs, dims, op, dtype)
        for r in range(N):
            assert np.array_equal(bits(got[r]), bits(want[r])), (dims, M, dtype, op, offset, r)
