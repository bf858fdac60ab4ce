"""GPU parity of the hierarchical (multi-dimensional) AllReduce, fused and
stepwise, against the oracle element by element (bit-exact): rank grids of
two to four levels, levels of size 1, ragged sizes and unaligned strides, in
place, a lone outermost level (the flat ring), a large size checked at
sampled elements against the oracle's closed form (segment boundaries
included), and HIP graph replays of the descriptor steps."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import DEV, alloc_ranks, bits, download, upload
from tests.test_gpu_parity import SIZES, check_equal, inputs

pytestmark = pytest.mark.gpu

DIMS = [(2, 2), (4, 2), (2, 4), (2, 2, 2), (3, 2, 2), (2, 3), (8, 2), (2, 2, 2, 2), (4, 1), (1, 4), (2, 1, 3), (8, 8),
        (4, 4, 4), (2, 1, 2, 2)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(xs, dims, dtype, op, fd, pad=0, in_place=False, blocks_per_cu=0):
    N, M = len(xs), len(xs[0])
    assert N == math.prod(dims)
    send = upload(xs, dtype, pad)
    recv = send if in_place else alloc_ranks(N, M, dtype, pad)
    ws = ccgpu.make_hierarchical_workspace(dims, M, dtype, fd, DEV)
    ccgpu.all_reduce_hierarchical(send, recv, dims, op=op, fuse_depth=fd, workspace=ws,
                                  blocks_per_cu=blocks_per_cu)
    torch.cuda.synchronize()
    return download(recv, dtype)


@pytest.mark.parametrize("fd", [0, 1])
@pytest.mark.parametrize("dtype", ["int32", "f32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_hierarchical_parity(fd, dtype, op):
    for dims in DIMS:
        N = math.prod(dims)
        for M in SIZES:
            pad = 3 if M % 2 else 0
            say(f"hier fd={fd} {dtype} {op} dims={dims} M={M} pad={pad}")
            xs = inputs(N, M, dtype, op, N)
            check_equal(run(xs, dims, dtype, op, fd, pad), cs.hierarchical_all_reduce(xs, dims, op, dtype),
                        f"hier fd={fd} {dtype} {op} dims={dims} M={M}")


@pytest.mark.parametrize("fd", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hierarchical_in_place(fd, dtype):
    dims, M = (4, 2), 20485
    xs = inputs(8, M, dtype, "sum", 3)
    say(f"hier fd={fd} {dtype} in place")
    check_equal(run(xs, dims, dtype, "sum", fd, in_place=True), cs.hierarchical_all_reduce(xs, dims, "sum", dtype),
                "hier in place")


@pytest.mark.parametrize("bpc", [1, 3])
def test_hierarchical_occupancy_caps(bpc):
    dims, M = (2, 2, 2), 200_003
    xs = inputs(8, M, "f32", "sum", 4)
    say(f"hier blocks_per_cu={bpc}")
    check_equal(run(xs, dims, "f32", "sum", 0, blocks_per_cu=bpc), cs.hierarchical_all_reduce(xs, dims, "sum", "f32"),
                f"hier blocks_per_cu={bpc}")


@pytest.mark.parametrize("fd", [0, 1])
def test_lone_outermost_level_is_the_flat_ring(fd):
    N, M = 8, 20485
    gen = torch.Generator(device=DEV).manual_seed(23)
    send = torch.randn(N, M, generator=gen, device=DEV)
    a = torch.empty_like(send)
    b = torch.empty_like(send)
    say(f"hier (1, 8) fd={fd} against the ring")
    ccgpu.all_reduce_hierarchical(send, a, (1, N), fuse_depth=fd)
    ccgpu.all_reduce(send, b, algo="ring", fuse_depth=fd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def _segment_marks(M, dims):
    """Every nested chunk boundary: the level-0 chunks of [0, M), each split
    into its level-1 chunks, and so on."""
    spans = [(0, M)]
    marks = set()
    for p in dims:
        nx = []
        for lo, hi in spans:
            b = cs.chunk_bounds(hi - lo, p)
            for c in range(p):
                nx.append((lo + b[c], lo + b[c + 1]))
                marks.add(lo + b[c])
        spans = nx
    return np.array(sorted(marks))


@pytest.mark.parametrize("dims", [(4, 2), (2, 4), (2, 2, 2), (8, 8), (4, 4, 4), (3, 1, 2, 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hierarchical_large_sampled(dims, dtype):
    """Many tiles per segment: fused and stepwise give the same bits
    everywhere, and the oracle's closed form at sampled elements."""
    N = math.prod(dims)
    M = (1 << 22) + 4099 if N <= 16 else (1 << 20) + 4099
    gen = torch.Generator(device=DEV).manual_seed(24)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    send = (torch.randn(N, M, generator=gen, device=DEV) * 1e-3).to(tdt)
    a = torch.empty_like(send)
    b = torch.empty_like(send)
    say(f"hier {dtype} large dims={dims} M={M}")
    ccgpu.all_reduce_hierarchical(send, a, dims, fuse_depth=0)
    ws = ccgpu.make_hierarchical_workspace(dims, M, dtype, 1, DEV)
    ccgpu.all_reduce_hierarchical(send, b, dims, fuse_depth=1, workspace=ws)
    torch.cuda.synchronize()
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(a.view(iv), b.view(iv))
    rng = np.random.default_rng(6)
    marks = _segment_marks(M, dims)
    idx = np.unique(np.concatenate([rng.integers(0, M, 300), marks, marks - 1]))
    idx = idx[(idx >= 0) & (idx < M)]
    ti = torch.from_numpy(idx).to(DEV)
    vals = np.stack(download(send.index_select(1, ti), dtype))
    got = download(a.index_select(1, ti), dtype)
    exp = cs.hier_fold_elements(vals, idx, M, dims, "sum", dtype)
    for r in range(N):
        assert np.array_equal(bits(got[r]), bits(exp)), (dims, r)


def test_hierarchical_steps_graph_replays():
    """The stepwise hierarchical AllReduce (descriptor steps) captured in a
    HIP graph: every replay equals the eager call."""
    dims, M = (4, 2), 200_003
    gen = torch.Generator(device=DEV).manual_seed(25)
    send = (torch.randn(8, M, generator=gen, device=DEV) * 1e-3).to(torch.bfloat16)
    ref = torch.empty_like(send)
    out = torch.empty_like(send)
    ws = ccgpu.make_hierarchical_workspace(dims, M, "bf16", 1, DEV)
    ccgpu.all_reduce_hierarchical(send, ref, dims, fuse_depth=1, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ccgpu.all_reduce_hierarchical(send, out, dims, fuse_depth=1, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ccgpu.all_reduce_hierarchical(send, out, dims, fuse_depth=1, workspace=ws)
    for k in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"hier graph replay {k}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), k
