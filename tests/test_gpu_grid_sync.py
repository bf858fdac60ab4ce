"""The stepwise ring AllReduce in one launch (grid_sync): workgroups take the
passes' tiles from an ordered queue and no tile of a pass starts before the
previous pass is complete.  It must give the oracle's ring bits, the same bits
as the kernel-per-pass schedule, and leave the wait timeout flag clear --
also when the grid is far larger than what can be resident, and when few
workgroups per CU are allowed."""
import sys

import numpy as np
import pytest
import torch

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import DEV, alloc_ranks, bits, download, upload
from tests.test_gpu_parity import SIZES, check_equal, inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(xs, dtype, op, fd, pad=0, in_place=False):
    N, M = len(xs), len(xs[0])
    send = upload(xs, dtype, pad)
    recv = send if in_place else alloc_ranks(N, M, dtype, pad)
    ws = ccgpu.make_workspace("all_reduce", N, M, dtype, "ring", fd, DEV, grid_sync=True)
    ccgpu.all_reduce(send, recv, op=op, fuse_depth=fd, workspace=ws, grid_sync=True)
    torch.cuda.synchronize()
    if ws is not None:
        assert not ccgpu.grid_sync_timed_out(ws)
    return download(recv, dtype)


@pytest.mark.parametrize("dtype", ["int32", "f32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "max", "prod"])
def test_grid_sync_parity(dtype, op):
    for N in (2, 3, 5, 8, 16):
        for fd in sorted({1, 2, N - 1}):
            for M in SIZES:
                pad = 3 if M % 2 else 0
                say(f"grid_sync {dtype} {op} N={N} fd={fd} M={M} pad={pad}")
                xs = inputs(N, M, dtype, op, fd)
                check_equal(run(xs, dtype, op, fd, pad), cs.ring_all_reduce(xs, op, dtype),
                            f"grid_sync {dtype} {op} N={N} fd={fd} M={M}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grid_sync_in_place(dtype):
    N, M = 8, 20485
    xs = inputs(N, M, dtype, "sum", 7)
    say(f"grid_sync in place {dtype}")
    check_equal(run(xs, dtype, "sum", 1, in_place=True), cs.ring_all_reduce(xs, "sum", dtype), "in place")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grid_sync_many_tiles_per_workgroup(dtype):
    """More tiles than resident workgroups, so each claim holds several tiles
    and data crosses workgroups between passes: equal to the kernel-per-pass
    schedule everywhere and to the oracle's ring fold at sampled elements."""
    N, M = 8, (1 << 23) + 4099
    gen = torch.Generator(device=DEV).manual_seed(11)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    send = (torch.randn(N, M, generator=gen, device=DEV) * 1e-3).to(tdt)
    a = torch.empty_like(send)
    b = torch.empty_like(send)
    say(f"grid_sync large {dtype} N={N} M={M}")
    ws1 = ccgpu.make_workspace("all_reduce", N, M, dtype, "ring", 1, DEV)
    ccgpu.all_reduce(send, a, fuse_depth=1, workspace=ws1)
    ws2 = ccgpu.make_workspace("all_reduce", N, M, dtype, "ring", 1, DEV, grid_sync=True)
    ccgpu.all_reduce(send, b, fuse_depth=1, workspace=ws2, grid_sync=True)
    torch.cuda.synchronize()
    assert not ccgpu.grid_sync_timed_out(ws2)
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(a.view(iv), b.view(iv))
    rng = np.random.default_rng(3)
    bnd = np.array(cs.chunk_bounds(M, N))
    idx = np.unique(np.concatenate([rng.integers(0, M, 500), bnd[1:-1], bnd[1:-1] - 1, [0, M - 1]]))
    ti = torch.from_numpy(idx).to(DEV)
    vals = download(send.index_select(1, ti), dtype)
    got = download(b.index_select(1, ti), dtype)
    exp = cs.ring_fold_elements(np.stack(vals), idx, M, "sum", dtype)
    for r in range(N):
        assert np.array_equal(bits(got[r]), bits(exp)), r


@pytest.mark.parametrize("bpc", [1, 3, 16])
def test_grid_sync_occupancy_caps(bpc):
    """Few or many workgroups per CU: the ordered queue needs no co-residency."""
    N, M = 8, 1 << 22
    gen = torch.Generator(device=DEV).manual_seed(13)
    send = (torch.randn(N, M, generator=gen, device=DEV) * 1e-3).to(torch.bfloat16)
    a = torch.empty_like(send)
    b = torch.empty_like(send)
    say(f"grid_sync bf16 N={N} M={M} blocks_per_cu={bpc}")
    ws1 = ccgpu.make_workspace("all_reduce", N, M, "bf16", "ring", 1, DEV)
    ccgpu.all_reduce(send, a, fuse_depth=1, workspace=ws1)
    ws2 = ccgpu.make_workspace("all_reduce", N, M, "bf16", "ring", 1, DEV, grid_sync=True)
    ccgpu.all_reduce(send, b, fuse_depth=1, workspace=ws2, grid_sync=True, blocks_per_cu=bpc)
    torch.cuda.synchronize()
    assert not ccgpu.grid_sync_timed_out(ws2)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_grid_sync_graph_replays():
    """Captured with its clearing kernel into a HIP graph and replayed with
    eager work in between; every replay equals the eager call."""
    N, M = 8, 300_001
    gen = torch.Generator(device=DEV).manual_seed(12)
    send = torch.randn(N, M, generator=gen, device=DEV) * 1e-3
    ref = torch.empty_like(send)
    out = torch.empty_like(send)
    ws = ccgpu.make_workspace("all_reduce", N, M, "f32", "ring", 2, DEV, grid_sync=True)
    ccgpu.all_reduce(send, ref, fuse_depth=2, workspace=ws, grid_sync=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ccgpu.all_reduce(send, out, fuse_depth=2, workspace=ws, grid_sync=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("grid_sync graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ccgpu.all_reduce(send, out, fuse_depth=2, workspace=ws, grid_sync=True)
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert not ccgpu.grid_sync_timed_out(ws), i
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), i
