"""Collectives captured into a HIP graph replay correctly: several replays,
with eager work and synchronizations between them, each equal to the eager
result (the kernels record no memset nodes)."""
import numpy as np
import pytest
import torch

from ring_allreduce_reduction_02_amd import ccgpu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("dtype,algo,fd", [(torch.float32, "ring", 0), (torch.float32, "ring", 1),
                                           (torch.bfloat16, "ring", 1), (torch.bfloat16, "hd", 1),
                                           (torch.float32, "butterfly", 0)])
def test_all_reduce_graph_replays(dtype, algo, fd):
    N, M = 8, 300_001
    g = torch.Generator(device=DEV).manual_seed(3)
    x = (torch.randn(N, M, generator=g, device=DEV) * 1e-2).to(dtype)
    name = "f32" if dtype == torch.float32 else "bf16"
    ws = ccgpu.make_workspace("all_reduce", N, M, name, algo, fd, DEV)
    eager = torch.empty_like(x)
    ccgpu.all_reduce(x, eager, algo=algo, fuse_depth=fd, workspace=ws)
    y = torch.empty_like(x)
    graph = capture(lambda: ccgpu.all_reduce(x, y, algo=algo, fuse_depth=fd, workspace=ws))
    iview = torch.int16 if dtype == torch.bfloat16 else torch.int32
    for _ in range(3):
        y.fill_(7)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(iview), eager.view(iview))


def test_rs_ag_buckets_a2a_graph_replays():
    N, S = 8, 40_000
    g = torch.Generator(device=DEV).manual_seed(4)
    x = torch.randn(N, N * S, generator=g, device=DEV)
    shard, full = torch.empty(N, S, device=DEV), torch.empty(N, N * S, device=DEV)
    ccgpu.reduce_scatter(x, shard)
    ccgpu.all_gather(shard, full)
    e_shard, e_full = shard.clone(), full.clone()
    offs, cnts = [0, 5000, 70_000], [4000, 60_000, 9_000]
    bk = torch.empty_like(x)
    ccgpu.all_reduce_buckets(x, bk, offs, cnts)
    e_bk = bk.clone()
    C = [[(i + j) % 5 for j in range(N)] for i in range(N)]
    a2a_in = torch.randn(N, 64 * 40, generator=g, device=DEV)
    a2a_out = torch.zeros(N, 64 * 40, device=DEV)
    ccgpu.all_to_all(a2a_in, a2a_out, C, 64)
    e_a2a = a2a_out.clone()

    def work():
        ccgpu.reduce_scatter(x, shard)
        ccgpu.all_gather(shard, full)
        ccgpu.all_reduce_buckets(x, bk, offs, cnts)
        ccgpu.all_to_all(a2a_in, a2a_out, C, 64, fuse_depth=1)
    graph = capture(work)
    for _ in range(3):
        for t in (shard, full, bk, a2a_out):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(shard, e_shard) and torch.equal(full, e_full)
        for o, c in zip(offs, cnts):
            assert torch.equal(bk[:, o:o + c], e_bk[:, o:o + c])
        assert torch.equal(a2a_out, e_a2a)
