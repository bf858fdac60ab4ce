"""GPU parity of the fused kernels when every chunk is exactly 2^k full tiles
(M = N x tile x 2^k, 16-byte aligned buffers): the kernels then take a
tile's chunk from a shift of the workgroup index instead of scanning the
chunk bounds.  AllReduce (ring, halving-doubling, butterfly, binomial tree,
pair-folded halving-doubling) and ReduceScatter (ring, halving-doubling),
bit-exact against the oracle, with the non-power-of-two neighbours of each
size for contrast."""
import sys

import numpy as np
import pytest
import torch

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import DEV, alloc_ranks, download, upload
from tests.test_gpu_parity import check_equal, inputs

pytestmark = pytest.mark.gpu
TILE = {"int32": 512, "f32": 512, "bf16": 1024}
ORACLE = {"ring": cs.ring_all_reduce, "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce,
          "tree": cs.tree_all_reduce}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sizes(N, dtype):
    t = TILE[dtype]
    return [N * t, N * t * 4, N * t * 3, N * t * 4 + 1]      # tiles per chunk 1, 4 (powers of two), 3, ragged


@pytest.mark.parametrize("dtype", ["int32", "f32", "bf16"])
@pytest.mark.parametrize("algo", ["ring", "hd", "butterfly", "tree"])
def test_all_reduce_pow2_tiles(dtype, algo):
    for N in (2, 4, 8, 16) + ((12, 5) if algo in ("ring", "hd", "tree") else ()):
        for M in _sizes(N, dtype):
            say(f"{algo} {dtype} N={N} M={M}")
            xs = inputs(N, M, dtype, "sum", N)
            send = upload(xs, dtype)
            recv = alloc_ranks(N, M, dtype)
            ccgpu.all_reduce(send, recv, algo=algo)
            torch.cuda.synchronize()
            check_equal(download(recv, dtype), ORACLE[algo](xs, "sum", dtype), f"{algo} {dtype} N={N} M={M}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo", ["ring", "hd"])
def test_reduce_scatter_pow2_tiles(dtype, algo):
    for N in (2, 4, 8, 16):
        for M in _sizes(N, dtype):
            if M % N:
                continue
            S = M // N
            say(f"reduce_scatter {algo} {dtype} N={N} M={M}")
            xs = inputs(N, M, dtype, "sum", N + 1)
            send = upload(xs, dtype)
            recv = alloc_ranks(N, S, dtype)
            ccgpu.reduce_scatter(send, recv, algo=algo)
            torch.cuda.synchronize()
            want = (cs.ring_reduce_scatter if algo == "ring" else cs.hd_reduce_scatter)(xs, "sum", dtype)
            check_equal(download(recv, dtype), want, f"rs {algo} {dtype} N={N} M={M}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("algo,fd,gs", [("ring", 1, False), ("ring", 3, False), ("ring", 1, True), ("hd", 1, False),
                                        ("butterfly", 1, False), ("ring_2port", 0, False)])
def test_stepwise_and_2port_pow2_tiles(dtype, algo, fd, gs):
    oracle = {"ring": cs.ring_all_reduce, "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce,
              "ring_2port": cs.ring2_all_reduce}[algo]
    for N in (2, 4, 8):
        for M in _sizes(N, dtype):
            say(f"{algo} fd={fd} grid_sync={gs} {dtype} N={N} M={M}")
            xs = inputs(N, M, dtype, "sum", 2 * N)
            send = upload(xs, dtype)
            recv = alloc_ranks(N, M, dtype)
            ws = ccgpu.make_workspace("all_reduce", N, M, dtype, algo, fd, DEV, grid_sync=gs)
            ccgpu.all_reduce(send, recv, algo=algo, fuse_depth=fd, workspace=ws, grid_sync=gs)
            torch.cuda.synchronize()
            if gs:
                assert not ccgpu.grid_sync_timed_out(ws)
            check_equal(download(recv, dtype), oracle(xs, "sum", dtype), f"{algo} fd={fd} {dtype} N={N} M={M}")


@pytest.mark.parametrize("algo,fd", [("ring", 0), ("ring", 1), ("ring", 3), ("hd", 1)])
def test_all_gather_pow2_tiles(algo, fd):
    dtype = "bf16"
    for N in (2, 4, 8):
        for M in _sizes(N, dtype):
            if M % N:
                continue
            S = M // N
            say(f"all_gather {algo} fd={fd} N={N} S={S}")
            xs = inputs(N, S, dtype, "sum", 5)
            send = upload(xs, dtype)
            recv = alloc_ranks(N, M, dtype)
            ccgpu.all_gather(send, recv, algo=algo, fuse_depth=fd)
            torch.cuda.synchronize()
            want = (cs.ring_all_gather if algo == "ring" else cs.hd_all_gather)(xs, dtype)
            check_equal(download(recv, dtype), want, f"ag {algo} fd={fd} N={N} S={S}")


@pytest.mark.parametrize("dims", [(2, 2, 2), (4, 2), (2, 4), (2, 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hierarchical_pow2_tiles(dims, dtype):
    N = int(np.prod(dims))
    for M in _sizes(N, dtype):
        say(f"hier {dims} {dtype} M={M}")
        xs = inputs(N, M, dtype, "sum", 7)
        send = upload(xs, dtype)
        recv = alloc_ranks(N, M, dtype)
        ccgpu.all_reduce_hierarchical(send, recv, dims)
        torch.cuda.synchronize()
        check_equal(download(recv, dtype), cs.hierarchical_all_reduce(xs, dims, "sum", dtype), f"hier {dims} M={M}")


@pytest.mark.parametrize("fd", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_int8_ef_pow2_tiles(fd, dtype):
    from oracle import compress as cp
    for N in (2, 4, 8):
        for M in _sizes(N, dtype):
            say(f"int8 ef fd={fd} {dtype} N={N} M={M}")
            g = np.random.default_rng([N, M]).standard_normal((N, M)).astype(np.float32) * 1e-2
            xs = [cs.f32_to_bf16_bits(x) for x in g] if dtype == "bf16" else list(g)
            es = [np.zeros(M, np.float32) for _ in range(N)]
            gt = upload(xs, dtype)
            et = upload(es, "f32")
            rt = alloc_ranks(N, M, dtype)
            n = ccgpu.int8_ef_workspace_size(N, M, dtype, fd)
            ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
            ccgpu.all_reduce_int8_ef(gt, et, rt, fuse_depth=fd, workspace=ws)
            torch.cuda.synchronize()
            want, we = cp.compressed_all_reduce(xs, es, 128, dtype)
            check_equal(download(rt, dtype), want, f"int8 fd={fd} {dtype} N={N} M={M}")
            check_equal(download(et, "f32"), we, f"int8 err fd={fd} {dtype} N={N} M={M}")
