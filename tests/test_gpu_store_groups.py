"""GPU parity of the copy paths that share or widen a tile's work, against the
oracle, bit for bit: the standalone AllGather whose tile stores are split
between two groups of threads (8-20 and more than 40 ranks; one group
elsewhere, on both sides of every boundary), and the copy-descriptor kernel
that moves two 16-byte vectors per thread (blocks that end in either half of
a 4 KiB tile, unaligned blocks, fills), for explicit and default occupancy."""
import sys

import numpy as np
import pytest
import torch

from oracle import alltoall as aa
from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import alloc_ranks, bits, download, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def values(n, dtype, seed):
    """n seeded values of dtype (bf16 as raw 16-bit patterns: a copy moves
    any pattern)."""
    g = np.random.default_rng([53, n, seed, len(dtype)])
    if dtype == "int32":
        return g.integers(-1000, 1000, size=n, dtype=np.int32)
    if dtype == "bf16":
        return g.integers(0, 1 << 16, size=n, dtype=np.uint16)
    return g.standard_normal(n).astype(np.float32)


def same(got, want, ctx):
    for r in range(len(want)):
        assert np.array_equal(bits(got[r]), bits(want[r])), f"{ctx}: rank {r} differs"


@pytest.mark.parametrize("N", [7, 8, 12, 16, 20, 21, 40, 41, 48, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "int32"])
def test_all_gather_store_groups(N, dtype):
    for S in (1, 7, 1024, 3001):
        for pad, offset in ((0, 0), (8, 0), (3, 1)):
            for bpc in (0, 1):
                say(f"all_gather N={N} {dtype} S={S} pad={pad} offset={offset} bpc={bpc}")
                shards = [values(S, dtype, 100 * r + S) for r in range(N)]
                send = upload(shards, dtype, pad, offset)
                recv = alloc_ranks(N, N * S, dtype, pad, offset)
                ccgpu.all_gather(send, recv, blocks_per_cu=bpc)
                torch.cuda.synchronize()
                same(download(recv, dtype), cs.ring_all_gather(shards, dtype), f"ag N={N} S={S} bpc={bpc}")


# block sizes around the copy kernel's 2 KiB halves and 4 KiB tiles, in bytes
EDGE_BYTES = [0, 16, 2032, 2048, 2064, 4080, 4096, 4112, 6144, 8208]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fd", [0, 1])
def test_all_to_all_tile_edges(dtype, fd):
    es = 4 if dtype == "f32" else 2
    g = np.random.default_rng([54, fd, es])
    for case in range(12):
        P = int(g.integers(2, 9))
        C = np.array([[EDGE_BYTES[int(g.integers(0, len(EDGE_BYTES)))] // es for _ in range(P)] for _ in range(P)])
        if case % 3 == 2:
            C[C > 0] += 1            # odd element counts: unaligned blocks
        bpc = int(g.choice([0, 4, 16]))
        say(f"a2a {dtype} fd={fd} case={case} P={P} bpc={bpc}")
        sends = [values(int(C[i].sum()), dtype, 7 * case + i) for i in range(P)]
        send = alloc_ranks(P, max(1, int(C.sum(1).max())), dtype, 4)
        for i in range(P):
            if sends[i].size:
                send[i, :sends[i].size].copy_(upload([sends[i]], dtype)[0])
        recv = alloc_ranks(P, max(1, int(C.sum(0).max())), dtype, 4)
        ccgpu.all_to_all(send, recv, C.tolist(), 1, fuse_depth=fd, blocks_per_cu=bpc)
        torch.cuda.synchronize()
        want = cs.all_to_all(sends, C, 1)
        got = download(recv, dtype)
        same([got[j][:want[j].size] for j in range(P)], want, f"a2a case {case}")


@pytest.mark.parametrize("fd", [0, 1])
def test_padded_dispatch_tile_edges(fd):
    """Rows of 2064 bytes (a row ends 16 bytes into a tile's second half)
    and capacities that leave free slots: copies and zero fills."""
    g = np.random.default_rng([55, fd])
    row = 1032                       # bf16 elements: 2064 bytes
    for case in range(6):
        N = int(g.choice([2, 4, 8]))
        E = N * int(g.integers(1, 3))
        Ce = g.integers(0, 7, size=(N, E))
        cap = int(g.integers(1, 6))
        say(f"padded dispatch fd={fd} case={case} N={N} E={E} cap={cap}")
        sends = [values(int(Ce[i].sum()) * row, "bf16", 11 * case + i) for i in range(N)]
        tok = alloc_ranks(N, max(1, int(Ce.sum(1).max()) * row), "bf16", 4)
        for i in range(N):
            if sends[i].size:
                tok[i, :sends[i].size].copy_(upload([sends[i]], "bf16")[0])
        exp = alloc_ranks(N, E * cap * row, "bf16", 4)
        ccgpu.moe_dispatch_padded(tok, exp, Ce.tolist(), cap, row, fuse_depth=fd)
        torch.cuda.synchronize()
        want, _ = aa.padded_dispatch(sends, Ce, cap, row)
        got = download(exp, "bf16")
        same([got[j][:want[j].size] for j in range(N)], want, f"padded case {case}")
