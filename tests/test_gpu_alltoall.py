"""MoE dispatch/combine at full size: N=8 ranks, 4096 tokens, top-8 of 64
experts with Zipf(1.2) loads, rows of 7168 bf16.  The oracle computes the
blocked transpose of row identities; every received row's tag and bytes are
checked, and combine (the transposed exchange) must restore the send buffers."""
import sys

import numpy as np
import pytest
import torch

import bench
from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu
N, H = 8, 7168


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    """Counts and tagged bf16 rows of the seeded synth inputs, in the layout
    bench.py times."""
    C, rows = bench.moe_inputs(N, H=H)
    rows_out = C.sum(axis=1)
    rows_in = C.sum(axis=0)
    Ls, Lr = int(rows_out.max()), int(rows_in.max())
    say(f"moe counts: rows sent {rows_out.tolist()}, received {rows_in.tolist()}, "
        f"skew {rows_in.max() / rows_in.mean():.2f}")
    send = bench.strided_ranks(N, Ls * H, torch.bfloat16, DEV)
    bench.upload([r.reshape(-1) for r in rows], send)
    yield C, rows, send, Ls, Lr
    del send
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fd", [0, 1])
def test_moe_dispatch_and_combine(moe, fd):
    C, rows, send, Ls, Lr = moe
    recv = bench.strided_ranks(N, Lr * H, torch.bfloat16, DEV).fill_(float("nan"))
    say(f"dispatch fd={fd}")
    ccgpu.all_to_all(send, recv, C.tolist(), H, fuse_depth=fd)
    torch.cuda.synchronize()
    got = bench.download(recv)
    exp = cs.all_to_all([r.reshape(-1) for r in rows], C, row=H)
    for j in range(N):
        n = len(exp[j])
        assert np.array_equal(got[j, :n], exp[j]), j
        # the tags name the (source, row) the oracle's transpose puts there
        tags = got[j, :n].reshape(-1, H)[:, :3].astype(np.int64)
        src = np.repeat(np.arange(N), C[:, j])
        first = np.cumsum(C, axis=1)[:, j] - C[:, j]          # block (i, j)'s first send row
        row = np.concatenate([np.arange(first[i], first[i] + C[i, j]) for i in range(N)])
        assert np.array_equal(tags[:, 0], src) and np.array_equal(tags[:, 1] | (tags[:, 2] << 16), row), j
    del got
    say(f"combine fd={fd}")
    back = bench.strided_ranks(N, Ls * H, torch.bfloat16, DEV).fill_(float("nan"))
    ccgpu.all_to_all(recv, back, C.T.tolist(), H, fuse_depth=fd)
    torch.cuda.synchronize()
    got = bench.download(back)
    for i in range(N):
        n = rows[i].size
        assert np.array_equal(got[i, :n], rows[i].reshape(-1)), i
