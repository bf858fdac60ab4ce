"""GPU parity of the AllToAll variants against the oracle, byte for byte:
the capacity-padded MoE dispatch and its combine (direct and pairwise; drops,
zero padding, capacity 0, unaligned rows) on random counts and on the MoE
workload's routing (8 ranks, 4096 tokens, top-8 of 64 experts, Zipf loads)
at capacity factors 1, 1.25 and 4, and the hierarchical AllToAll (equal to
the flat exchange) for several node shapes, with graph replays."""
import sys

import numpy as np
import pytest
import torch

from oracle import alltoall as aa
from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu, synth
from tests.gpu_util import DEV, NP_DT, np_to_torch, torch_to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _rows(n_rows, row, dtype, seed):
    g = np.random.default_rng(seed)
    if dtype == "bf16":
        return g.integers(1, 65535, size=n_rows * row, dtype=np.uint16)
    return g.integers(-1000, 1000, size=n_rows * row).astype(NP_DT[dtype])


def _upload(parts, width, dtype, pad=24):
    """[N, width] rank buffers (row stride width + pad) holding parts[i] at the
    start of row i, the rest poisoned."""
    N = len(parts)
    buf = torch.empty(N, width + pad, dtype={"bf16": torch.bfloat16, "int32": torch.int32,
                                             "f32": torch.float32}[dtype], device=DEV)
    buf.view(torch.uint8).fill_(0xA5)
    t = buf[:, :width]
    for i, p in enumerate(parts):
        if p.size:
            t[i, :p.size].copy_(np_to_torch(p, dtype).to(DEV))
    return t


def _moe_counts(N=8, tokens=4096, E=64, k=8):
    ch = synth.moe_routing(N, tokens, E, k)
    return np.stack([aa.dispatch_counts_by_expert(c, E) for c in ch])


def _check_padded(Ce, cap, row, dtype, fd, label):
    N, E = Ce.shape
    sends = [_rows(int(Ce[i].sum()), row, dtype, 100 + i) for i in range(N)]
    tok_w = max(1, int(Ce.sum(axis=1).max()) * row)
    exp_w = max(1, E * cap * row)
    tok = _upload(sends, tok_w, dtype)
    exp = _upload([np.zeros(0, NP_DT[dtype])] * N, exp_w, dtype)
    say(f"padded dispatch {label} fd={fd}")
    ccgpu.moe_dispatch_padded(tok, exp, Ce.tolist(), cap, row, fuse_depth=fd)
    torch.cuda.synchronize()
    want, _ = aa.padded_dispatch(sends, Ce, cap, row)
    got = torch_to_np(exp, dtype)
    for j in range(N):
        n = E * cap * row
        assert np.array_equal(got[j, :n].view(np.uint8), want[j].view(np.uint8)), (label, "dispatch", j)
    back = _upload([np.zeros(0, NP_DT[dtype])] * N, tok_w, dtype)
    say(f"padded combine {label} fd={fd}")
    ccgpu.moe_combine_padded(exp, back, Ce.tolist(), cap, row, fuse_depth=fd)
    torch.cuda.synchronize()
    want_b = aa.padded_combine(want, Ce, cap, row)
    got_b = torch_to_np(back, dtype)
    for i in range(N):
        n = want_b[i].size
        assert np.array_equal(got_b[i, :n].view(np.uint8), want_b[i].view(np.uint8)), (label, "combine", i)


@pytest.mark.parametrize("fd", [0, 1])
@pytest.mark.parametrize("dtype,row", [("bf16", 64), ("bf16", 3), ("int32", 5), ("f32", 8)])
def test_padded_random_counts(fd, dtype, row):
    for (N, E, cap, seed) in [(2, 2, 3, 1), (4, 8, 2, 2), (4, 8, 6, 3), (8, 16, 0, 4), (8, 64, 5, 5), (3, 9, 4, 6)]:
        Ce = np.random.default_rng(seed).integers(0, 7, size=(N, E))
        _check_padded(Ce, cap, row, dtype, fd, f"N={N} E={E} cap={cap} {dtype} row={row}")


@pytest.mark.parametrize("fd", [0, 1])
@pytest.mark.parametrize("factor", [(1, 1), (5, 4), (4, 1)])
def test_padded_moe_routing(fd, factor):
    """The MoE workload's routing (per source, rows per expert) with the
    capacity from the formula at C = 1, 1.25, 4; rows narrowed to 64 bf16 so
    the oracle checks every byte."""
    Ce = _moe_counts()
    cap = ccgpu.moe_capacity(1, 4096, 8, 64, *factor)
    assert cap == aa.source_capacity(4096, 8, 64, f"{factor[0] / factor[1]}")
    v = aa.padded_volume(Ce, cap)
    say(f"moe routing C={factor}: capacity {cap}, dropped {v['dropped_rows']} of {v['dropless_rows']} rows")
    _check_padded(Ce, cap, 64, "bf16", fd, f"moe C={factor}")


HIER = [(8, 2), (8, 4), (6, 3), (4, 1), (4, 4), (16, 4), (12, 2)]


@pytest.mark.parametrize("dtype,row", [("bf16", 64), ("bf16", 3), ("int32", 5), ("f32", 4)])
def test_hierarchical_all_to_all(dtype, row):
    for (P, L) in HIER:
        g = np.random.default_rng([P, L, row])
        for trial in range(2):
            C = g.integers(0, 6, size=(P, P))
            if trial:
                C[g.random((P, P)) < 0.5] = 0
            sends = [_rows(int(C[i].sum()), row, dtype, 10 * i + trial) for i in range(P)]
            send = _upload(sends, max(1, int(C.sum(axis=1).max()) * row), dtype)
            recv = _upload([np.zeros(0, NP_DT[dtype])] * P, max(1, int(C.sum(axis=0).max()) * row), dtype)
            ws = ccgpu.make_all_to_all_hierarchical_workspace(C.tolist(), row, dtype, L, DEV)
            say(f"hierarchical all_to_all P={P} L={L} {dtype} row={row} trial={trial}")
            ccgpu.all_to_all_hierarchical(send, recv, C.tolist(), L, row, workspace=ws)
            torch.cuda.synchronize()
            want = cs.all_to_all(sends, C, row)
            got = torch_to_np(recv, dtype)
            for j in range(P):
                n = want[j].size
                assert np.array_equal(got[j, :n].view(np.uint8), want[j].view(np.uint8)), (P, L, trial, j)


@pytest.mark.parametrize("L", [2, 4])
def test_hierarchical_moe_routing_and_graph(L):
    """The MoE workload's rank-to-rank counts, 64-element bf16 rows; the
    three phases captured in a HIP graph replay to the same bytes."""
    C = synth.moe_counts(8)
    row = 64
    sends = [_rows(int(C[i].sum()), row, "bf16", 50 + i) for i in range(8)]
    send = _upload(sends, int(C.sum(axis=1).max()) * row, "bf16")
    recv = _upload([np.zeros(0, np.uint16)] * 8, int(C.sum(axis=0).max()) * row, "bf16")
    ws = ccgpu.make_all_to_all_hierarchical_workspace(C.tolist(), row, "bf16", L, DEV)
    recv.zero_()                      # the replays below start from zeros too
    say(f"hierarchical moe L={L}")
    ccgpu.all_to_all_hierarchical(send, recv, C.tolist(), L, row, workspace=ws)
    torch.cuda.synchronize()
    want = cs.all_to_all(sends, C, row)
    ref = recv.clone()
    got = torch_to_np(recv, "bf16")
    for j in range(8):
        assert np.array_equal(got[j, :want[j].size], want[j]), j
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ccgpu.all_to_all_hierarchical(send, recv, C.tolist(), L, row, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ccgpu.all_to_all_hierarchical(send, recv, C.tolist(), L, row, workspace=ws)
    for k in range(3):
        recv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"hierarchical graph replay {k}")
        assert torch.equal(recv.view(torch.int16), ref.view(torch.int16)), k
