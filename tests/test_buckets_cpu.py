"""Bucket plan (cc_bucket_plan) against the oracle's packing rule, and the
bucketed AllReduce's argument validation (no device needed)."""
import ctypes
import math

import numpy as np
import pytest

from oracle import ccsim as cs
from ring_allreduce_reduction_02_amd import ccgpu, synth
from tests.test_abi_cpu import FAKE, no_gpu_only


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cap", [25 * 1024 * 1024, 1 << 20, 1])
def test_bucket_plan_matches_oracle(seed, cap):
    g = np.random.default_rng(seed)
    sizes = [int(math.floor(math.exp(v))) for v in g.uniform(math.log(4096), math.log(16_777_216), 120)]
    for align in (1, 128):
        bof, toff, boff, bcnt = ccgpu.bucket_plan(sizes, 2, cap, align)
        ref = cs.bucket_pack(sizes, 2, cap)
        assert len(boff) == len(ref)
        for b, members in enumerate(ref):
            assert [t for t in range(len(sizes)) if bof[t] == b] == sorted(members)
            # back to back in packing order, starting at the bucket offset
            pos = boff[b]
            for t in members:
                assert toff[t] == pos
                pos += sizes[t]
            assert bcnt[b] == sum(sizes[t] for t in members)
            assert boff[b] % align == 0
            if b:
                assert boff[b] >= boff[b - 1] + bcnt[b - 1]


def test_bucket_plan_workload_sizes():
    sizes = synth.tensor_sizes_log_uniform()
    bof, toff, boff, bcnt = ccgpu.bucket_plan(sizes, 2, 25 * 1024 * 1024, 128)
    assert len(boff) == len(cs.bucket_pack(sizes, 2, 25 * 1024 * 1024))
    assert all(c * 2 <= 25 * 1024 * 1024 or sum(1 for t in range(len(sizes)) if bof[t] == b) == 1
               for b, c in enumerate(bcnt))


def test_bucket_plan_edge_cases():
    assert ccgpu.bucket_plan([], 2, 100, 1) == ([], [], [], [])
    bof, toff, boff, bcnt = ccgpu.bucket_plan([0, 5, 0], 4, 100, 1)
    assert boff == [0] and bcnt == [5]
    with pytest.raises(ccgpu.CCError):
        ccgpu.bucket_plan([1], 0, 100, 1)


@no_gpu_only
def test_bucketed_all_reduce_validation():
    L = ccgpu.load()
    cfg = ccgpu.Config(0, 0, None, 0, 0)
    s, r = ccgpu.RankBuf(FAKE, 4096), ccgpu.RankBuf(FAKE + (1 << 30), 4096)

    def call(offs, cnts, N=4, cfg_=cfg, send=s, recv=r):
        n = len(offs)
        o = (ctypes.c_size_t * max(n, 1))(*offs)
        c = (ctypes.c_size_t * max(n, 1))(*cnts)
        return L.cc_all_reduce_buckets(send, recv, o, c, n, 1, 0, N, ctypes.byref(cfg_), None)

    assert call([], []) == ccgpu.CC_OK
    assert call([0, 10], [20, 5]) == ccgpu.CC_ERR_INVALID_ARG            # overlap
    assert call([0], [2000]) == ccgpu.CC_ERR_INVALID_ARG                 # beyond the 4096 B stride
    # halving-doubling with N = 3 runs each bucket as its own pair-folded AllReduce
    assert call([0], [10], N=3, cfg_=ccgpu.Config(1, 0, None, 0, 0)) == ccgpu.CC_ERR_NO_DEVICE
    assert call([0], [10], N=4, cfg_=ccgpu.Config(7, 0, None, 0, 0)) == ccgpu.CC_ERR_INVALID_ARG   # unknown algo
    assert L.cc_all_reduce_buckets(s, r, None, None, 2, 1, 0, 4, ctypes.byref(cfg), None) == ccgpu.CC_ERR_INVALID_ARG
    assert call([0, 40], [10, 0]) == ccgpu.CC_ERR_NO_DEVICE               # valid: only the device is missing
