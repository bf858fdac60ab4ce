"""Host logic of the INT8 compression entry points, without a GPU: message
size, workspace size, and argument checks (valid calls report that no device
is present)."""
import ctypes
import math

import pytest
import torch

from oracle import compress as cp
from ring_allreduce_reduction_02_amd import ccgpu

E = ccgpu


def test_message_bytes_match_the_oracle():
    for M in (0, 1, 127, 128, 129, 1000, 1 << 20, 67_108_864):
        assert ccgpu.int8_message_bytes(M) == cp.message_bytes(M, 128)
    assert ccgpu.QUANT_BLOCK == 128


def test_workspace_sizes():
    r = lambda v: -(-v // 256) * 256
    for N, M in ((8, 1000), (3, 1 << 20), (16, 5)):
        assert ccgpu.int8_ef_workspace_size(N, M, "f32", 0) == 0
        assert ccgpu.int8_ef_workspace_size(N, M, "bf16", 1) == N * (r(M) + r(4 * math.ceil(M / 128)))
    assert ccgpu.int8_ef_workspace_size(8, 0, "f32", 1) == 0


def _rb(base, stride):
    return E.RankBuf(base, stride)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device status")
def test_argument_checks():
    L = ccgpu.load()
    g, e, r = _rb(1 << 20, 1 << 16), _rb(1 << 30, 1 << 16), _rb(1 << 34, 1 << 16)
    q, s = _rb(1 << 36, 1 << 16), _rb(1 << 38, 1 << 16)
    cfg = E.Config(0, 0, None, 0, 0, 0)
    c = lambda x: ctypes.byref(x)
    M, N = 1000, 4
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(cfg), None) == E.CC_ERR_NO_DEVICE
    assert L.cc_all_reduce_int8_ef(g, e, g, M, 2, N, c(cfg), None) == E.CC_ERR_NO_DEVICE      # in place
    assert L.cc_all_reduce_int8_ef(g, e, r, 0, 1, N, c(cfg), None) == E.CC_OK
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 0, N, c(cfg), None) == E.CC_ERR_UNSUPPORTED    # int32
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(E.Config(1, 0, None, 0, 0, 0)), None) == E.CC_ERR_UNSUPPORTED
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(E.Config(0, 1, None, 0, 0, 1)), None) == E.CC_ERR_UNSUPPORTED
    assert L.cc_all_reduce_int8_ef(g, g, r, M, 1, N, c(cfg), None) == E.CC_ERR_INVALID_ARG    # err overlaps grad
    assert L.cc_all_reduce_int8_ef(g, e, _rb((1 << 20) + 64, 1 << 16), M, 1, N, c(cfg), None) == E.CC_ERR_INVALID_ARG
    assert L.cc_all_reduce_int8_ef(g, _rb(1 << 30, 64), r, M, 1, N, c(cfg), None) == E.CC_ERR_INVALID_ARG  # short err rows
    # two-kernel form: workspace required, and it must not overlap the buffers
    cfg1 = E.Config(0, 1, None, 0, 0, 0)
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(cfg1), None) == E.CC_ERR_INVALID_ARG
    ws = ccgpu.int8_ef_workspace_size(N, M, "f32", 1)
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(E.Config(0, 1, 1 << 40, ws, 0, 0)), None) == E.CC_ERR_NO_DEVICE
    assert L.cc_all_reduce_int8_ef(g, e, r, M, 1, N, c(E.Config(0, 1, 1 << 30, ws, 0, 0)), None) == E.CC_ERR_INVALID_ARG
    # the two halves
    assert L.cc_quantize_ef(g, e, q, s, M, 1, N, c(cfg), None) == E.CC_ERR_NO_DEVICE
    assert L.cc_quantize_ef(g, e, q, q, M, 1, N, c(cfg), None) == E.CC_ERR_INVALID_ARG         # q overlaps scales
    assert L.cc_all_reduce_dequant(q, s, r, M, 2, N, c(cfg), None) == E.CC_ERR_NO_DEVICE
    assert L.cc_all_reduce_dequant(q, s, q, M, 2, N, c(cfg), None) == E.CC_ERR_INVALID_ARG     # recv overlaps q
    assert L.cc_all_reduce_dequant(q, s, r, M, 0, N, c(cfg), None) == E.CC_ERR_UNSUPPORTED
    out = ctypes.c_size_t(0)
    assert L.cc_int8_message_bytes(10, None) == E.CC_ERR_INVALID_ARG
    assert L.cc_int8_message_bytes(10, ctypes.byref(out)) == E.CC_OK and out.value == 14
