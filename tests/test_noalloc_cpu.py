"""cc_all_reduce_noalloc's host-side checks (no GPU needed): a caller
workspace and staging beyond the fixed scratch are refused before any device
call."""
import ctypes

import pytest

from ring_allreduce_reduction_02_amd import ccgpu

FAKE = 0x7F0000000000    # never dereferenced: every call below fails validation first


def _noalloc(count, N, dtype, cfg):
    s, r = ccgpu.RankBuf(FAKE, 1 << 30), ccgpu.RankBuf(FAKE + (1 << 40), 1 << 30)
    return ccgpu.raw("cc_all_reduce_noalloc", s, r, count, dtype, 0, N, ctypes.byref(cfg), None)


def test_scratch_size_constant_matches_header():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "cc.h")).read()
    m = re.search(r"#define CC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == ccgpu.NOALLOC_SCRATCH_BYTES


def test_refuses_a_workspace():
    cfg = ccgpu.Config(0, 1, FAKE + (1 << 42), 1 << 20, 0, 0)
    assert _noalloc(100, 8, 2, cfg) == ccgpu.CC_ERR_INVALID_ARG
    assert "no workspace" in ccgpu.load().cc_last_error().decode()


@pytest.mark.parametrize("algo,fd,N,count", [("ring", 1, 8, 4_194_305), ("hd", 1, 8, 524_289), ("tree", 1, 5, 838_861)])
def test_refuses_staging_beyond_the_scratch(algo, fd, N, count):
    need = ccgpu.workspace_size("all_reduce", N, count, "bf16", algo, fd)
    assert need > ccgpu.NOALLOC_SCRATCH_BYTES
    cfg = ccgpu.Config(ccgpu.ALGOS[algo], fd, None, 0, 0, 0)
    assert _noalloc(count, N, 2, cfg) == ccgpu.CC_ERR_INVALID_ARG
    assert "scratch" in ccgpu.load().cc_last_error().decode()


def test_bad_arguments_are_still_refused():
    cfg = ccgpu.Config(0, 0, None, 0, 0, 0)
    assert _noalloc(100, 0, 1, cfg) == ccgpu.CC_ERR_INVALID_ARG      # nranks < 1
    assert _noalloc(100, 8, 9, cfg) == ccgpu.CC_ERR_INVALID_ARG      # dtype
