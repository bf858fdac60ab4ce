"""The rank-stride rule the bench lays its workloads out with: the payload
rounded up to a power of two P, plus max(32 KiB, P/1024), or plus 1 MiB
for P of 4 to 32 MiB."""
import bench


def test_rank_stride_rule():
    assert bench.rank_stride_bytes(256 << 20) == (256 << 20) + (256 << 10)     # 8 x 256 MiB fp32 rows
    assert bench.rank_stride_bytes(128 << 20) == (128 << 20) + (128 << 10)     # 16 x 128 MiB
    assert bench.rank_stride_bytes(32 << 20) == (32 << 20) + (1 << 20)         # 64 x 32 MiB
    assert bench.rank_stride_bytes((4 << 20) - 1) == (4 << 20) + (1 << 20)     # the int32 ring's 4 MiB rows
    assert bench.rank_stride_bytes((2 << 20) + 1) == (4 << 20) + (1 << 20)
    assert bench.rank_stride_bytes(2 << 20) == (2 << 20) + (32 << 10)
    assert bench.rank_stride_bytes((32 << 20) + 1) == (64 << 20) + (64 << 10)
    assert bench.rank_stride_bytes(552_812_320) == (1 << 30) + (1 << 20)       # 276,406,160 bf16 elements
    assert bench.rank_stride_bytes(8 << 20) == (8 << 20) + (1 << 20)
    assert bench.rank_stride_bytes(1000) == 1024 + (32 << 10)
    for row in (1, 4095, 1 << 20, (1 << 31) + 1):
        s = bench.rank_stride_bytes(row)
        assert s >= row + (32 << 10) and s % 16 == 0


def test_strided_ranks_cpu():
    import torch
    x = bench.strided_ranks(3, 1000, torch.float32, "cpu")
    assert tuple(x.shape) == (3, 1000)
    assert x.stride(0) * 4 == bench.rank_stride_bytes(4000)
