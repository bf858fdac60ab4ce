"""Pins for oracle/compress.py: the textbook's INT8 formula on a hand example,
the block-wise message size and 3.88x ratio, the s_b / 2 error bound and the
block-vs-tensor error, Tables 3 and 4 of the error-feedback section
(tests/golden/error_feedback_table4.json), the telescoping identity, and the
compressed AllReduce: equal to the ring AllReduce of the dequantized
contributions, exact for values the 8-bit grid holds, and within the
quantization bound of the true sum."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ccsim as cs
from oracle import compress as cp

GOLD = os.path.join(os.path.dirname(__file__), "golden", "error_feedback_table4.json")


def test_int8_formula_hand_example():
    """[MLSys-6] 量化: s = max|g| / 127, g_int8 = round(g / s), g_hat = g_int8 s."""
    g = np.array([0.5, -1.27, 0.254, 0.0], dtype=np.float32)
    s = cp.block_scales(g, 4)
    assert s[0] == np.float32(np.float32(1.27) / np.float32(127))
    q = cp.quantize(g, s, 4)
    assert q.tolist() == [50, -127, 25, 0]
    v = cp.dequantize(q, s, 4)
    assert np.allclose(v, [0.5, -1.27, 0.25, 0.0], atol=1e-6)
    # an all-zero block sends zeros with scale 0
    z = np.zeros(5, np.float32)
    assert cp.block_scales(z, 4).tolist() == [0.0, 0.0]
    assert cp.quantize(z, cp.block_scales(z, 4), 4).tolist() == [0] * 5


def test_round_half_even_and_clamp():
    u = np.array([127.0, 2.5, -2.5, 3.5, -127.0, 0.49], dtype=np.float32)
    s = cp.block_scales(u, 8)
    assert s[0] == np.float32(1.0)
    assert cp.quantize(u, s, 8).tolist() == [127, 2, -2, 4, -127, 0]


def test_message_size_and_ratio():
    """[MLSys-6] 分块量化: d + 4d/b bytes, 4b/(b+4) = 3.88 at b = 128."""
    gd = json.load(open(GOLD))
    assert round(cp.compression_ratio(128), 2) == gd["block_bytes_ratio_at_128"]
    assert cp.compression_ratio(64) == pytest.approx(4 * 64 / 68)
    assert cp.message_bytes(1024, 128) == 1024 + 32
    assert cp.message_bytes(1000, 128) == 1000 + 4 * 8          # last block short
    assert 4 * 1024 / cp.message_bytes(1024, 128) == pytest.approx(cp.compression_ratio(128))


@pytest.mark.parametrize("block", [32, 128])
def test_block_error_bound(block):
    """|u - v| <= s_b / 2 up to float32 rounding of s and of q * s."""
    g = np.random.default_rng(block).standard_t(2, size=10_000).astype(np.float32)
    e = np.zeros_like(g)
    q, s, v, en = cp.ef_compress(g, e, block)
    sb = np.repeat(s, block)[:g.size].astype(np.float64)
    err = np.abs(g.astype(np.float64) - v.astype(np.float64))
    assert np.all(err <= 0.5 * sb * (1 + 2 ** -20) + np.abs(g) * 2 ** -23)
    assert np.array_equal(en, (g - v).astype(np.float32))


def test_block_scales_beat_one_tensor_scale_on_heavy_tails():
    """[MLSys-6] 分块量化: one scale per block adapts to the local range; with
    heavy-tailed values the tensor-wide scale's error is several times
    larger."""
    g = np.random.default_rng(7).standard_t(2, size=128 * 512).astype(np.float32)
    e = np.zeros_like(g)
    _, _, vb, _ = cp.ef_compress(g, e, 128)
    _, _, vt, _ = cp.ef_compress(g, e, g.size)
    eb = np.mean(np.abs(g - vb))
    et = np.mean(np.abs(g - vt))
    assert et / eb > 2.0


def test_tables_3_and_4():
    """[MLSys-6] 错误反馈与残差累积, Tables 3 and 4, Example 1.2: the naive
    greedy compressor sends nothing of a true total of 1.6; with error
    feedback it sends 2 and keeps a residual of -0.4."""
    gd = json.load(open(GOLD))
    rows = cp.ef_trace(gd["g"], cp.threshold_compressor, feedback=True)
    for got, want in zip(rows, gd["table4_rows"]):
        assert got == pytest.approx((want["g"], want["e"], want["g_plus_e"], want["v"], want["e_next"],
                                     want["cum_v"]), abs=1e-12)
    naive = cp.ef_trace(gd["g"], cp.threshold_compressor, feedback=False)
    assert naive[-1][5] == gd["naive_transmitted"]
    assert np.cumsum(gd["g"]).tolist() == pytest.approx(gd["table3_cumulative_true"])
    assert rows[-1][5] == gd["ef_transmitted"] and rows[-1][4] == pytest.approx(gd["ef_final_residual"])


def test_telescoping_sum_exact():
    """sum v_t = sum g_t + e_1 - e_(K+1), exactly, in rationals."""
    g = [Fraction(int(x), 97) for x in np.random.default_rng(3).integers(-60, 60, size=40)]
    comp = lambda x: Fraction(round(x * 4), 4)          # a 2-bit-like grid, any compressor works
    rows = cp.ef_trace(g, comp)
    assert sum(r[3] for r in rows) == sum(g) + 0 - rows[-1][4]


def test_ef_keeps_the_long_run_average():
    """The transmitted average approaches the true one when e stays bounded."""
    g = np.full(2000, 0.013, np.float32)
    e = np.zeros(1, np.float32)
    sent = 0.0
    for t in range(2000):
        _, _, v, e = cp.ef_compress(g[t:t + 1], e, 1)
        # one element per block: v == u exactly, so the residual is 0: no loss
        sent += float(v[0])
    assert sent == pytest.approx(float(g.sum()), rel=1e-5)
    # a block with a large neighbour quantizes the small value to 0 and the
    # feedback carries it until it crosses a quantization step
    big = np.float32(1.27)
    e = np.zeros(2, np.float32)
    sent_small = 0.0
    for t in range(100):
        _, _, v, e = cp.ef_compress(np.array([big, 0.003], np.float32), e, 2)
        sent_small += float(v[1])
    assert sent_small == pytest.approx(0.3, abs=0.011)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [2, 3, 8])
def test_compressed_all_reduce_structure(dtype, N):
    """The compressed AllReduce is the ring AllReduce of the dequantized
    contributions; every rank gets the same result, and the new error
    accumulators are u - v."""
    M = 1000
    g = np.random.default_rng([N, M]).standard_normal((N, M)).astype(np.float32) * 1e-2
    xs = [cs.f32_to_bf16_bits(x) for x in g] if dtype == "bf16" else list(g)
    es = [np.random.default_rng([N, r]).standard_normal(M).astype(np.float32) * 1e-4 for r in range(N)]
    out, en = cp.compressed_all_reduce(xs, es, 128, dtype)
    vs = []
    for r in range(N):
        q, s, v, e_next = cp.ef_compress(xs[r], es[r], 128, dtype)
        assert np.array_equal(en[r], e_next)
        vs.append(v)
    ring = cs.ring_all_reduce(vs, "sum", "f32")
    for r in range(N):
        want = cs.f32_to_bf16_bits(ring[r]) if dtype == "bf16" else ring[r]
        assert np.array_equal(np.asarray(out[r]).view(np.uint8), np.asarray(want).view(np.uint8))
    # the message path gives the same bits
    msgs = [cp.ef_compress(xs[r], es[r], 128, dtype)[:2] for r in range(N)]
    again = cp.all_reduce_of_messages([m[0] for m in msgs], [m[1] for m in msgs], 128, dtype)
    for r in range(N):
        assert np.array_equal(np.asarray(again[r]).view(np.uint8), np.asarray(out[r]).view(np.uint8))


def test_compressed_all_reduce_is_exact_on_the_grid_and_bounded_off_it():
    """Values that are integers in [-127, 127] times a power of two with the
    block maximum 127 s quantize exactly, so the result is the plain sum
    (brute force against Python integers); random values stay within the sum
    of the ranks' s_b / 2 bounds of the true sum."""
    N, M = 4, 512
    g = np.random.default_rng(1).integers(-127, 128, size=(N, M))
    g[:, ::128] = 127                                      # every block's maximum is 127
    xs = [(x * 2.0 ** -7).astype(np.float32) for x in g]
    zeros = [np.zeros(M, np.float32)] * N
    out, en = cp.compressed_all_reduce(xs, zeros, 128)
    want = g.sum(axis=0) * 2.0 ** -7
    assert np.array_equal(out[0], want.astype(np.float32))
    assert all(not e.any() for e in en)
    r = np.random.default_rng(2).standard_normal((N, M)).astype(np.float32)
    out, _ = cp.compressed_all_reduce(list(r), zeros, 128)
    bound = sum(np.repeat(cp.block_scales(r[k], 128), 128) / 2 for k in range(N)) * (1 + 1e-5) + 1e-6
    assert np.all(np.abs(out[0].astype(np.float64) - r.astype(np.float64).sum(0)) <= bound)
