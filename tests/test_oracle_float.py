"""Floating point: fold order, error bound against an order-free fp64 sum,
bf16 rounding against a library routine, denormals, NaN/signed-zero MAX."""
import numpy as np
import pytest
import torch

from oracle import ccsim as cs

CASES = [(2, 1), (3, 2), (4, 1), (4, 9), (5, 23), (8, 8), (8, 61), (16, 45), (16, 3)]


def _floats(N, M, dtype, seed=0, scale=1.0):
    g = np.random.default_rng([9, N, M, seed])
    xs = [(g.standard_normal(M) * scale).astype(np.float32) for _ in range(N)]
    if dtype == "bf16":
        xs = [cs.f32_to_bf16_bits(x) for x in xs]
    return xs


@pytest.mark.parametrize("N,M", CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_ring_steps_equal_chain_closed_form(N, M, dtype, op):
    """The step simulator (snapshots, per-step chunk indices) and the fold
    chain written without steps agree bit for bit."""
    xs = _floats(N, M, dtype)
    out = cs.ring_all_reduce(xs, op, dtype)
    vals = np.stack(xs)
    chain = cs.ring_fold_elements(vals, np.arange(M), M, op, dtype)
    for r in range(N):
        assert np.array_equal(out[r].view(np.uint8), chain.view(np.uint8))
    if M % N == 0:
        rs = cs.ring_reduce_scatter(xs, op, dtype)
        chain_rs = cs.ring_fold_elements(vals, np.arange(M), M, op, dtype, standalone_rs=True)
        S = M // N
        for r in range(N):
            assert np.array_equal(rs[r].view(np.uint8), chain_rs[r * S:(r + 1) * S].view(np.uint8))


@pytest.mark.parametrize("N,M", [(2, 5), (4, 9), (8, 61), (16, 45)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hd_and_butterfly_steps_equal_tree_closed_forms(N, M, dtype):
    xs = _floats(N, M, dtype, seed=1)
    vals = np.stack(xs)
    hd = cs.hd_all_reduce(xs, "sum", dtype)
    hd_c = cs.hd_fold_elements(vals, np.arange(M), M, "sum", dtype)
    bf = cs.butterfly_all_reduce(xs, "sum", dtype)
    for r in range(N):
        assert np.array_equal(hd[r].view(np.uint8), hd_c.view(np.uint8))
        assert np.array_equal(bf[r].view(np.uint8), cs.butterfly_fold_elements(vals, r, "sum", dtype).view(np.uint8))


def test_fold_order_is_visible():
    """Ring, halving-doubling and butterfly associate differently, and a sum
    that always starts at rank 0 differs from the ring's: a wrong start rank or
    tree in either side of a parity test shows up in the low bits."""
    N, M = 8, 4096
    xs = _floats(N, M, "f32", seed=2)
    ring = cs.ring_all_reduce(xs, "sum", "f32")[0]
    hd = cs.hd_all_reduce(xs, "sum", "f32")[0]
    bf = cs.butterfly_all_reduce(xs, "sum", "f32")[0]
    naive = xs[0].copy()
    for r in range(1, N):
        naive = naive + xs[r]
    assert not np.array_equal(ring, naive)
    assert not np.array_equal(ring, hd)
    assert not np.array_equal(hd, bf)
    assert not np.array_equal(ring, bf)


@pytest.mark.parametrize("algo", ["ring", "hd", "butterfly"])
def test_error_bound_against_fp64(algo):
    """Norm-wise relative error vs the order-free fp64 sum: <= 1e-5 for fp32,
    <= 1e-2 for bf16 (Gaussian gradients, N = 8)."""
    fn = {"ring": cs.ring_all_reduce, "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce}[algo]
    N, M = 8, 20000
    for dtype, tol, sigma in (("f32", 1e-5, 1e-3), ("bf16", 1e-2, 1e-2)):
        xs = _floats(N, M, dtype, seed=3, scale=sigma)
        ref = cs.plain_reduce(xs, "sum", dtype)
        out = fn(xs, "sum", dtype)
        y = out[0] if dtype == "f32" else cs.bf16_bits_to_f32(out[0])
        err = cs.norm_rel_error(y, ref)
        assert err <= tol, err
        # and the bound has teeth: dropping one rank's contribution violates it
        bad = ref - cs.to_acc(xs[3], dtype).astype(np.float64)
        assert cs.norm_rel_error(bad, ref) > tol


def test_bf16_widening_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = cs.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_rounding_against_torch():
    g = np.random.default_rng(4)
    x = np.concatenate([
        (g.standard_normal(200000) * 10.0 ** g.integers(-40, 38, size=200000)).astype(np.float32),
        g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    # ties: exactly halfway between two bf16 values, both parities of the low kept bit
    base = g.integers(0, 2 ** 16, size=20000, dtype=np.uint32) << 16
    ties = (base | 0x8000).astype(np.uint32).view(np.float32)
    edge = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 3.4028235e38,
                     1e-45, -1e-45, 1.1754942e-38, 5.877472e-39], dtype=np.float32)
    x = np.concatenate([x, ties, edge])
    x = x[~np.isnan(x)]
    ours = cs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_nan_stays_nan_and_quiet():
    x = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0x7FFFFFFF], dtype=np.uint32).view(np.float32)
    b = cs.f32_to_bf16_bits(x)
    f = cs.bf16_bits_to_f32(b)
    assert np.isnan(f).all()
    assert ((b & 0x0040) != 0).all()
    assert list(b >> 15) == [0, 1, 0, 0]


def test_f32_denormals_are_kept():
    tiny = np.array([1e-45, 2e-45, -3e-45, 1e-39], dtype=np.float32)
    xs = [tiny.copy() for _ in range(4)]
    out = cs.ring_all_reduce(xs, "sum", "f32")[0]
    assert (out != 0).all()
    assert np.array_equal(out, (tiny * 4).astype(np.float32))


def test_float_max_semantics():
    a = np.array([np.nan, 0.0, -0.0, -0.0, 1.0, -2.0], dtype=np.float32)
    b = np.array([1.0, -0.0, 0.0, -0.0, np.nan, -3.0], dtype=np.float32)
    r = cs.combine("max", a, b)
    r2 = cs.combine("max", b, a)
    assert np.array_equal(r.view(np.uint32), r2.view(np.uint32))
    assert np.isnan(r[0]) and np.isnan(r[4])
    assert r.view(np.uint32)[1] == 0 and r.view(np.uint32)[2] == 0
    assert r.view(np.uint32)[3] == 0x80000000
    assert r[5] == -2.0
