"""The alpha-beta fit recovers a known alpha and beta from synthetic timings."""
import numpy as np
import pytest

from ring_allreduce_reduction_02_amd import calib


def test_alpha_beta_recovery():
    alpha, beta = 3.5e-6, 1 / 600e9
    N = 8
    steps = [2 * (N - 1)] * 9
    sizes = [4096 * 4 ** k for k in range(9)]
    sent = [2 * (N - 1) * s // N for s in sizes]
    t = [alpha * n + beta * b for n, b in zip(steps, sent)]
    fit = calib.fit_alpha_beta(steps, sent, t)
    assert fit["alpha_us_per_step"] == pytest.approx(alpha * 1e6, rel=1e-6)
    assert fit["link_GBps"] == pytest.approx(600, rel=1e-6)
    assert fit["n_star_bytes"] == pytest.approx(alpha / beta, rel=1e-6)


def test_fused_fit_recovery():
    b = np.array([2 ** k for k in range(12, 32, 2)], dtype=float)
    t = 4e-6 + b / 6.2e12
    fit = calib.fit_fixed_plus_bandwidth(b, t)
    assert fit["t0_us"] == pytest.approx(4.0, rel=1e-6)
    assert fit["bw_GBps"] == pytest.approx(6200, rel=1e-6)


def test_launch_alpha_beta_recovery_over_several_rank_counts():
    t0, alpha, beta = 6e-6, 1.2e-6, 1 / 450e9
    steps, sent, t = [], [], []
    for N in (4, 8, 16):
        for s in [4096 * 4 ** k for k in range(10)]:
            steps.append(2 * (N - 1))
            sent.append(2 * (N - 1) * s // N)
            t.append(t0 + alpha * steps[-1] + beta * sent[-1])
    fit = calib.fit_launch_alpha_beta(steps, sent, t)
    assert fit["t0_us"] == pytest.approx(6.0, rel=1e-5)
    assert fit["alpha_us_per_step"] == pytest.approx(1.2, rel=1e-5)
    assert fit["link_GBps"] == pytest.approx(450, rel=1e-5)
    assert fit["max_rel_residual"] < 1e-9


def test_ring_tree_crossover_balances_the_two_models():
    a, b = 5e-6, 1 / 50e9
    for N in (8, 64, 100, 1024):
        c = calib.ring_tree_crossover(N, a, b)
        lg = np.log2(N)
        ring = 2 * (N - 1) * a + 2 * (N - 1) / N * c["exact"] * b
        tree = 2 * lg * a + 2 * lg * c["exact"] * b
        assert ring == pytest.approx(tree)
    # the passage's printed example: about 3.8 MB for alpha 5 us, 50 GB/s, N = 100
    assert calib.ring_tree_crossover(100, a, b)["log"] / 1e6 == pytest.approx(3.76, abs=0.01)


def test_bench_refuses_more_than_one_gpu():
    import subprocess, sys, os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_multidim_time_matches_the_oracle_model():
    """The bench's per-level model equals the oracle's BlueConnect model and
    gives Napkin Math 1.6's 8 x 8 GPU budget (about 8.3 ms for 1 GB at 450 and
    50 GB/s)."""
    from oracle import ccsim as cs
    for dims in ((8, 8), (3, 2, 2), (4, 1, 2), (64,)):
        a, b = [1e-6 * (i + 1) for i in range(len(dims))], [1e-11 * (i + 2) for i in range(len(dims))]
        assert calib.multidim_time(1e8, dims, a, b) == pytest.approx(cs.multidim_time_model(1e8, dims, a, b))
    assert sum(calib.multidim_time(1e9, (8, 8), (0, 0), (1 / 450e9, 1 / 50e9))) == pytest.approx(8.26e-3, abs=1e-5)


def test_pairwise_time_matches_the_oracle_model():
    from oracle import ccsim as cs
    g = np.random.default_rng(2)
    for N in (2, 3, 8):
        C = g.integers(0, 1000, size=(N, N))
        mx = [max(int(C[i, (i + k) % N]) for i in range(N)) for k in range(N)]
        assert calib.pairwise_time(mx, 3e-6, 2e-11) == pytest.approx(cs.pairwise_time_model(C, 3e-6, 2e-11))
