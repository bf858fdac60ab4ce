"""The INT8 kernels' shortcut for round-half-even(u / s), replayed on the CPU
in float32: u times the reciprocal of s (pushed a full ulp either way, as the
hardware reciprocal may be), used only where it lies more than 1e-4 from
every half-integer, must round to the same integer as the correctly rounded
quotient -- on random blocks and on quotients placed a few ulps from ties."""
import numpy as np

F32 = np.float32


def _shortcut(u, s, shift):
    """None where the kernel takes the IEEE division, else its integer."""
    r = F32(F32(1.0) / s)
    if shift:
        r = np.nextafter(r, F32(np.inf) if shift > 0 else F32(0.0), dtype=F32)
    est = F32(u * r)
    frac = abs(F32(est - F32(np.trunc(est))))
    if not (s >= F32(2.0 ** -100) and abs(F32(frac - F32(0.5))) > F32(1e-4)):
        return None
    return float(np.rint(est))


def _check(u, s):
    want = float(np.rint(F32(u / s)))
    taken = 0
    for shift in (-1, 0, 1):
        got = _shortcut(u, s, shift)
        if got is not None:
            taken += 1
            assert got == want, (float(u), float(s), shift)
    return taken


def test_random_blocks():
    rng = np.random.default_rng(8)
    for scale in (1e-30, 1e-6, 1e-3, 1.0, 1e6, 1e30):
        taken = total = 0
        for _ in range(300):
            u = (rng.standard_t(3, size=128) * scale).astype(F32)
            s = F32(F32(np.max(np.abs(u))) / F32(127.0))
            for x in u:
                taken += _check(x, s)
                total += 3
        # the division is the rare path, except for scales below 2^-100
        assert taken > 0.99 * total if scale > 1e-20 else taken == 0, (scale, taken, total)


def test_near_ties():
    rng = np.random.default_rng(9)
    for _ in range(4000):
        s = F32(rng.uniform(1e-6, 1e3))
        n = int(rng.integers(-127, 127))
        base = F32(F32(n + 0.5) * s)
        x = base
        for _ in range(int(rng.integers(0, 40))):
            x = np.nextafter(x, F32(np.inf) if rng.integers(2) else F32(-np.inf), dtype=F32)
        _check(x, s)
