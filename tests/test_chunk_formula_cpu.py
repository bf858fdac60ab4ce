"""The kernels' closed-form chunk lookups, replayed on the CPU in the same
float arithmetic, against exact integer division.

For element e under the floor bounds floor(c M / N), the chunk is
floor(((e+1) N - 1) / M).  The kernels estimate it in float32: two
u64->f32 conversions, a reciprocal within one ulp, and a product.  One
64-bit remainder check then corrects the estimate.  A chunk's start
floor(c M / N) comes from a double product with the rounded reciprocal of
N, followed by one integer check.

These tests replay both estimates with the reciprocal pushed a full ulp
either way, over random and adversarial (M, N, e).  They show the single
correction lands on the exact quotient wherever the error argument says
it must: quotients below N <= 64, and c M below 2^47."""
import numpy as np

F32 = np.float32


def _u64_to_f32(x):
    return F32(F32(x >> 32) * F32(4294967296.0) + F32(x & 0xFFFFFFFF))


def _chunk_est(M, N, e, ulp_shift):
    num = (e + 1) * N - 1
    fm = _u64_to_f32(M)
    r = F32(F32(1.0) / fm)
    if ulp_shift:
        r = np.nextafter(r, F32(np.inf) if ulp_shift > 0 else F32(0.0), dtype=F32)
    q = int(F32(_u64_to_f32(num) * r))
    rem = num - q * M
    if rem < 0:
        q -= 1
    elif rem >= M:
        q += 1
    return q


def _bound_est(M, N, c, ulp_shift):
    x = c * M
    r = 1.0 / float(N)
    if ulp_shift:
        r = np.nextafter(r, np.inf if ulp_shift > 0 else 0.0)
    q = int(float(x) * r)
    if q * N > x:
        q -= 1
    elif (q + 1) * N <= x:
        q += 1
    return q


def _cases(rng, count):
    for _ in range(count):
        N = int(rng.integers(1, 65))
        M = int(rng.integers(1, 1 << int(rng.integers(1, 42))))
        yield N, M


def test_chunk_of_random():
    rng = np.random.default_rng(2026)
    for N, M in _cases(rng, 3000):
        bounds = [c * M // N for c in range(N + 1)]
        picks = set(int(v) for v in rng.integers(0, M, 6))
        for c in range(N):                       # both sides of every bound
            for e in (bounds[c], bounds[c] - 1, bounds[c + 1] - 1):
                if 0 <= e < M:
                    picks.add(e)
        picks.add(M - 1)
        for e in picks:
            want = ((e + 1) * N - 1) // M
            assert bounds[want] <= e < bounds[want + 1]          # the closed form is the chunk
            for shift in (-1, 0, 1):
                assert _chunk_est(M, N, e, shift) == want, (M, N, e, shift)


def test_chunk_of_near_integer_quotients():
    # numerators one below and at multiples of M: the float product sits on
    # either side of an integer
    rng = np.random.default_rng(7)
    for N, M in _cases(rng, 2000):
        for k in range(1, N):
            # smallest e with (e+1) N - 1 >= k M, and its predecessor
            e = -(-(k * M + 1) // N) - 1
            for ee in (e - 1, e, e + 1):
                if 0 <= ee < M:
                    want = ((ee + 1) * N - 1) // M
                    for shift in (-1, 0, 1):
                        assert _chunk_est(M, N, ee, shift) == want, (M, N, ee, shift)


def test_bound_of():
    rng = np.random.default_rng(11)
    for N, M in _cases(rng, 3000):
        for c in range(N + 1):
            want = c * M // N
            for shift in (-1, 0, 1):
                assert _bound_est(M, N, c, shift) == want, (M, N, c, shift)
    # exact multiples (x / N an integer) and the largest products allowed
    for N in (3, 7, 12, 63, 64):
        for M in (N * 12345, (1 << 41) - 1, (1 << 41) - N, 1 << 40):
            for c in range(N + 1):
                for shift in (-1, 0, 1):
                    assert _bound_est(M, N, c, shift) == c * M // N, (M, N, c, shift)


def _hier_seg_est(M, N, bnd, e, shift):
    """The hierarchical kernel's segment lookup: the flat floor chunk of e
    (the estimate above), then the steps that settle it on the segment
    bounds; returns the segment and the number of steps taken."""
    s = _chunk_est(M, N, e, shift)
    steps = 0
    while s > 0 and e < bnd[s]:
        s -= 1
        steps += 1
    while s + 1 < N and e >= bnd[s + 1]:
        s += 1
        steps += 1
    return s, steps


def _hier_segments_exact(M, dims):
    """The nested segments cut exactly: level-0 chunks, each cut into its
    level-1 chunks, ... as (lo, hi, code)."""
    cur = [(0, M, 0)]
    for i, p in enumerate(dims):
        nxt = []
        for lo, hi, code in cur:
            span = hi - lo
            for c in range(p):
                nxt.append((lo + c * span // p, lo + (c + 1) * span // p, code | (c << (8 * i))))
        cur = nxt
    return cur


def test_hier_segment_lookup():
    """The lookup lands on the segment for any estimate; the nested floor
    bounds stay within a few elements of the flat ones, so where segments
    hold more than a few elements the flat chunk of an element is its
    segment or one beside it and the lookup takes at most one step."""
    rng = np.random.default_rng(5)
    grids = [(2, 2, 2), (4, 2), (2, 4), (8, 8), (4, 4, 4), (3, 5), (2, 3, 4, 2), (7, 9), (16, 4)]
    for dims in grids:
        N = int(np.prod(dims))
        for _ in range(40):
            M = int(rng.integers(1, 1 << int(rng.integers(1, 40))))
            segs = _hier_segments_exact(M, dims)
            bnd = [lo for lo, _, _ in segs] + [M]
            for k, (lo, hi, _) in enumerate(segs):
                if hi == lo:
                    continue
                for e in {lo, hi - 1, (lo + hi) // 2, max(lo, hi - 3), min(hi - 1, lo + 2)}:
                    for shift in (-1, 0, 1):
                        s, steps = _hier_seg_est(M, N, bnd, e, shift)
                        assert s == k, (M, dims, e, shift, s, k)
                        # with segments of more than a few elements the estimate is off by one at most
                        assert steps <= 1 or M < 8 * N, (M, dims, e, shift, steps)
