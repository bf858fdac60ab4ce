"""The capacity-padded MoE exchange's one-launch row kernel (k_moe_rows), its
index arithmetic restated in Python and replayed on the CPU: for every
output row (one workgroup each) the source row it copies, or none for a zero
row, must be what the descriptor plan of the same exchange
(cc_all_to_all_plan) copies to that row, and every destination row must be
written exactly once."""
import numpy as np
import pytest

from ring_allreduce_reduction_02_amd import ccgpu


def kernel_rows(dispatch, N, E, cap, rowb, cnt, sb, ss, db, ds):
    """(source address or None, destination address) per workgroup, in the
    kernel's grid order."""
    epr = E // N
    rows_pre = [0]
    for i in range(N):
        rows_pre.append(rows_pre[-1] + int(cnt[i].sum()))
    total = N * E * cap if dispatch else rows_pre[N]
    out = []
    for idx in range(total):
        src = None
        if dispatch:
            # expert side's order: expert rank j, token rank i, local expert l, slot s
            b, s = divmod(idx, cap)
            j, rem = divmod(b, N * epr)
            i, l = divmod(rem, epr)
            e = j * epr + l
            dst = db + j * ds + (rem * cap + s) * rowb
            if s < cnt[i, e]:
                src = sb + i * ss + (int(cnt[i, :e].sum()) + s) * rowb
        else:
            # token rank i's rows, sorted by expert
            i = 0
            while i + 1 < N and rows_pre[i + 1] <= idx:
                i += 1
            r = idx - rows_pre[i]
            e, d = 0, 0
            while e + 1 < E and d + cnt[i, e] <= r:
                d += cnt[i, e]
                e += 1
            s = r - d
            dst = db + i * ds + r * rowb
            if s < cap:
                j, l = divmod(e, epr)
                src = sb + j * ss + ((i * epr + l) * cap + s) * rowb
        out.append((src, dst))
    return out


def plan_rows(kind, N, E, cap, rowb, cnt, sb, ss, db, ds):
    recs = ccgpu.all_to_all_plan(kind, ccgpu.RankBuf(sb, ss), ccgpu.RankBuf(db, ds), cnt.tolist(), N,
                                 elem_per_row=rowb // 2, dtype="bf16", nexperts=E, capacity=cap)
    rows = []
    for (_, src, dst, nb) in recs:
        assert nb % rowb == 0
        for k in range(nb // rowb):
            rows.append((src + k * rowb if src else None, dst + k * rowb))
    return rows


@pytest.mark.parametrize("seed", range(8))
def test_row_kernel_matches_the_descriptor_plan(seed):
    g = np.random.default_rng([20261202, 77, seed])
    TOK, EXP = 1 << 40, 1 << 44
    for _ in range(6):
        N = int(g.choice([1, 2, 3, 4, 8]))
        E = N * int(g.integers(1, 5))
        cap = int(g.integers(1, 9))
        cnt = g.integers(0, 12, size=(N, E))
        cnt[g.random(size=(N, E)) < 0.2] = 0
        rowb = int(g.choice([32, 48, 14336]))
        TS, XS = 1 << 24, 1 << 26
        got = kernel_rows(True, N, E, cap, rowb, cnt, TOK, TS, EXP, XS)
        want = plan_rows("moe_dispatch", N, E, cap, rowb, cnt, TOK, TS, EXP, XS)
        assert sorted(got, key=lambda x: x[1]) == sorted(want, key=lambda x: x[1])
        dsts = [d for _, d in got]
        assert len(set(dsts)) == len(dsts) == N * E * cap
        got = kernel_rows(False, N, E, cap, rowb, cnt, EXP, XS, TOK, TS)
        want = plan_rows("moe_combine", N, E, cap, rowb, cnt, EXP, XS, TOK, TS)
        assert sorted(got, key=lambda x: x[1]) == sorted(want, key=lambda x: x[1])
        dsts = [d for _, d in got]
        assert len(set(dsts)) == len(dsts) == int(cnt.sum())
