"""Acceptance rule for a selection made in fp32 against the fp64 oracle.

Exact equality is required except where the oracle itself is within a hair of a
decision boundary: a block that differs is excused if its oracle score lies
within `tol` of the score at the oracle's boundary, and with top-p on, the kept
count may differ by one when the oracle's cumulative mass at the smaller count
is within `tol` of top_p.
"""
import numpy as np

from oracle.select import select_row


def row_matches(s, forced, k_max, top_p, got, tol=1e-4) -> bool:
    s = np.asarray(s, np.float64)
    got = np.sort(np.asarray(got))
    ref = select_row(s, forced, k_max, top_p)
    if np.array_equal(got, ref):
        return True
    f = np.zeros(s.size, bool) if forced is None else (np.asarray(forced) != 0)
    rank = np.argsort(-s, kind="stable")
    F = rank[f[rank]]
    cand = rank[~f[rank]]
    n_f = min(F.size, k_max)
    if not set(F[:n_f].tolist()) <= set(got.tolist()):
        # forced blocks may only differ by near-ties among themselves when capped
        if F.size <= k_max:
            return False
    n_ref = ref.size - n_f
    n_got = got.size - n_f
    if n_got != n_ref:
        if not (top_p < 1.0 and abs(n_got - n_ref) == 1 and min(n_got, n_ref) >= 1):
            return False
        e = np.exp(s - s.max())
        p = e / e.sum()
        c = np.cumsum(p[cand])
        if abs(c[min(n_got, n_ref) - 1] - top_p) > tol:
            return False
    expect = set(F[:n_f].tolist()) | set(cand[:n_got].tolist())
    diff = expect ^ set(got.tolist())
    if not diff:
        return True
    if n_got == 0:
        return False
    b = s[cand[n_got - 1]]
    return all(abs(s[j] - b) <= tol for j in diff)


def check_selection(S, forced, k_max, top_p, kv_idx, kv_cnt, tol=1e-4):
    """S [..., nqb, nkb] (the scores the selection saw), outputs from the GPU.
    Returns (n_rows, n_exact, bad_rows)."""
    S = np.asarray(S, np.float64)
    nqb, nkb = S.shape[-2:]
    flatS = S.reshape(-1, nqb, nkb)
    fi = kv_idx.reshape(-1, nqb, kv_idx.shape[-1])
    fc = kv_cnt.reshape(-1, nqb)
    bad, exact, n = [], 0, 0
    for u in range(flatS.shape[0]):
        for qb in range(nqb):
            got = fi[u, qb, :fc[u, qb]]
            fr = None if forced is None else forced[qb]
            n += 1
            if np.array_equal(np.sort(got), select_row(flatS[u, qb], fr, k_max, top_p)):
                exact += 1
            elif not row_matches(flatS[u, qb], fr, k_max, top_p, got, tol):
                bad.append((u, qb))
    return n, exact, bad
