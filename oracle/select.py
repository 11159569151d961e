"""Per-query-block key-block selection: forced set, top-k cap, top-p budget.

* USV page, Figure 2 caption: a budget is split between local cube attention and
  long-range attention over key cubes picked by top-k selection.
* Sparse VideoGen2 page, Abstract: top-p dynamic budget control.
* machinebrief LVSA article: a fixed block-sparse budget at long horizons.

Rule applied to one row of scores S[0..nkb) with forced set F and cap k_max:

1. Forced blocks outrank every other block; among themselves, and among the
   rest, blocks are ranked by score, higher first, equal scores by lower index.
2. If |F| >= k_max, keep the k_max best-ranked forced blocks and stop.
3. Otherwise rank the non-forced candidates. With top_p < 1, compute
   p_j = softmax(S)_j over all nkb scores, accumulate p over the ranked
   candidates, and keep the shortest prefix (length >= 1) whose sum reaches
   top_p; with top_p >= 1 keep every candidate. Cap the prefix at k_max - |F|.
4. Output the kept indices in ascending order.
"""
from __future__ import annotations

import numpy as np


def select_row(scores, forced=None, k_max: int = 1, top_p: float = 1.0) -> np.ndarray:
    s = np.asarray(scores, np.float64)
    nkb = s.size
    f = np.zeros(nkb, bool) if forced is None else (np.asarray(forced) != 0)
    # stable sort of -s: higher score first, equal scores keep ascending index
    rank = np.argsort(-s, kind="stable")
    forced_ranked = rank[f[rank]]
    if forced_ranked.size >= k_max:
        return np.sort(forced_ranked[:k_max])
    cand = rank[~f[rank]]
    room = k_max - forced_ranked.size
    if top_p < 1.0 and cand.size:
        e = np.exp(s - s.max())
        p = e / e.sum()
        c = np.cumsum(p[cand])
        reach = np.nonzero(c >= top_p)[0]
        r = int(reach[0]) + 1 if reach.size else cand.size
        r = max(r, 1)
    else:
        r = cand.size
    keep = np.concatenate([forced_ranked, cand[:min(r, room)]])
    return np.sort(keep)


def select(scores, forced=None, k_max: int = 1, top_p: float = 1.0):
    """scores [..., nqb, nkb]; forced [nqb, nkb] shared by every (b, h) or None.

    Returns (kv_idx [..., nqb, k_max] padded with -1, kv_cnt [..., nqb]).
    """
    s = np.asarray(scores)
    nqb, nkb = s.shape[-2:]
    flat = s.reshape(-1, nqb, nkb)
    idx = np.full(flat.shape[:2] + (k_max,), -1, np.int32)
    cnt = np.zeros(flat.shape[:2], np.int32)
    for u in range(flat.shape[0]):
        for qb in range(nqb):
            kept = select_row(flat[u, qb], None if forced is None else forced[qb], k_max, top_p)
            idx[u, qb, :kept.size] = kept
            cnt[u, qb] = kept.size
    return idx.reshape(s.shape[:-1] + (k_max,)), cnt.reshape(s.shape[:-1])

