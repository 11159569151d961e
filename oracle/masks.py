"""Block masks from token patterns, and the block-list form of a mask.

Sparse Video-Gen page, "Approach": spatial heads attend block-wise within a frame,
temporal heads attend slash-wise to the same position across frames. Its
"Limitations" note that the sparsity ratios are hand-set; here they are window
widths passed in by the caller.

Readings adopted where the page is silent:
* a spatial pattern keeps token pairs with |t_q - t_k| <= w in natural order
  (w = 0 is "same frame");
* a temporal pattern keeps pairs with |s_q - s_k| <= w, s = y*W + x, and is
  stated in frame-major order, where same-position tokens are contiguous;
* a (query block, key block) pair is kept iff some token pair in it is kept
  (the any-rule); inside a kept block every valid pair attends.
"""
from __future__ import annotations

import numpy as np

from .layout import grid_coords, frame_major_map


def _coord_at_position(grid, kind: str) -> np.ndarray:
    """The pattern coordinate of the token found at each position of the pattern's layout."""
    T, Hh, W = grid
    t, y, x = grid_coords(T, Hh, W)
    if kind == "spatial":
        return t                                   # natural layout, coordinate = frame
    if kind == "temporal":
        pi = frame_major_map(T, Hh, W)
        s = y * W + x
        c = np.empty_like(s)
        c[pi] = s                                  # frame-major position pi[n] holds token n
        return c
    raise ValueError(kind)


def pattern_mask_bruteforce(grid, bs: int, kind: str, w: int) -> np.ndarray:
    """Any-rule block mask [nb, nb] by testing every token pair (small grids only)."""
    c = _coord_at_position(grid, kind)
    N = c.size
    if N > 8192:
        raise ValueError("brute force is for small grids")
    nb = -(-N // bs)
    keep = np.abs(c[:, None] - c[None, :]) <= w            # [N, N] token pattern
    out = np.zeros((nb, nb), np.uint8)
    for qb in range(nb):
        rows = keep[qb * bs:min((qb + 1) * bs, N)]
        for kb in range(nb):
            out[qb, kb] = rows[:, kb * bs:min((kb + 1) * bs, N)].any()
    return out


def pattern_mask(grid, bs: int, kind: str, w: int) -> np.ndarray:
    """Any-rule block mask [nb, nb] from each block's [min, max] coordinate.

    Exact whenever the coordinates inside a block cover every integer between
    their min and max, which holds for both layouts (each steps by 0 or 1); the
    brute-force version pins this on small and mid-size grids.
    """
    c = _coord_at_position(grid, kind)
    N = c.size
    nb = -(-N // bs)
    starts = np.arange(nb) * bs
    lo = np.minimum.reduceat(c, starts)
    hi = np.maximum.reduceat(c, starts)
    return ((lo[:, None] - w <= hi[None, :]) & (lo[None, :] <= hi[:, None] + w)).astype(np.uint8)


def mask_to_list(mask: np.ndarray, max_kv: int | None = None):
    """Ascending kept key-block indices per query-block row.

    mask [..., nqb, nkb] -> (kv_idx [..., nqb, max_kv] padded with -1, kv_cnt [..., nqb]).
    """
    m = np.asarray(mask) != 0
    nkb = m.shape[-1]
    max_kv = nkb if max_kv is None else max_kv
    cnt = m.sum(-1).astype(np.int32)
    if cnt.size and cnt.max() > max_kv:
        raise ValueError("row has more kept blocks than max_kv")
    idx = np.full(m.shape[:-1] + (max_kv,), -1, np.int32)
    flat_m = m.reshape(-1, nkb)
    flat_i = idx.reshape(-1, max_kv)
    for r in range(flat_m.shape[0]):
        nz = np.nonzero(flat_m[r])[0]
        flat_i[r, :nz.size] = nz
    return idx, cnt


def list_to_mask(kv_idx: np.ndarray, kv_cnt: np.ndarray, nkb: int) -> np.ndarray:
    """Inverse of mask_to_list (entries past kv_cnt are ignored)."""
    lead = kv_cnt.shape
    out = np.zeros(lead + (nkb,), np.uint8)
    fi = kv_idx.reshape(-1, kv_idx.shape[-1])
    fc = kv_cnt.reshape(-1)
    fo = out.reshape(-1, nkb)
    for r in range(fc.size):
        fo[r, fi[r, :fc[r]]] = 1
    return out
