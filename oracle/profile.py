"""Online per-head pattern choice from a sample of query rows.

Sparse Video-Gen page, "Approach" and "Key results": on about 1 % of the query
rows, each candidate sparse pattern's output is compared with dense attention,
and each head takes the pattern with the lower error.

Readings adopted where the page is silent:
* the sampled rows are given by the caller and shared by all heads;
* the error of candidate p is the sum over sampled rows and channels of
  (o_p - o_dense)^2 (its argmin equals the relative-L2 argmin, the denominator
  being shared by all candidates);
* a candidate mask is stated in its own layout (natural, or frame-major for the
  temporal pattern) and is evaluated through that layout's map, so no tensor is
  moved: kept(i, j) = M_p[L(i) // bs, L(j) // bs];
* exact ties go to the lowest candidate index.
"""
from __future__ import annotations

import numpy as np

from .attention import dense_attention, masked_attention
from .layout import frame_major_map


def layout_blocks(grid, bs: int, layout: int) -> np.ndarray:
    """Block id of every natural position under layout 0 (natural) or 1 (frame-major)."""
    T, Hh, W = grid
    N = T * Hh * W
    if layout == 0:
        return np.arange(N) // bs
    if layout == 1:
        return frame_major_map(T, Hh, W) // bs
    raise ValueError(layout)


def profile_heads(q, k, v, grid, bs: int, rows, cand_masks, cand_layout, scale=None):
    """Returns (err [B,H,P] float64, choice [B,H] int32)."""
    rows = np.asarray(rows, np.int64)
    o_dense, _ = dense_attention(q, k, v, scale, rows)
    B, H = o_dense.shape[:2]
    P = len(cand_layout)
    err = np.zeros((B, H, P))
    for p in range(P):
        blk = layout_blocks(grid, bs, int(cand_layout[p]))
        o_p, _ = masked_attention(q, k, v, cand_masks[p], blk, blk, scale, rows=rows)
        err[:, :, p] = ((o_p - o_dense) ** 2).sum(axis=(-1, -2))
    choice = np.argmin(err, axis=-1).astype(np.int32)
    return err, choice
