"""The three end-to-end flows, computed in natural token coordinates.

Softmax attention is equivariant under a permutation P of the tokens:
softmax((PQ)(PK)^T) PV = P softmax(QK^T) V. So "permute, attend under a mask
stated in the new layout, permute back" equals attending in natural order under
the mask pulled back through the layout map. The oracle uses the pulled-back
form; the GPU path moves the tensors. Agreement pins both.

* svg_pipeline: Sparse Video-Gen page, "Approach": spatial heads use a
  same-frame window in natural order; temporal heads use a same-position band in
  frame-major order; each head's pattern comes from the row profiler.
* cube_pipeline: USV page, Figure 2 caption (3D cubes, top-k cube selection) and
  Sparse VideoGen2 page, Abstract (top-p budget).
* long_pipeline: machinebrief LVSA article (block-sparse attention at a long
  horizon) read as a local window plus top-k long-range blocks under one softmax
  (USV page, Figure 2 caption: local and long-range outputs are fused).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import masked_attention
from .layout import cube_map, frame_major_map
from .masks import pattern_mask
from .select import select


def svg_pipeline(q, k, v, grid, bs, choice, w_spatial, w_temporal, scale=None, rows=None):
    """choice[b, h]: 0 spatial, 1 temporal. Returns (o, lse) in natural order."""
    q = np.asarray(q)
    B, H, N, D = q.shape
    T, Hh, W = grid
    m_s = pattern_mask(grid, bs, "spatial", w_spatial)
    m_t = pattern_mask(grid, bs, "temporal", w_temporal)
    blk_nat = np.arange(N) // bs
    blk_fm = frame_major_map(T, Hh, W) // bs
    R = N if rows is None else len(rows)
    o = np.zeros((B, H, R, D))
    lse = np.zeros((B, H, R))
    for b in range(B):
        for h in range(H):
            if choice[b][h] == 0:
                m, blk = m_s, blk_nat
            else:
                m, blk = m_t, blk_fm
            ob, lb = masked_attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                      m, blk, blk, scale, rows=rows)
            o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]
    return o, lse


def cube_scores(q, k, grid, c=4, scale=None):
    """Pooled cube scores in natural coordinates: mean of each cube's tokens."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, H, N, D = q.shape
    slot, counts, n_slots = cube_map(*grid, c)
    cube = slot // c ** 3
    nc = counts.size
    order = np.argsort(cube, kind="stable")          # tokens grouped by cube
    starts = np.cumsum(counts) - counts               # every cube holds >= 1 token
    qp = np.add.reduceat(q[:, :, order], starts, axis=2) / counts[None, None, :, None]
    kp = np.add.reduceat(k[:, :, order], starts, axis=2) / counts[None, None, :, None]
    assert qp.shape == (B, H, nc, D)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return scale * np.einsum("bhqd,bhkd->bhqk", qp, kp)


def cube_pipeline(q, k, v, grid, k_max, top_p, scale=None, rows=None):
    """Returns (o, lse, kv_idx, kv_cnt) with o in natural order."""
    S = cube_scores(q, k, grid, 4, scale)
    idx, cnt = select(S, None, k_max, top_p)
    nc = S.shape[-1]
    mask = np.zeros(S.shape, np.uint8)
    B, H = S.shape[:2]
    for b in range(B):
        for h in range(H):
            for qb in range(nc):
                mask[b, h, qb, idx[b, h, qb, :cnt[b, h, qb]]] = 1
    slot, _, _ = cube_map(*grid, 4)
    cube = slot // 64
    o, lse = masked_attention(q, k, v, mask, cube, cube, scale, rows=rows)
    return o, lse, idx, cnt


def long_pipeline(q, k, v, grid, bs, w_local, k_total, scale=None, rows=None, scores=None):
    """Local window (forced) plus top-(k_total - |local|) blocks by pooled score."""
    from .scores import block_scores
    q = np.asarray(q)
    N = q.shape[2]
    forced = pattern_mask(grid, bs, "spatial", w_local)
    S = block_scores(q, k, bs, None, scale)[0] if scores is None else scores
    idx, cnt = select(S, forced, k_total, 1.0)
    nb = S.shape[-1]
    B, H = S.shape[:2]
    mask = np.zeros(S.shape, np.uint8)
    for b in range(B):
        for h in range(H):
            for qb in range(nb):
                mask[b, h, qb, idx[b, h, qb, :cnt[b, h, qb]]] = 1
    blk = np.arange(N) // bs
    o, lse = masked_attention(q, k, v, mask, blk, blk, scale, rows=rows)
    return o, lse, idx, cnt
