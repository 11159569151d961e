"""Block mean-pooling and pooled query-key block scores.

USV page, Figure 2 caption: long-range sparse attention keeps key cubes picked by
top-k cube selection. The page gives no scoring formula; the reading adopted is
the plainest one: each block is summarised by the mean of its valid rows, and the
score of a (query block, key block) pair is scale * <mean q, mean k> with
scale = 1/sqrt(D), the same scale as the attention logits.
"""
from __future__ import annotations

import math

import numpy as np


def block_means(x, bs: int, blk_len=None) -> np.ndarray:
    """x [B,H,N,D] -> [B,H,nb,D] float64: mean over the valid rows of each block.

    Valid rows are the first blk_len[b] rows of block b (all rows that exist when
    blk_len is None; the last block may be short). A block with no valid row
    pools to zero.
    """
    x = np.asarray(x, np.float64)
    B, H, N, D = x.shape
    nb = -(-N // bs)
    out = np.zeros((B, H, nb, D))
    for blk in range(nb):
        lo = blk * bs
        hi = min(lo + bs, N)
        if blk_len is not None:
            hi = min(hi, lo + int(blk_len[blk]))
        if hi > lo:
            out[:, :, blk] = x[:, :, lo:hi].mean(axis=2)
    return out


def block_scores(q, k, bs: int, blk_len=None, scale=None):
    """S [B,H,nqb,nkb] = scale * mean_q @ mean_k^T, plus the pooled vectors."""
    qp = block_means(q, bs, blk_len)
    kp = block_means(k, bs, blk_len)
    D = qp.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return scale * np.einsum("bhqd,bhkd->bhqk", qp, kp), qp, kp
