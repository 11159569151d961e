"""Masked softmax attention: the exact result of block-sparse attention.

Block-sparse attention (machinebrief LVSA article: block-sparse attention; Sparse
VideoGen2 page, Abstract: compute only the critical tokens; OSP-Next page,
"Method": sparse attention kept compatible with FlashAttention kernels) skips
(query block, key block) tiles whose mask bit is 0. Skipping only drops work whose
contribution is exactly zero, so the result is plain softmax attention over the
kept keys:

    J(i)   = { valid key j : M[block(i), block(j)] = 1 }
    s_ij   = scale * <q_i, k_j>,  scale = 1/sqrt(D) unless given
    o_i    = sum_{j in J(i)} softmax_j(s_ij) v_j
    lse_i  = log sum_{j in J(i)} exp(s_ij)

A query with J(i) empty, or a query slot that is not valid (cube padding), gets
o_i = 0 and lse_i = -inf.

Block ids come from a per-position map, so the same function serves the natural
layout (block = position // bs), the cube layout, and masks stated in another
layout and pulled back to natural coordinates (block = layout_position // bs).
"""
from __future__ import annotations

import math

import numpy as np


def _mask_getter(mask: np.ndarray, B: int, H: int):
    m = np.asarray(mask)
    if m.ndim == 2:
        return lambda b, h: m
    if m.ndim == 3:
        if m.shape[0] != H:
            raise ValueError("per-head mask must have H rows")
        return lambda b, h: m[h]
    if m.ndim == 4:
        return lambda b, h: m[b, h]
    raise ValueError("mask must be [nqb,nkb], [H,nqb,nkb] or [B,H,nqb,nkb]")


def _keys_by_block(kblk: np.ndarray, k_valid: np.ndarray, nkb: int):
    order = np.argsort(kblk, kind="stable")
    order = order[k_valid[order]]
    counts = np.bincount(kblk[order], minlength=nkb)
    return np.split(order, np.cumsum(counts)[:-1])


def masked_attention(q, k, v, mask, qblk, kblk, scale=None, q_valid=None, k_valid=None,
                     rows=None, return_probs=False):
    """General form. q,k,v [B,H,N,D]; mask [nqb,nkb] | [H,nqb,nkb] | [B,H,nqb,nkb];
    qblk[i] / kblk[j] block id of query position i / key position j.

    Returns (o [B,H,R,D], lse [B,H,R]) in float64 for the query rows ``rows``
    (all N when None); with return_probs also P [B,H,R,N].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    qblk = np.asarray(qblk, np.int64)
    kblk = np.asarray(kblk, np.int64)
    q_valid = np.ones(N, bool) if q_valid is None else np.asarray(q_valid, bool)
    k_valid = np.ones(Nk, bool) if k_valid is None else np.asarray(k_valid, bool)
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    get = _mask_getter(mask, B, H)
    nkb = get(0, 0).shape[1]
    keys_of = _keys_by_block(kblk, k_valid, nkb)

    R = rows.size
    o = np.zeros((B, H, R, D))
    lse = np.full((B, H, R), -np.inf)
    probs = np.zeros((B, H, R, Nk)) if return_probs else None
    row_blk = qblk[rows]
    for b in range(B):
        for h in range(H):
            M = get(b, h)
            for qb in np.unique(row_blk):
                sel = np.nonzero((row_blk == qb) & q_valid[rows])[0]
                if sel.size == 0:
                    continue
                kept = np.nonzero(M[qb])[0]
                if kept.size == 0:
                    continue
                keys = np.concatenate([keys_of[kb] for kb in kept])
                if keys.size == 0:
                    continue
                s = scale * (q[b, h, rows[sel]] @ k[b, h, keys].T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                p = e / l
                o[b, h, sel] = p @ v[b, h, keys]
                lse[b, h, sel] = (m + np.log(l))[:, 0]
                if return_probs:
                    probs[b, h, sel[:, None], keys[None, :]] = p
    if return_probs:
        return o, lse, probs
    return o, lse


def block_valid(N: int, bs: int, blk_len=None) -> np.ndarray:
    """Validity of each position of a blocked layout: position i is valid iff its
    offset inside block i // bs is below that block's valid length."""
    pos = np.arange(N)
    if blk_len is None:
        return np.ones(N, bool)
    blk_len = np.asarray(blk_len)
    return (pos % bs) < blk_len[pos // bs]


def block_sparse_attention(q, k, v, mask, bs: int, blk_len=None, scale=None, rows=None,
                           return_probs=False):
    """Blocked layout: position i belongs to block i // bs; blk_len (optional) gives
    the number of valid leading positions of each block (cube layout padding)."""
    N = np.asarray(q).shape[2]
    pos = np.arange(N)
    valid = block_valid(N, bs, blk_len)
    return masked_attention(q, k, v, mask, pos // bs, pos // bs, scale, valid, valid,
                            rows, return_probs)


def dense_attention(q, k, v, scale=None, rows=None):
    """Full attention: every key kept (one block covering everything)."""
    N = np.asarray(q).shape[2]
    Nk = np.asarray(k).shape[2]
    return masked_attention(q, k, v, np.ones((1, 1), np.uint8), np.zeros(N, np.int64),
                            np.zeros(Nk, np.int64), scale, rows=rows)


def kept_flops(mask, bs: int, N: int, D: int, blk_len=None, B: int = 1, H: int = 1) -> float:
    """Algorithmic flops of block-sparse attention: 4*D per valid (query, key) pair
    of every kept block (Q K^T and P V), padding and softmax excluded."""
    nb = -(-N // bs)
    if blk_len is None:
        n = np.full(nb, bs, np.int64)
        n[-1] = N - (nb - 1) * bs
    else:
        n = np.asarray(blk_len, np.int64)
    m = np.asarray(mask, np.int64)
    if m.ndim == 2:
        m = np.broadcast_to(m, (B, H) + m.shape)
    elif m.ndim == 3:
        m = np.broadcast_to(m, (B,) + m.shape)
    pairs = np.einsum("bhqk,q,k->", m, n, n)
    return 4.0 * D * float(pairs)
