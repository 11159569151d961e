"""Gradients of block-sparse attention (test infrastructure only).

The forward (``oracle.attention``) is plain softmax attention over the kept keys
J(i) of each query. Training it end to end (USV page, Abstract and Figure 2
caption: an end-to-end trainable sparsification of the attention; OSP-Next page,
"Method": sparse fine-tuning) needs the gradients of o with respect to q, k and v
for an upstream gradient do. The chain rule through

    s_ij = scale <q_i, k_j>,  p_ij = softmax_j(s_ij) over J(i),  o_i = sum_j p_ij v_j

gives, with every sum over kept (i, j) pairs only,

    dv_j  = sum_i p_ij do_i
    dp_ij = <do_i, v_j>
    ds_ij = p_ij (dp_ij - delta_i),  delta_i = sum_j p_ij dp_ij  (= <do_i, o_i>)
    dq_i  = scale sum_j ds_ij k_j
    dk_j  = scale sum_i ds_ij q_i

A query with no kept key, or a position that is not valid (cube padding), takes
no part: its own gradients are zero and it adds nothing to anyone else's.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _keys_by_block, _mask_getter, block_valid


def masked_attention_bwd(q, k, v, do, mask, qblk, kblk, scale=None, q_valid=None, k_valid=None):
    """General form (same conventions as ``attention.masked_attention``).

    q, k, v, do [B, H, N, D]; mask [nqb, nkb] | [H, nqb, nkb] | [B, H, nqb, nkb];
    qblk[i] / kblk[j] block ids of query position i / key position j.
    Returns (dq, dk, dv) in float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    qblk = np.asarray(qblk, np.int64)
    kblk = np.asarray(kblk, np.int64)
    q_valid = np.ones(N, bool) if q_valid is None else np.asarray(q_valid, bool)
    k_valid = np.ones(Nk, bool) if k_valid is None else np.asarray(k_valid, bool)
    get = _mask_getter(mask, B, H)
    nkb = get(0, 0).shape[1]
    keys_of = _keys_by_block(kblk, k_valid, nkb)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            M = get(b, h)
            for qb in np.unique(qblk):
                rows = np.nonzero((qblk == qb) & q_valid)[0]
                if rows.size == 0:
                    continue
                kept = np.nonzero(M[qb])[0]
                if kept.size == 0:
                    continue
                keys = np.concatenate([keys_of[kb] for kb in kept])
                if keys.size == 0:
                    continue
                s = scale * (q[b, h, rows] @ k[b, h, keys].T)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                dp = do[b, h, rows] @ v[b, h, keys].T
                delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, h, rows] += scale * (ds @ k[b, h, keys])
                dk[b, h, keys] += scale * (ds.T @ q[b, h, rows])
                dv[b, h, keys] += p.T @ do[b, h, rows]
    return dq, dk, dv


def block_sparse_attention_bwd(q, k, v, do, mask, bs: int, blk_len=None, scale=None):
    """Blocked layout: position i belongs to block i // bs; blk_len (optional) gives
    the number of valid leading positions of each block."""
    N = np.asarray(q).shape[2]
    pos = np.arange(N)
    valid = block_valid(N, bs, blk_len)
    return masked_attention_bwd(q, k, v, do, mask, pos // bs, pos // bs, scale, valid, valid)


def kept_flops_bwd(mask, bs: int, N: int, D: int, blk_len=None, B: int = 1, H: int = 1) -> float:
    """Algorithmic flops of the backward pass: per valid kept (query, key) pair,
    2 D each for S (recomputed), dP, dV, dQ and dK -> 10 D."""
    from .attention import kept_flops
    return kept_flops(mask, bs, N, D, blk_len, B, H) * 10.0 / 4.0


def block_sparse_attention_bwd_rows(q, k, v, do, mask, bs: int, q_rows, k_rows, blk_len=None, scale=None):
    """The same gradients at selected positions only, for checks at full video
    sizes: dq at the query rows ``q_rows`` and (dk, dv) at the key rows ``k_rows``.

    dq_i needs query i's own softmax row over J(i); dk_j and dv_j need the rows of
    every query whose block keeps block(j), so the softmax of each such query block
    is formed once (over all of its kept keys) and its column j read off. Returns
    float64 dq [B, H, len(q_rows), D], dk and dv [B, H, len(k_rows), D].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    q_rows = np.asarray(q_rows, np.int64)
    k_rows = np.asarray(k_rows, np.int64)
    pos = np.arange(N)
    blk = pos // bs
    valid = block_valid(N, bs, blk_len)
    get = _mask_getter(mask, B, H)
    nb = get(0, 0).shape[1]
    keys_of = _keys_by_block(blk, valid, nb)

    dq = np.zeros((B, H, q_rows.size, D))
    dk = np.zeros((B, H, k_rows.size, D))
    dv = np.zeros((B, H, k_rows.size, D))
    for b in range(B):
        for h in range(H):
            M = get(b, h)
            cache = {}

            def block_terms(qb):
                # (rows, keys, P, dS) of query block qb, or None when it keeps nothing
                if qb not in cache:
                    rows = np.nonzero((blk == qb) & valid)[0]
                    kept = np.nonzero(M[qb])[0]
                    keys = np.concatenate([keys_of[kb] for kb in kept]) if kept.size else np.zeros(0, np.int64)
                    if rows.size == 0 or keys.size == 0:
                        cache[qb] = None
                    else:
                        s = scale * (q[b, h, rows] @ k[b, h, keys].T)
                        e = np.exp(s - s.max(axis=1, keepdims=True))
                        p = e / e.sum(axis=1, keepdims=True)
                        dp = do[b, h, rows] @ v[b, h, keys].T
                        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                        cache[qb] = (rows, keys, p, ds)
                return cache[qb]

            for r, i in enumerate(q_rows):
                t = block_terms(blk[i]) if valid[i] else None
                if t is None:
                    continue
                rows, keys, p, ds = t
                at = np.searchsorted(rows, i)
                dq[b, h, r] = scale * (ds[at] @ k[b, h, keys])
            for r, j in enumerate(k_rows):
                if not valid[j]:
                    continue
                for qb in np.nonzero(M[:, blk[j]])[0]:
                    t = block_terms(qb)
                    if t is None:
                        continue
                    rows, keys, p, ds = t
                    col = np.nonzero(keys == j)[0][0]
                    dv[b, h, r] += p[:, col] @ do[b, h, rows]
                    dk[b, h, r] += scale * (ds[:, col] @ q[b, h, rows])
    return dq, dk, dv
