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
