"""Semantic-aware permutation (test infrastructure only).

Sparse VideoGen2 page (Abstract): tokens are clustered by semantic similarity
with k-means and reordered so that the tokens of a cluster are contiguous; a
cluster's mean represents it when critical tokens are identified, and a top-p
budget picks, for every query cluster, the key clusters it attends to. The page
gives no further detail; the plainest reading, used here:

* k-means (Lloyd's algorithm) per (b, h), separately on the queries (Cq clusters)
  and on the keys (Ck clusters; values follow the keys). Seeds: the tokens at
  positions floor(c N / C). One iteration assigns every token to its nearest
  centroid in squared Euclidean distance, argmin_c ||x - m_c||^2 with the exact
  (fp64) centroids, ties to the lower index, and then replaces each centroid by
  the mean of its members (a cluster left empty keeps its centroid). After the
  last iteration the returned centroids are the means of the returned
  assignment.
* Cluster-major order: a stable sort of the tokens by cluster (members of a
  cluster keep their natural order); cluster c occupies the positions
  [off_c, off_c + n_c), off the exclusive prefix sum of the sizes n.
* Cluster-pair score, weighted by size: S_ab = scale <cq_a, ck_b> + log n_b. The
  softmax of a row of S is the share of query cluster a's attention that key
  cluster b would take if every key equalled its centroid (n_b keys, each with
  weight exp(scale <cq_a, ck_b>)); an empty key cluster scores -inf.
* Top-p over those scores with the selection rule of ``oracle.select``.
* Attention: query i of cluster a attends to the keys of the key clusters kept
  for a; this is ``oracle.attention.masked_attention`` with the cluster ids as
  block ids, so the permutation changes where rows are stored, not the result.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import masked_attention
from .select import select


def assign(x: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Nearest centroid of every row of x [N, D]: argmin_c ||x - m_c||^2 in fp64,
    the first minimum (lower index) on a tie. The squared distance is expanded as
    ||x||^2 + ||m_c||^2 - 2 <x, m_c> so that one matrix product serves all pairs."""
    x = np.asarray(x, np.float64)
    m = np.asarray(centroids, np.float64)
    d = (x * x).sum(axis=1)[:, None] + (m * m).sum(axis=1)[None, :] - 2.0 * (x @ m.T)
    return np.argmin(d, axis=1)


def update(x: np.ndarray, labels: np.ndarray, centroids: np.ndarray):
    """Member means (empty clusters keep their centroid) and member counts."""
    x = np.asarray(x, np.float64)
    C = centroids.shape[0]
    counts = np.bincount(labels, minlength=C)
    sums = np.zeros((C, x.shape[1]))
    np.add.at(sums, labels, x)
    out = np.asarray(centroids, np.float64).copy()
    nz = counts > 0
    out[nz] = sums[nz] / counts[nz, None]
    return out, counts


def kmeans(x: np.ndarray, C: int, iters: int):
    """Lloyd's k-means on x [N, D]: (centroids [C, D], labels [N], counts [C])."""
    x = np.asarray(x, np.float64)
    N = x.shape[0]
    assert 1 <= C <= N and iters >= 1
    cent = x[(np.arange(C) * N) // C].copy()
    for _ in range(iters):
        labels = assign(x, cent)
        cent, counts = update(x, labels, cent)
    return cent, labels, counts


def kmeans_heads(x: np.ndarray, C: int, iters: int):
    """k-means of every (b, h) of x [B, H, N, D]."""
    B, H, N, D = x.shape
    cent = np.zeros((B, H, C, D))
    labels = np.zeros((B, H, N), np.int64)
    counts = np.zeros((B, H, C), np.int64)
    for b in range(B):
        for h in range(H):
            cent[b, h], labels[b, h], counts[b, h] = kmeans(x[b, h], C, iters)
    return cent, labels, counts


def cluster_order(labels: np.ndarray, C: int):
    """Stable cluster-major order of one head: (perm, offsets) with perm[p] the
    token stored at position p and offsets [C + 1] the cluster boundaries."""
    labels = np.asarray(labels, np.int64)
    perm = np.argsort(labels, kind="stable")
    counts = np.bincount(labels, minlength=C)
    off = np.concatenate([[0], np.cumsum(counts)])
    return perm, off


def cluster_scores(cq: np.ndarray, ck: np.ndarray, k_counts: np.ndarray, scale: float) -> np.ndarray:
    """S_ab = scale <cq_a, ck_b> + log n_b (-inf for an empty key cluster)."""
    s = scale * (np.asarray(cq, np.float64) @ np.asarray(ck, np.float64).T)
    with np.errstate(divide="ignore"):
        bias = np.log(np.asarray(k_counts, np.float64))
    return s + bias[None, :]


def semantic_pipeline(q, k, v, Cq: int, Ck: int, iters: int, top_p: float, k_max=None, scale=None, rows=None):
    """The whole layer in natural coordinates: k-means of Q and K per head, size-
    weighted cluster scores, top-p selection, attention over the kept clusters.

    Returns (o, lse, parts) with parts = dict of labels, centroids, counts, scores
    and the kept lists (kv_idx [B, H, Cq, k_max], kv_cnt [B, H, Cq])."""
    q = np.asarray(q, np.float64)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    k_max = Ck if k_max is None else int(k_max)
    cq, lq, nq = kmeans_heads(q, Cq, iters)
    ck, lk, nk = kmeans_heads(np.asarray(k, np.float64), Ck, iters)
    S = np.zeros((B, H, Cq, Ck))
    for b in range(B):
        for h in range(H):
            S[b, h] = cluster_scores(cq[b, h], ck[b, h], nk[b, h], scale)
    idx, cnt = select(S, None, k_max, top_p)
    o = np.zeros((B, H, N if rows is None else len(rows), D))
    lse = np.zeros(o.shape[:3])
    for b in range(B):
        for h in range(H):
            mask = np.zeros((Cq, Ck), np.uint8)
            for a in range(Cq):
                mask[a, idx[b, h, a, :cnt[b, h, a]]] = 1
            ob, lb = masked_attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], mask,
                                      lq[b, h], lk[b, h], scale, rows=rows)
            o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]
    parts = dict(q_labels=lq, k_labels=lk, q_centroids=cq, k_centroids=ck, q_counts=nq, k_counts=nk, scores=S,
                 kv_idx=idx, kv_cnt=cnt)
    return o, lse, parts


def kept_flops_semantic(q_counts, k_counts, kv_idx, kv_cnt, D: int) -> float:
    """4 D per (query, key) pair of every kept (query cluster, key cluster)."""
    total = 0.0
    q_counts = np.asarray(q_counts)
    k_counts = np.asarray(k_counts)
    B, H, Cq = q_counts.shape
    for b in range(B):
        for h in range(H):
            for a in range(Cq):
                kept = kv_idx[b, h, a, :kv_cnt[b, h, a]]
                total += float(q_counts[b, h, a]) * float(k_counts[b, h, kept].sum())
    return 4.0 * D * total
