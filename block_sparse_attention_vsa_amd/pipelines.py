"""The three flows of the pages, as sequences of libvsa calls on one stream.

Each function only orders calls to the library's entry points and allocates
their outputs; every step runs in a HIP kernel.

* svg_layer: Sparse Video-Gen page, "Approach": pattern masks, per-head choice
  from sampled rows, frame-major permutation of temporal heads, block-sparse
  attention, inverse permutation (by default the choice is read on the device
  and the two permutations are folded into the attention kernel).
* cube_layer: USV page, Figure 2 caption (3D cubes, top-k cube selection) with
  the top-p budget of the Sparse VideoGen2 page, Abstract.
* long_layer: machinebrief LVSA article (block-sparse attention at a long
  horizon): a local window forced, the rest of a fixed budget by pooled score.
* semantic_layer: Sparse VideoGen2 page, Abstract: k-means of Q and K per head,
  cluster-major storage, size-weighted top-p over cluster pairs, attention over
  the kept clusters without padding, and O moved back to natural order.
* skiparse_layer: OSP-Next page, "Method": a fixed token-wise or group-wise
  spatial pattern, stored subset by subset so it is a block-diagonal mask of
  dense tiles.
"""
from __future__ import annotations

import math

from . import (VSA_PATTERN_SPATIAL, VSA_PATTERN_TEMPORAL, VSA_PERM_CUBE4, VSA_PERM_FRAME_MAJOR,
               vsa_block_scores, vsa_block_sparse_attn_fwd, vsa_block_sparse_attn_fwd_chosen,
               vsa_cube_block_len, vsa_cube_dims, vsa_mask_to_list,
               vsa_pattern_mask, vsa_permute, vsa_profile_heads, vsa_select_topk, vsa_kmeans,
               vsa_cluster_order, vsa_gather_rows, vsa_cluster_scores, vsa_varlen_sparse_attn_fwd,
               vsa_skiparse_block_len, vsa_skiparse_mask, vsa_skiparse_permute)


def svg_masks(grid, bs, w_spatial, w_temporal, device="cuda"):
    """Candidate masks [2, nb, nb]: 0 = spatial (natural order), 1 = temporal
    (frame-major order)."""
    import torch
    N = grid[0] * grid[1] * grid[2]
    nb = -(-N // bs)
    cand = torch.empty((2, nb, nb), dtype=torch.uint8, device=device)
    vsa_pattern_mask(grid, bs, VSA_PATTERN_SPATIAL, w_spatial, out=cand[0])
    vsa_pattern_mask(grid, bs, VSA_PATTERN_TEMPORAL, w_temporal, out=cand[1])
    return cand


def svg_layer(q, k, v, grid, bs, w_spatial, w_temporal, rows, scale=None, choice=None, cand=None, workspace=None,
              stats=None, fused=True):
    """Returns (o, choice_host). `choice` (host: [H], or [B][H]) skips the
    profiler; `rows` (device int32) are the sampled query rows otherwise. The
    host choice comes back as [H] for B = 1 and as [B][H] otherwise.

    fused (default): the attention kernel reads each (batch entry, head)'s choice
    on the device, compacts the chosen candidate's mask rows itself and applies
    the frame-major order of temporal heads in its loads and stores; the host
    copy of the choice is taken after the attention launch. fused=False (B = 1
    only): the same result, bit for bit, through host choice -> mask -> list ->
    permute -> attention -> inverse permute."""
    import torch
    B, H = q.shape[:2]
    if B != 1 and not fused:
        raise ValueError("the separate path permutes heads by a per-head choice; call it per batch entry")
    if cand is None:
        cand = svg_masks(grid, bs, w_spatial, w_temporal, q.device)
    if choice is None:
        _, ch = vsa_profile_heads(q, k, v, grid, bs, rows, cand, [0, 1], scale=scale, workspace=workspace)
    else:
        rows_c = [choice] if B == 1 and not isinstance(choice[0], (list, tuple)) else choice
        ch = torch.tensor([[int(c) for c in r] for r in rows_c], dtype=torch.int32, device=q.device)
        if tuple(ch.shape) != (B, H):
            raise ValueError(f"choice must give one candidate per (batch entry, head): {B} x {H}")
    if fused:
        o = vsa_block_sparse_attn_fwd_chosen(q, k, v, grid, bs, cand, [0, 1], ch, scale=scale)
        if stats is not None:
            stats.update(cand=cand, choice=ch)
        host_ch = [[int(c) for c in r] for r in ch.cpu().tolist()]
        return o, host_ch[0] if B == 1 else host_ch
    sel = [int(c) for c in ch[0].cpu().tolist()]           # host decision: which heads move
    qm = vsa_permute(q, grid, VSA_PERM_FRAME_MAJOR, False, sel)
    km = vsa_permute(k, grid, VSA_PERM_FRAME_MAJOR, False, sel)
    vm = vsa_permute(v, grid, VSA_PERM_FRAME_MAJOR, False, sel)
    idx, cnt = vsa_mask_to_list(cand, head_mask_idx=sel, B=B)
    om = vsa_block_sparse_attn_fwd(qm, km, vm, bs, kv_idx=idx, kv_cnt=cnt, scale=scale)
    o = vsa_permute(om, grid, VSA_PERM_FRAME_MAJOR, True, sel)
    if stats is not None:
        stats.update(kv_idx=idx, kv_cnt=cnt, cand=cand)
    return o, sel


def cube_budget(grid, k_frac):
    n_cubes, _ = vsa_cube_dims(grid)
    return n_cubes, max(1, int(math.floor(k_frac * n_cubes)))


def cube_layer(q, k, v, grid, k_frac, top_p, scale=None, stats=None):
    """Returns o in natural order."""
    n_cubes, k_max = cube_budget(grid, k_frac)
    qc = vsa_permute(q, grid, VSA_PERM_CUBE4)
    kc = vsa_permute(k, grid, VSA_PERM_CUBE4)
    blk = vsa_cube_block_len(grid, device=q.device)
    S, _, _ = vsa_block_scores(qc, kc, 64, blk_len=blk, scale=scale)
    idx, cnt = vsa_select_topk(S, k_max, top_p)
    # V is moved right before the attention reads it, so the last-level cache holds K and V then
    vc = vsa_permute(v, grid, VSA_PERM_CUBE4)
    oc = vsa_block_sparse_attn_fwd(qc, kc, vc, 64, kv_idx=idx, kv_cnt=cnt, blk_len=blk, scale=scale)
    o = vsa_permute(oc, grid, VSA_PERM_CUBE4, inverse=True)
    if stats is not None:
        stats.update(kv_idx=idx, kv_cnt=cnt, blk_len=blk, scores=S)
    return o


def long_layer(q, k, v, grid, bs, w_local, k_total, scale=None, stats=None):
    forced = vsa_pattern_mask(grid, bs, VSA_PATTERN_SPATIAL, w_local, device=q.device)
    S, _, _ = vsa_block_scores(q, k, bs, scale=scale)
    idx, cnt = vsa_select_topk(S, k_total, 1.0, forced=forced)
    o = vsa_block_sparse_attn_fwd(q, k, v, bs, kv_idx=idx, kv_cnt=cnt, scale=scale)
    if stats is not None:
        stats.update(kv_idx=idx, kv_cnt=cnt, forced=forced, scores=S)
    return o


def semantic_layer(q, k, v, Cq, Ck, iters, top_p, k_max=None, scale=None, stats=None):
    """Returns o in natural order; `stats` receives the intermediate tensors."""
    cq, lq, nq = vsa_kmeans(q, Cq, iters)
    ck, lk, nk = vsa_kmeans(k, Ck, iters)
    pq, oq = vsa_cluster_order(lq, Cq)
    pk, ok = vsa_cluster_order(lk, Ck)
    qs = vsa_gather_rows(q, pq)
    ks = vsa_gather_rows(k, pk)
    vs = vsa_gather_rows(v, pk)
    S = vsa_cluster_scores(cq, ck, nk, scale=scale)
    idx, cnt = vsa_select_topk(S, Ck if k_max is None else k_max, top_p)
    os_ = vsa_varlen_sparse_attn_fwd(qs, ks, vs, oq, ok, kv_idx=idx, kv_cnt=cnt, scale=scale)
    o = vsa_gather_rows(os_, pq, inverse=True)
    if stats is not None:
        stats.update(q_centroids=cq, k_centroids=ck, q_labels=lq, k_labels=lk, q_counts=nq, k_counts=nk,
                     q_perm=pq, k_perm=pk, q_off=oq, k_off=ok, scores=S, kv_idx=idx, kv_cnt=cnt)
    return o


def skiparse_layer(q, k, v, grid, mode, k_factor, bs=128, scale=None, stats=None):
    """Returns o in natural order: Q, K, V moved subset by subset, block-sparse
    attention under the block-diagonal mask with the blocks' valid lengths, O
    moved back."""
    qs = vsa_skiparse_permute(q, grid, mode, k_factor, bs)
    ks = vsa_skiparse_permute(k, grid, mode, k_factor, bs)
    vs = vsa_skiparse_permute(v, grid, mode, k_factor, bs)
    blk = vsa_skiparse_block_len(grid, mode, k_factor, bs, device=q.device)
    m = vsa_skiparse_mask(grid, mode, k_factor, bs, device=q.device)
    B, H = q.shape[:2]
    mask = m.expand(B, H, -1, -1).contiguous()
    idx, cnt = vsa_mask_to_list(mask)
    os_ = vsa_block_sparse_attn_fwd(qs, ks, vs, bs, kv_idx=idx, kv_cnt=cnt, blk_len=blk, scale=scale)
    o = vsa_skiparse_permute(os_, grid, mode, k_factor, bs, inverse=True)
    if stats is not None:
        stats.update(mask=m, blk_len=blk, kv_idx=idx, kv_cnt=cnt, permuted=(qs, ks, vs), o_permuted=os_)
    return o
