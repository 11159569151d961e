"""GPU parity of vsa_block_sparse_attn_fwd against the oracle (element by element
on small grids spanning several tiles with ragged tails; sampled rows at the
full video shapes), plus determinism and mask/list equivalence."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import attention as OA
from oracle import layout as OL
from oracle import masks as OM
from tests.gpu_util import (announce, assert_close_bf16, assert_lse_close, dev, dev_i32, dev_u8, host,
                            F32_MAX_ABS)
from workloads import TINY, WAN480, HUNYUAN720, LONG126, make_qkv, random_block_mask, sample_rows

pytestmark = pytest.mark.gpu


def rand_mask(H, nb, density, seed, diag=True):
    m = (np.random.default_rng(seed).random((1, H, nb, nb)) < density).astype(np.uint8)
    if diag:
        m[:, :, np.arange(nb), np.arange(nb)] = 1
    return m


def test_tiny_fp32_random_mask_full_oracle():
    w = TINY
    announce("attn tiny fp32 4x8x8 D=64 bs=64")
    q, k, v = make_qkv(w)
    mask = random_block_mask(w)[None]                       # [1, H, 4, 4], 8 of 16 per head
    assert (mask.sum((-1, -2)) == 8).all()
    o, lse = V.vsa_block_sparse_attn_fwd(dev(q, torch.float32), dev(k, torch.float32), dev(v, torch.float32),
                                         w.bs, mask=dev_u8(mask), return_lse=True)
    ro, rl = OA.block_sparse_attention(q, k, v, mask, w.bs)
    assert np.abs(host(o) - ro).max() <= F32_MAX_ABS
    assert_lse_close(host(lse), rl, "tiny lse")


@pytest.mark.parametrize("N,bs,D,H", [(1000, 128, 128, 3), (777, 64, 128, 2), (640, 128, 64, 2), (300, 64, 64, 2),
                                      (128, 128, 128, 1), (65, 64, 128, 1)])
def test_bf16_random_masks_ragged_full_oracle(N, bs, D, H):
    announce(f"attn bf16 random N={N} bs={bs} D={D} H={H}")
    rng = np.random.default_rng(N + bs + D)
    q = rng.standard_normal((1, H, N, D)).astype(np.float32)
    k = rng.standard_normal((1, H, N, D)).astype(np.float32)
    v = rng.standard_normal((1, H, N, D)).astype(np.float32)
    qd, kd, vd = dev(q), dev(k), dev(v)
    q, k, v = host(qd), host(kd), host(vd)                   # the exact bf16 values the GPU sees
    nb = -(-N // bs)
    mask = rand_mask(H, nb, 0.4, N)
    o, lse = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=dev_u8(mask), return_lse=True)
    ro, rl = OA.block_sparse_attention(q, k, v, mask, bs)
    assert_close_bf16(host(o), ro, f"N={N} bs={bs} D={D}")
    assert_lse_close(host(lse), rl, f"N={N} bs={bs} D={D}")
    # list form gives bit-identical results to the mask form
    idx, cnt = OM.mask_to_list(mask)
    o2 = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, kv_idx=dev_i32(idx), kv_cnt=dev_i32(cnt))
    assert torch.equal(o, o2)
    # determinism
    o3 = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=dev_u8(mask))
    assert torch.equal(o, o3)



# Per-element bound from the kernel's roundings: P is rounded to bf16 (8
# significant bits: relative error at most 2^-8) before P V and O once to bf16
# (2^-8 of |O|); the fp32 scores, sums and exponentials add under 2e-4 relative
# at these sizes. With p the exact normalised probabilities:
# |O_kernel - O| <= (2^-8 + 2e-4) (sum_j p_j |v_j| + |O|).
@pytest.mark.parametrize("N,bs,amp", [(1000, 128, 1.0), (777, 64, 1.0), (1000, 128, 3.0)])
def test_bf16_attention_within_its_rounding_bound(N, bs, amp):
    announce(f"attn bf16 rounding bound N={N} bs={bs} amp={amp}")
    rng = np.random.default_rng(N + bs + 7)
    H, D = 2, 128
    q, k, v = (rng.standard_normal((1, H, N, D)).astype(np.float32) * a for a in (amp, amp, 1.0))
    qd, kd, vd = dev(q), dev(k), dev(v)
    q, k, v = host(qd), host(kd), host(vd)
    mask = rand_mask(H, -(-N // bs), 0.4, N + 1)
    o = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=dev_u8(mask))
    ro, _, p = OA.block_sparse_attention(q, k, v, mask, bs, return_probs=True)
    bound = (2.0 ** -8 + 2e-4) * (np.einsum("bhij,bhjd->bhid", p, np.abs(v)) + np.abs(ro))
    d = np.abs(host(o) - ro)
    print(f"bf16 rounding bound N={N} bs={bs} amp={amp}: worst |d| / bound {(d / bound).max():.3f}, "
          f"max |d| {d.max():.3e}, mean |d| / mean |O| {d.mean() / np.abs(ro).mean():.3e}")
    assert (d <= bound).all()


@pytest.mark.parametrize("slope", [10.0, 3.0, -6.0])
def test_offset_paths_with_scores_rising_or_falling_along_the_keys(slope):
    """Every query's score moves by `slope` log2 units per 64 keys (plus a little
    noise), so the kernel's running offset has to move on every sub-tile (10), the
    lanes' p sums pass 2^8 while the offset may stay (3), or the first sub-tile
    holds the row maximum and the offset never moves (-6). Each element within the
    bound of its two bf16 roundings; LSE to the oracle."""
    announce(f"attn bf16 offset paths slope={slope}")
    rng = np.random.default_rng(31)
    N, bs, D, H = 500, 128, 128, 2
    scale = 1.0 / np.sqrt(D)
    per_key = slope / 64 / (scale * np.log2(np.e))       # channel-0 step of k per key
    q = (0.05 * rng.standard_normal((1, H, N, D))).astype(np.float32)
    k = (0.05 * rng.standard_normal((1, H, N, D))).astype(np.float32)
    v = rng.standard_normal((1, H, N, D)).astype(np.float32)
    q[..., 0] = 1.0
    k[..., 0] = per_key * (np.arange(N) - (N - 1 if slope > 0 else 0))
    qd, kd, vd = dev(q), dev(k), dev(v)
    q, k, v = host(qd), host(kd), host(vd)
    mask = np.ones((1, H, 4, 4), np.uint8)
    o, lse = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=dev_u8(mask), return_lse=True)
    ro, rl, p = OA.block_sparse_attention(q, k, v, mask, bs, return_probs=True)
    bound = (2.0 ** -8 + 2e-4) * (np.einsum("bhij,bhjd->bhid", p, np.abs(v)) + np.abs(ro))
    d = np.abs(host(o) - ro)
    print(f"offset paths slope={slope}: worst |d| / bound {(d / bound).max():.3f}")
    assert (d <= bound).all()
    assert_lse_close(host(lse), rl, f"offset paths slope={slope}")

def test_empty_rows_and_scaled_logits():
    announce("attn bf16 empty rows / large logits")
    N, bs, D, H = 512, 128, 128, 2
    rng = np.random.default_rng(5)
    q = (4.0 * rng.standard_normal((1, H, N, D))).astype(np.float32)
    k = (4.0 * rng.standard_normal((1, H, N, D))).astype(np.float32)
    v = rng.standard_normal((1, H, N, D)).astype(np.float32)
    qd, kd, vd = dev(q), dev(k), dev(v)
    q, k, v = host(qd), host(kd), host(vd)
    mask = rand_mask(H, 4, 0.5, 9, diag=False)
    mask[0, 0, 2, :] = 0                                    # an empty query block
    o, lse = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=dev_u8(mask), return_lse=True)
    ro, rl = OA.block_sparse_attention(q, k, v, mask, bs)
    go, gl = host(o), host(lse)
    assert (go[0, 0, 256:384] == 0).all() and np.isneginf(gl[0, 0, 256:384]).all()
    assert_close_bf16(go, ro, "large logits")
    assert_lse_close(gl, rl, "large logits", tol=2e-3)


def test_cube_layout_blk_len_small_grid():
    """Cube layout: partial cubes are padded slots (invalid keys, zero outputs)."""
    grid = (5, 6, 9)
    announce(f"attn bf16 cube layout grid={grid}")
    H, D = 2, 128
    rng = np.random.default_rng(7)
    N = int(np.prod(grid))
    x = [rng.standard_normal((1, H, N, D)).astype(np.float32) for _ in range(3)]
    slot, counts, n_slots = OL.cube_map(*grid, 4)
    xc = [OL.permute(t, grid, "cube4") for t in x]
    qd, kd, vd = (dev(t) for t in xc)
    qc, kc, vc = host(qd), host(kd), host(vd)
    nc = counts.size
    mask = rand_mask(H, nc, 0.5, 3)
    blk = dev_i32(counts)
    o, lse = V.vsa_block_sparse_attn_fwd(qd, kd, vd, 64, mask=dev_u8(mask), blk_len=blk, return_lse=True)
    ro, rl = OA.block_sparse_attention(qc, kc, vc, mask, 64, counts)
    go = host(o)
    pad = np.setdiff1d(np.arange(n_slots), slot)
    assert (go[:, :, pad] == 0).all()
    assert_close_bf16(go, ro, "cube")
    assert_lse_close(host(lse), rl, "cube")


def _spatial_case(w, H, n_random, seed):
    q, k, v = make_qkv(w, H=H)
    mask = OM.pattern_mask(w.grid, w.bs, "spatial", w.extra.get("w_spatial", w.extra.get("w_local", 1)))
    rows = sample_rows(w.N, w.bs, n_random, seed)
    return q, k, v, mask, rows


@pytest.mark.parametrize("w,H", [(WAN480, 12), (HUNYUAN720, 3), (LONG126, 2)])
def test_full_shape_spatial_masks_sampled_rows(w, H):
    """The video shapes at full N (the benchmarked launch configuration), on
    every block's first and last row plus seeded rows."""
    announce(f"attn bf16 full shape {w.name} H={H}")
    q, k, v, mask, rows = _spatial_case(w, H, 1024, w.seed)
    idx, cnt = OM.mask_to_list(mask)
    B = 1
    kv_idx = np.broadcast_to(idx, (B, H) + idx.shape).copy()
    kv_cnt = np.broadcast_to(cnt, (B, H) + cnt.shape).copy()
    o, lse = V.vsa_block_sparse_attn_fwd(dev(q), dev(k), dev(v), w.bs, kv_idx=dev_i32(kv_idx),
                                         kv_cnt=dev_i32(kv_cnt), return_lse=True)
    go, gl = host(o)[:, :, rows], host(lse)[:, :, rows]
    ro, rl = OA.block_sparse_attention(q, k, v, mask, w.bs, rows=rows)
    assert_close_bf16(go, ro, w.name)
    assert_lse_close(gl, rl, w.name)


@pytest.mark.parametrize("w,H", [(WAN480, 2), (HUNYUAN720, 3), (LONG126, 2)])
def test_every_tile_kept_at_the_large_shapes_sampled_rows(w, H):
    """The dense baselines the speedups are quoted against: every tile kept at the
    Wan, HunyuanVideo and long-horizon shapes (at the last two, 8 heads' K and V
    outgrow the last-level cache and work items are dealt to the XCDs in runs); sampled rows
    (first and last row of every 16th block and of the last block, plus seeded
    rows) against dense attention."""
    announce(f"attn bf16 every tile kept {w.name} H={H}")
    qd, kd, vd = (dev(x) for x in make_qkv(w, H=H))
    q, k, v = host(qd), host(kd), host(vd)                   # the exact bf16 values the GPU sees
    nb = w.nb
    mask = np.ones((1, H, nb, nb), np.uint8)
    o, lse = V.vsa_block_sparse_attn_fwd(qd, kd, vd, w.bs, mask=dev_u8(mask), return_lse=True)
    blocks = np.r_[np.arange(0, nb, 16), nb - 1]
    rows = np.unique(np.concatenate([blocks * w.bs, np.minimum(blocks * w.bs + w.bs, w.N) - 1,
                                     np.random.default_rng(w.seed).choice(w.N, 256, replace=False)]))
    ro, rl = OA.dense_attention(q, k, v, rows=rows)
    assert_close_bf16(host(o)[:, :, rows], ro, f"{w.name} every tile kept")
    assert_lse_close(host(lse)[:, :, rows], rl, f"{w.name} every tile kept")

