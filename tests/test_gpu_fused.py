"""GPU parity of vsa_block_sparse_attn_fwd_permuted (frame-major permutation
folded into the attention kernel): bit-identical to the separate
permute -> attention -> inverse-permute sequence, and close to the oracle's
masked attention evaluated through the frame-major map."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import attention as OA
from oracle import layout as OL
from oracle import masks as OM
from oracle import pipeline as OP
from tests.gpu_util import announce, assert_close_bf16, assert_lse_close, dev, dev_i32, dev_u8, host
from workloads import HUNYUAN720, WAN480, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

FM = V.VSA_PERM_FRAME_MAJOR


def separate(qd, kd, vd, grid, bs, head_fm, **blocks):
    qm = V.vsa_permute(qd, grid, FM, False, head_fm)
    km = V.vsa_permute(kd, grid, FM, False, head_fm)
    vm = V.vsa_permute(vd, grid, FM, False, head_fm)
    om, lm = V.vsa_block_sparse_attn_fwd(qm, km, vm, bs, return_lse=True, **blocks)
    return V.vsa_permute(om, grid, FM, True, head_fm), lm


def lse_to_natural(lm, grid, head_fm):
    pi = torch.from_numpy(OL.frame_major_map(*grid)).to(lm.device)
    out = lm.clone()
    for h, f in enumerate(head_fm):
        if f:
            out[:, h] = lm[:, h, pi]
    return out


def oracle_mixed(q, k, v, grid, bs, mask, head_fm, rows=None):
    """Oracle output in natural order: a frame-major head's blocks are taken
    along pi (query block of token n = pi[n] // bs, same for keys)."""
    N = q.shape[2]
    pi = OL.frame_major_map(*grid)
    nat = np.arange(N) // bs
    fmb = pi // bs
    R = N if rows is None else len(rows)
    o = np.zeros((q.shape[0], q.shape[1], R, q.shape[3]))
    lse = np.zeros((q.shape[0], q.shape[1], R))
    for h, f in enumerate(head_fm):
        blk = fmb if f else nat
        oh, lh = OA.masked_attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], mask[:, h:h + 1], blk, blk,
                                     rows=rows)
        o[:, h], lse[:, h] = oh[:, 0], lh[:, 0]
    return o, lse


@pytest.mark.parametrize("grid,bs,form", [((5, 6, 10), 64, "mask"), ((5, 6, 10), 128, "list"),
                                          ((7, 9, 11), 128, "mask"), ((3, 4, 5), 64, "list"),
                                          ((2, 3, 40), 128, "list")])
def test_fused_matches_separate_and_oracle_small(grid, bs, form):
    H, head_fm = 3, [1, 0, 1]
    N = int(np.prod(grid))
    nb = -(-N // bs)
    announce(f"fused attn grid={grid} bs={bs} form={form}")
    rng = np.random.default_rng(N + bs)
    qd, kd, vd = (dev(rng.standard_normal((1, H, N, 128)).astype(np.float32)) for _ in range(3))
    q, k, v = host(qd), host(kd), host(vd)
    mask = (rng.random((1, H, nb, nb)) < 0.35).astype(np.uint8)
    mask[0, 1, 0, :] = 0                                       # a query block with nothing kept
    if form == "mask":
        blocks = dict(mask=dev_u8(mask))
    else:
        idx, cnt = OM.mask_to_list(mask)
        blocks = dict(kv_idx=dev_i32(idx), kv_cnt=dev_i32(cnt))
    o_sep, l_sep = separate(qd, kd, vd, grid, bs, head_fm, **blocks)
    o_f, l_f = V.vsa_block_sparse_attn_fwd_permuted(qd, kd, vd, grid, bs, head_fm=head_fm, return_lse=True, **blocks)
    assert torch.equal(o_f, o_sep), "fused output differs from the separate permutes"
    assert torch.equal(l_f, lse_to_natural(l_sep, grid, head_fm)), "fused LSE differs"
    ro, rl = oracle_mixed(q, k, v, grid, bs, mask, head_fm)
    assert_close_bf16(host(o_f), ro, f"fused grid={grid}")
    assert_lse_close(host(l_f), rl, f"fused grid={grid}")


def test_fused_no_heads_moved_equals_plain_attention():
    grid, bs, H = (4, 8, 9), 128, 2
    N = int(np.prod(grid))
    nb = -(-N // bs)
    announce("fused attn, no frame-major head")
    rng = np.random.default_rng(3)
    qd, kd, vd = (dev(rng.standard_normal((1, H, N, 128)).astype(np.float32)) for _ in range(3))
    mask = dev_u8((rng.random((1, H, nb, nb)) < 0.5).astype(np.uint8))
    o1 = V.vsa_block_sparse_attn_fwd(qd, kd, vd, bs, mask=mask)
    for hf in (None, [0, 0]):
        o2 = V.vsa_block_sparse_attn_fwd_permuted(qd, kd, vd, grid, bs, head_fm=hf, mask=mask)
        assert torch.equal(o1, o2)


def test_fused_wan_full_shape_mixed_heads():
    """Wan 480p, 12 heads, spatial w=1 on even heads and temporal w=0 (frame-major)
    on odd heads, in the launch configuration of the step: bit-identical to the
    separate permutes; sampled rows against the oracle."""
    w = WAN480
    announce("fused attn wan full mixed heads")
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    head_fm = [h % 2 for h in range(w.H)]
    cand = np.stack([OM.pattern_mask(w.grid, w.bs, "spatial", 1), OM.pattern_mask(w.grid, w.bs, "temporal", 0)])
    idx, cnt = V.vsa_mask_to_list(dev_u8(cand), head_mask_idx=head_fm, B=1)
    o_sep, _ = separate(qd, kd, vd, w.grid, w.bs, head_fm, kv_idx=idx, kv_cnt=cnt)
    o_f = V.vsa_block_sparse_attn_fwd_permuted(qd, kd, vd, w.grid, w.bs, head_fm=head_fm, kv_idx=idx, kv_cnt=cnt)
    assert torch.equal(o_f, o_sep)
    rows = sample_rows(w.N, w.bs, 512, 21)
    mask = cand[head_fm][None]
    ro, _ = oracle_mixed(host(qd), host(kd), host(vd), w.grid, w.bs, mask, head_fm, rows=rows)
    assert_close_bf16(host(o_f)[:, :, rows], ro, "fused wan")


@pytest.mark.parametrize("grid,bs", [((5, 6, 10), 64), ((7, 9, 11), 128)])
def test_chosen_matches_permuted_per_head_masks(grid, bs):
    """Device-side choice: B = 2, per-(b, h) choices over two candidates (natural
    and frame-major), one out-of-range entry (that head keeps nothing)."""
    B, H = 2, 3
    N = int(np.prod(grid))
    nb = -(-N // bs)
    announce(f"chosen attn grid={grid} bs={bs}")
    rng = np.random.default_rng(N * 7 + bs)
    qd, kd, vd = (dev(rng.standard_normal((B, H, N, 128)).astype(np.float32)) for _ in range(3))
    cand = (rng.random((2, nb, nb)) < 0.4).astype(np.uint8)
    layout = [0, 1]
    choice = np.array([[0, 1, 1], [1, 7, 0]], np.int32)
    o_c, l_c = V.vsa_block_sparse_attn_fwd_chosen(qd, kd, vd, grid, bs, dev_u8(cand), layout, dev_i32(choice),
                                                  return_lse=True)
    for b in range(B):
        ok = (choice[b] >= 0) & (choice[b] < 2)
        masks = np.stack([cand[c] if o else np.zeros((nb, nb), np.uint8) for c, o in zip(choice[b], ok)])[None]
        head_fm = [layout[c] if o else 0 for c, o in zip(choice[b], ok)]
        o_p, l_p = V.vsa_block_sparse_attn_fwd_permuted(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(),
                                                        vd[b:b + 1].contiguous(), grid, bs, head_fm=head_fm,
                                                        mask=dev_u8(masks), return_lse=True)
        assert torch.equal(o_c[b:b + 1], o_p), f"batch {b}: output differs"
        assert torch.equal(l_c[b:b + 1], l_p), f"batch {b}: LSE differs"
    assert (host(o_c)[1, 1] == 0).all() and np.isneginf(host(l_c)[1, 1]).all()


def test_chosen_wan_full_shape_matches_list_path():
    w = WAN480
    announce("chosen attn wan full")
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    sel = [(h * 5) % 3 % 2 for h in range(w.H)]
    cand = dev_u8(np.stack([OM.pattern_mask(w.grid, w.bs, "spatial", 1), OM.pattern_mask(w.grid, w.bs, "temporal", 0)]))
    o_c = V.vsa_block_sparse_attn_fwd_chosen(qd, kd, vd, w.grid, w.bs, cand, [0, 1], dev_i32(np.array([sel])))
    idx, cnt = V.vsa_mask_to_list(cand, head_mask_idx=sel, B=1)
    o_l = V.vsa_block_sparse_attn_fwd_permuted(qd, kd, vd, w.grid, w.bs, head_fm=sel, kv_idx=idx, kv_cnt=cnt)
    assert torch.equal(o_c, o_l)


def test_fused_hunyuan_full_shape_sampled():
    """HunyuanVideo 720p in the launch configuration the benchmark times: 24 heads,
    118,800 tokens, even heads spatial w=2, odd heads temporal w=276 through the
    frame-major map folded into the kernel; sampled rows of two spatial and two
    temporal heads against the oracle's pipeline."""
    w = HUNYUAN720
    announce("fused attn hunyuan full shape")
    q, k, v = make_qkv(w)
    head_fm = [h % 2 for h in range(w.H)]
    cand = np.stack([OM.pattern_mask(w.grid, w.bs, "spatial", w.extra["w_spatial"]),
                     OM.pattern_mask(w.grid, w.bs, "temporal", w.extra["w_temporal"])])
    idx, cnt = V.vsa_mask_to_list(dev_u8(cand), head_mask_idx=head_fm, B=1)
    o = V.vsa_block_sparse_attn_fwd_permuted(dev(q), dev(k), dev(v), w.grid, w.bs, head_fm=head_fm, kv_idx=idx,
                                             kv_cnt=cnt)
    heads = [0, 1, 22, 23]
    rows = sample_rows(w.N, w.bs, 128, 23)
    ro, _ = OP.svg_pipeline(q[:, heads], k[:, heads], v[:, heads], w.grid, w.bs, [[head_fm[h] for h in heads]],
                            w.extra["w_spatial"], w.extra["w_temporal"], rows=rows)
    assert_close_bf16(host(o[:, heads])[:, :, rows], ro, "fused hunyuan")
