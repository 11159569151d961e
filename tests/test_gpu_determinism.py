"""Determinism of the hot-path calls (the same call twice on the same inputs
gives the same bits): a race on LDS, a missing barrier or a read of scratch
left by an earlier call would show up here. Every call runs at the benched
Wan 480p shape (12 heads, 21 x 30 x 52 tokens) or at its layer's own shape,
with a different call in between so that scratch and caches hold other data
on the second run."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from oracle import masks as OM
from tests.gpu_util import announce, dev, dev_i32, dev_u8
from workloads import WAN480, WAN480_CUBE, WAN480_SEMANTIC, make_qkv, profile_rows

pytestmark = pytest.mark.gpu


def same(a, b, what):
    """Bit-identical tensors (or tuples of tensors)."""
    if isinstance(a, (tuple, list)):
        for i, (x, y) in enumerate(zip(a, b)):
            same(x, y, f"{what}[{i}]")
        return
    assert a.shape == b.shape and a.dtype == b.dtype, what
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"{what}: not bit-identical"


@pytest.fixture(scope="module")
def wan():
    q, k, v = make_qkv(WAN480)
    return dev(q), dev(k), dev(v)


def cands(w, device="cuda"):
    return PL.svg_masks(w.grid, w.bs, w.extra["w_spatial"], w.extra["w_temporal"], device)


def test_profile_twice(wan):
    announce("determinism: profile")
    q, k, v = wan
    w = WAN480
    rows = dev_i32(profile_rows(w))
    cand = cands(w)
    a = V.vsa_profile_heads(q, k, v, w.grid, w.bs, rows, cand, [0, 1])
    # another profile in between (other candidates) leaves other records in its scratch
    V.vsa_profile_heads(q, k, v, w.grid, w.bs, rows, cand.flip(0).contiguous(), [1, 0])
    b = V.vsa_profile_heads(q, k, v, w.grid, w.bs, rows, cand, [0, 1])
    same(a, b, "profile")


def test_chosen_split_twice(wan):
    announce("determinism: chosen attention, 6/6 split")
    q, k, v = wan
    w = WAN480
    cand = cands(w)
    ch = torch.tensor([[h % 2 for h in range(w.H)]], dtype=torch.int32, device="cuda")
    a = V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch)
    V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], 1 - ch)
    b = V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch)
    same(a, b, "chosen")


def test_backward_twice(wan):
    announce("determinism: backward")
    q, k, v = wan
    w = WAN480
    mask = dev_u8(np.broadcast_to(OM.pattern_mask(w.grid, w.bs, "spatial", 1), (1, w.H, w.nb, w.nb)).copy())
    o, lse = V.vsa_block_sparse_attn_fwd(q, k, v, w.bs, mask=mask, return_lse=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    a = V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, w.bs, mask=mask)
    V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, -do, w.bs, mask=mask)
    b = V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, w.bs, mask=mask)
    same(a, b, "backward")


def test_fp8_twice(wan):
    announce("determinism: fp8")
    q, k, v = wan
    w = WAN480
    mask = dev_u8(np.broadcast_to(OM.pattern_mask(w.grid, w.bs, "spatial", 1), (1, w.H, w.nb, w.nb)).copy())

    def run():
        q8, qs = V.vsa_fp8_quantize(q, V.VSA_FP8_ROWS)
        k8, ks = V.vsa_fp8_quantize(k, V.VSA_FP8_ROWS)
        vt, vs = V.vsa_fp8_quantize(v, V.VSA_FP8_VT)
        return (q8, k8, vt, qs, ks, vs) + tuple(V.vsa_block_sparse_attn_fwd_fp8(q8, k8, vt, qs, ks, vs, w.bs,
                                                                                mask=mask, return_lse=True))
    a = run()
    V.vsa_fp8_quantize(k, V.VSA_FP8_VT)
    b = run()
    same(a, b, "fp8")


def test_cube_layer_twice():
    announce("determinism: cube layer steps")
    w = WAN480_CUBE
    q, k, v = (dev(x) for x in make_qkv(w))
    bl = V.vsa_cube_block_len(w.grid)

    def run():
        qc = V.vsa_permute(q, w.grid, V.VSA_PERM_CUBE4)
        kc = V.vsa_permute(k, w.grid, V.VSA_PERM_CUBE4)
        vc = V.vsa_permute(v, w.grid, V.VSA_PERM_CUBE4)
        S, qp, kp = V.vsa_block_scores(qc, kc, 64, blk_len=bl)
        idx, cnt = V.vsa_select_topk(S, 93, w.extra["top_p"])
        oc = V.vsa_block_sparse_attn_fwd(qc, kc, vc, 64, kv_idx=idx, kv_cnt=cnt, blk_len=bl)
        return qc, S, qp, kp, idx, cnt, V.vsa_permute(oc, w.grid, V.VSA_PERM_CUBE4, inverse=True)
    a = run()
    b = run()
    # entries past a row's count are unspecified: compare the kept prefixes
    idx_a, cnt_a, idx_b, cnt_b = a[4], a[5], b[4], b[5]
    same(cnt_a, cnt_b, "cube kv_cnt")
    keep = torch.arange(idx_a.shape[-1], device="cuda") < cnt_a.unsqueeze(-1)
    assert torch.equal(idx_a[keep], idx_b[keep]), "cube kv_idx: not bit-identical"
    same(a[:4] + a[6:], b[:4] + b[6:], "cube layer")


def test_semantic_layer_twice():
    announce("determinism: semantic layer")
    w = WAN480_SEMANTIC
    q, k, v = (dev(x) for x in make_qkv(w))
    e = w.extra
    a = PL.semantic_layer(q, k, v, e["Cq"], e["Ck"], e["iters"], e["top_p"])
    PL.semantic_layer(k, q, v, e["Cq"], e["Ck"], e["iters"], e["top_p"])
    b = PL.semantic_layer(q, k, v, e["Cq"], e["Ck"], e["iters"], e["top_p"])
    same(a, b, "semantic layer")


@pytest.mark.parametrize("mode", [V.VSA_SKIPARSE_TOKEN, V.VSA_SKIPARSE_GROUP])
def test_skiparse_layer_twice(wan, mode):
    announce(f"determinism: skiparse mode {mode}")
    q, k, v = wan
    w = WAN480
    a = PL.skiparse_layer(q, k, v, w.grid, mode, 2, 128)
    b = PL.skiparse_layer(q, k, v, w.grid, mode, 2, 128)
    same(a, b, "skiparse layer")
