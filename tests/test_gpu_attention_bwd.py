"""GPU parity of vsa_block_sparse_attn_bwd (dQ, dK, dV) against the oracle's fp64
gradients: element by element on small ragged problems (mask and list forms,
both block sizes, padding, empty query blocks, key blocks nobody keeps), and on
sampled rows at the full cube-layout video shape with the top-p lists."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import attention_bwd as OB
from oracle import layout as OL
from oracle import masks as OM
from oracle import pipeline as OP
from oracle import select as OSel
from tests.gpu_util import announce, assert_grad_close, dev, dev_i32, dev_u8, host
from workloads import WAN480_CUBE, make_qkv, rng, to_bf16_values

pytestmark = pytest.mark.gpu


def inputs(B, H, N, seed, amp=1.0):
    g = np.random.default_rng(seed)
    q, k = (amp * g.standard_normal((B, H, N, 128)) for _ in range(2))
    v, do = (g.standard_normal((B, H, N, 128)) for _ in range(2))
    t = [dev(x) for x in (q, k, v, do)]
    return t, [host(x) for x in t]                     # device bf16 and the exact values it holds


def rand_mask(B, H, nb, density, seed):
    m = (np.random.default_rng(seed).random((B, H, nb, nb)) < density).astype(np.uint8)
    m[..., np.arange(nb), np.arange(nb)] = 1
    return m


def run(td, bs, mask=None, idx=None, cnt=None, blk_len=None):
    q, k, v, do = td
    kw = dict(mask=mask, kv_idx=idx, kv_cnt=cnt, blk_len=blk_len)
    o, lse = V.vsa_block_sparse_attn_fwd(q, k, v, bs, return_lse=True, **kw)
    return V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, bs, **kw)


def check(got, ref, what, **tol):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert_grad_close(host(g), r, f"{what} {name}", **tol)


@pytest.mark.parametrize("N,bs,H", [(1000, 128, 3), (777, 64, 2), (300, 64, 2), (128, 128, 1), (65, 64, 1),
                                    (1, 128, 1)])
def test_bwd_random_masks_ragged_full_oracle(N, bs, H):
    announce(f"attn bwd random N={N} bs={bs} H={H}")
    td, th = inputs(1, H, N, N + bs)
    nb = -(-N // bs)
    mask = rand_mask(1, H, nb, 0.4, N)
    g = run(td, bs, mask=dev_u8(mask))
    check(g, OB.block_sparse_attention_bwd(*th, mask, bs), f"N={N} bs={bs}")
    # list form (ascending lists): bit-identical to the mask form
    idx, cnt = OM.mask_to_list(mask)
    g2 = run(td, bs, idx=dev_i32(idx), cnt=dev_i32(cnt))
    for a, b in zip(g, g2):
        assert torch.equal(a, b)
    # bit-reproducible
    g3 = run(td, bs, mask=dev_u8(mask))
    for a, b in zip(g, g3):
        assert torch.equal(a, b)


@pytest.mark.parametrize("bs", [64, 128])
def test_bwd_padding_empty_blocks_and_batches(bs):
    """blk_len padding (a block with no valid slot, one with a single slot),
    padding slots holding large values, an empty query block and a key block no
    query keeps, with different masks per (b, h)."""
    announce(f"attn bwd padding bs={bs}")
    B, H, nb = 2, 2, 6
    N = nb * bs
    lens = np.array([bs, bs - 28, 0, bs // 2, bs, 1], np.int32)
    valid = np.arange(N) % bs < lens[np.arange(N) // bs]
    g0 = np.random.default_rng(bs)
    arrs = [g0.standard_normal((B, H, N, 128)) for _ in range(4)]
    for a in arrs:
        a[:, :, ~valid] = 300.0                        # padding contents must not matter
    td = [dev(a) for a in arrs]
    th = [host(t) for t in td]
    mask = rand_mask(B, H, nb, 0.5, bs + 1)
    mask[0, 1, 3, :] = 0                               # an empty query block
    mask[1, 0, :, 4] = 0                               # a key block nobody keeps
    blk = dev_i32(lens)
    g = run(td, bs, mask=dev_u8(mask), blk_len=blk)
    ref = OB.block_sparse_attention_bwd(*th, mask, bs, blk_len=lens)
    check(g, ref, f"padding bs={bs}")
    dq, dk, dv = (host(t) for t in g)
    for t in (dq, dk, dv):
        assert (t[:, :, ~valid] == 0).all()
    assert (dq[0, 1, 3 * bs:4 * bs] == 0).all()
    assert (dk[1, 0, 4 * bs:5 * bs] == 0).all() and (dv[1, 0, 4 * bs:5 * bs] == 0).all()


def test_bwd_large_logits():
    announce("attn bwd large logits")
    td, th = inputs(1, 2, 640, 21, amp=4.0)
    mask = rand_mask(1, 2, 5, 0.5, 22)
    g = run(td, 128, mask=dev_u8(mask))
    check(g, OB.block_sparse_attention_bwd(*th, mask, 128), "large logits", mean_rel=2.5e-2)


def test_bwd_unsorted_list_order():
    """Given the same forward outputs, dK and dV do not depend on the order of a
    list row (they walk the transposed block set); dQ sums in the list's order, so
    it matches to tolerance. (The forward itself sums in list order, so its LSE may
    differ in the last bits between orders; both backward calls share one.)"""
    announce("attn bwd unsorted lists")
    td, th = inputs(1, 2, 896, 31)
    mask = rand_mask(1, 2, 7, 0.45, 32)
    idx, cnt = OM.mask_to_list(mask)
    rev = idx.copy()
    for h in range(2):
        for qb in range(7):
            c = cnt[0, h, qb]
            rev[0, h, qb, :c] = idx[0, h, qb, :c][::-1]
    q, k, v, do = td
    o, lse = V.vsa_block_sparse_attn_fwd(q, k, v, 128, mask=dev_u8(mask), return_lse=True)
    ga = V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, 128, mask=dev_u8(mask))
    gr = V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, 128, kv_idx=dev_i32(rev), kv_cnt=dev_i32(cnt))
    assert torch.equal(ga[1], gr[1]) and torch.equal(ga[2], gr[2])
    check(gr, OB.block_sparse_attention_bwd(*th, mask, 128), "reversed lists")


def test_bwd_cube_wan_full_shape_sampled():
    """The cube-layout video shape (12 heads, 624 cubes of 64 slots, top-p lists
    of at most 93 blocks) in the launch configuration the benchmark times: dQ at
    sampled query slots and dK, dV at sampled key slots of two heads against the
    oracle; mask and list forms bit-identical."""
    w = WAN480_CUBE
    announce("attn bwd cube wan full shape")
    q, k, v = make_qkv(w)
    do = to_bf16_values(rng(w.seed, 40).standard_normal(q.shape).astype(np.float32))
    S = OP.cube_scores(q, k, w.grid)
    n_cubes = S.shape[-1]
    k_max = int(np.floor(w.extra["k_frac"] * n_cubes))
    idx, cnt = OSel.select(S, None, k_max, w.extra["top_p"])
    slot, counts, n_slots = OL.cube_map(*w.grid, 4)
    host_c = [OL.permute(x, w.grid, "cube4") for x in (q, k, v, do)]
    td = [dev(x) for x in host_c]
    blk = dev_i32(counts)
    g = run(td, 64, idx=dev_i32(idx), cnt=dev_i32(cnt), blk_len=blk)
    mask = OM.list_to_mask(idx, cnt, n_cubes)
    gm = run(td, 64, mask=dev_u8(mask), blk_len=blk)
    for a, b in zip(g, gm):
        assert torch.equal(a, b)
    heads = [0, 11]
    r = rng(3, 41)
    q_rows = np.unique(np.concatenate([[0, 63], r.choice(n_slots, 40, replace=False), [n_slots - 64, n_slots - 1]]))
    k_rows = np.unique(np.concatenate([[5], r.choice(n_slots, 4, replace=False), [n_slots - 60]]))
    ref = OB.block_sparse_attention_bwd_rows(*(x[:, heads] for x in host_c), mask[:, heads], 64, q_rows, k_rows,
                                             blk_len=counts)
    dq, dk, dv = (host(t[:, heads]) for t in g)
    assert_grad_close(dq[:, :, q_rows], ref[0], "cube wan dq")
    assert_grad_close(dk[:, :, k_rows], ref[1], "cube wan dk")
    assert_grad_close(dv[:, :, k_rows], ref[2], "cube wan dv")
    valid = np.arange(n_slots) % 64 < counts[np.arange(n_slots) // 64]
    for t in (dq, dk, dv):
        assert (t[:, :, ~valid] == 0).all()


def test_bwd_spatial_wan_full_shape_sampled():
    """The Wan 480p backward as the benchmark times it (12 heads, N = 32760,
    bs 128, the spatial w=1 block mask on every head, 256 key blocks with a
    ragged last block of 120 keys): dQ at sampled query rows and dK, dV at
    sampled key rows (first, middle and ragged last key block) of two heads
    against the oracle; mask and list forms bit-identical."""
    from workloads import WAN480
    w = WAN480
    announce("attn bwd spatial wan full shape")
    q, k, v = make_qkv(w)
    do = to_bf16_values(rng(w.seed, 40).standard_normal(q.shape).astype(np.float32))
    td = [dev(x) for x in (q, k, v, do)]
    m = OM.pattern_mask(w.grid, w.bs, "spatial", 1)
    mask = np.broadcast_to(m, (1, w.H, w.nb, w.nb)).copy()
    g = run(td, w.bs, mask=dev_u8(mask))
    idx, cnt = OM.mask_to_list(mask)
    gl = run(td, w.bs, idx=dev_i32(idx), cnt=dev_i32(cnt))
    for a, b in zip(g, gl):
        assert torch.equal(a, b)
    heads = [0, 11]
    r = rng(4, 41)
    q_rows = np.unique(np.concatenate([[0, 127], r.choice(w.N, 40, replace=False), [w.N - 120, w.N - 1]]))
    k_rows = np.array([3, 128 * 131 + 77, w.N - 119, w.N - 1])
    ref = OB.block_sparse_attention_bwd_rows(*(x[:, heads] for x in (q, k, v, do)), m, w.bs, q_rows, k_rows)
    dq, dk, dv = (host(t[:, heads]) for t in g)
    assert_grad_close(dq[:, :, q_rows], ref[0], "wan spatial dq")
    assert_grad_close(dk[:, :, k_rows], ref[1], "wan spatial dk")
    assert_grad_close(dv[:, :, k_rows], ref[2], "wan spatial dv")
