"""The Python binding checks the full shape, dtype and layout of every tensor
argument before it calls the library: the kernels index each buffer from the
sizes alone, so a mis-shaped mask, list, length table, output or workspace would
otherwise be read or written past its end on the GPU.

These run on the CPU with CPU tensors. Shape checks come first, so a wrong shape
raises its own error; a call whose every shape is right gets as far as the
device check ("must be device tensors") and never reaches a launch."""
import os

import pytest
import torch

import block_sparse_attention_vsa_amd as V

pytestmark = pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvsa.so not built")

BF, F32, U8, I32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32
DEVICE_MSG = "device tensors"


def z(shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def shape_error(fn, *args, match=None, **kw):
    with pytest.raises((ValueError, TypeError), match=match) as e:
        fn(*args, **kw)
    assert DEVICE_MSG not in str(e.value), f"reached the device check: {e.value}"


def reaches_device_check(fn, *args, **kw):
    with pytest.raises(ValueError, match=DEVICE_MSG):
        fn(*args, **kw)


# ---- block-sparse attention (natural order): B=1, H=2, N=300, bs=64 -> nb=5 ----
B, H, N, D, BS, NB = 1, 2, 300, 128, 64, 5


def qkv(n=N):
    return z((B, H, n, D)), z((B, H, n, D)), z((B, H, n, D))


def test_attention_accepts_right_shapes():
    q, k, v = qkv()
    reaches_device_check(V.vsa_block_sparse_attn_fwd, q, k, v, BS, mask=z((B, H, NB, NB), U8))
    reaches_device_check(V.vsa_block_sparse_attn_fwd, q, k, v, BS, kv_idx=z((B, H, NB, 3), I32),
                         kv_cnt=z((B, H, NB), I32), blk_len=z((NB,), I32), return_lse=True)


@pytest.mark.parametrize("what", ["mask_2d", "mask_per_head_only", "mask_short", "mask_dtype", "idx_rows",
                                  "cnt_shape", "cnt_missing", "both_forms", "no_form", "blk_len", "out", "lse",
                                  "k_shape", "v_dtype", "noncontig"])
def test_attention_rejects_bad_shapes(what):
    q, k, v = qkv()
    kw = dict(mask=z((B, H, NB, NB), U8))
    if what == "mask_2d":
        kw = dict(mask=z((NB, NB), U8))              # a pattern mask passed as-is with H > 1
    elif what == "mask_per_head_only":
        kw = dict(mask=z((H, NB, NB), U8))
    elif what == "mask_short":
        kw = dict(mask=z((B, H, NB - 1, NB), U8))
    elif what == "mask_dtype":
        kw = dict(mask=z((B, H, NB, NB), I32))
    elif what == "idx_rows":
        kw = dict(kv_idx=z((B, H, NB - 1, 3), I32), kv_cnt=z((B, H, NB), I32))
    elif what == "cnt_shape":
        kw = dict(kv_idx=z((B, H, NB, 3), I32), kv_cnt=z((B, 1, NB), I32))
    elif what == "cnt_missing":
        kw = dict(kv_idx=z((B, H, NB, 3), I32))
    elif what == "both_forms":
        kw = dict(mask=z((B, H, NB, NB), U8), kv_idx=z((B, H, NB, 3), I32), kv_cnt=z((B, H, NB), I32))
    elif what == "no_form":
        kw = {}
    elif what == "blk_len":
        kw["blk_len"] = z((NB - 1,), I32)
    elif what == "out":
        kw["out"] = z((B, H, N - 1, D))
    elif what == "lse":
        kw["lse"] = z((B, H, N), BF)
    elif what == "k_shape":
        k = z((B, H, N + 1, D))
    elif what == "v_dtype":
        v = z((B, H, N, D), F32)
    elif what == "noncontig":
        q = z((B, H, D, N)).transpose(2, 3)
    shape_error(V.vsa_block_sparse_attn_fwd, q, k, v, BS, **kw)


GRID = (3, 10, 10)   # N = 300


def test_permuted_and_chosen_check_masks_and_choice():
    q, k, v = qkv()
    reaches_device_check(V.vsa_block_sparse_attn_fwd_permuted, q, k, v, GRID, BS, head_fm=[1, 0],
                         mask=z((B, H, NB, NB), U8))
    shape_error(V.vsa_block_sparse_attn_fwd_permuted, q, k, v, GRID, BS, head_fm=[1, 0], mask=z((NB, NB), U8))
    shape_error(V.vsa_block_sparse_attn_fwd_permuted, q, k, v, GRID, BS, head_fm=[1], mask=z((B, H, NB, NB), U8))
    shape_error(V.vsa_block_sparse_attn_fwd_permuted, q, k, v, (3, 10, 11), BS, mask=z((B, H, NB, NB), U8))
    cand = z((2, NB, NB), U8)
    reaches_device_check(V.vsa_block_sparse_attn_fwd_chosen, q, k, v, GRID, BS, cand, [0, 1], z((B, H), I32))
    shape_error(V.vsa_block_sparse_attn_fwd_chosen, q, k, v, GRID, BS, z((2, NB, NB - 1), U8), [0, 1],
                z((B, H), I32))
    shape_error(V.vsa_block_sparse_attn_fwd_chosen, q, k, v, GRID, BS, cand, [0], z((B, H), I32))
    shape_error(V.vsa_block_sparse_attn_fwd_chosen, q, k, v, GRID, BS, cand, [0, 1], z((B, H + 1), I32))
    shape_error(V.vsa_block_sparse_attn_fwd_chosen, q, k, v, GRID, BS, cand, [0, 1], z((B, H), I32),
                blk_len=z((NB + 1,), I32))


def test_backward_checks_every_buffer():
    q, k, v = qkv()
    o, do, lse = z((B, H, N, D)), z((B, H, N, D)), z((B, H, N), F32)
    m = z((B, H, NB, NB), U8)
    reaches_device_check(V.vsa_block_sparse_attn_bwd, q, k, v, o, lse, do, BS, mask=m)
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, z((B, H, N, 64)), lse, do, BS, mask=m)
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, o, z((B, H, N - 1), F32), do, BS, mask=m)
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, o, lse, do, BS, mask=z((B, 1, NB, NB), U8))
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, o, lse, do, BS, mask=m, dk=z((B, H, N, D), F32))
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, o, lse, do, BS, mask=m, workspace=z((10,), U8))
    shape_error(V.vsa_block_sparse_attn_bwd, q, k, v, o, lse, do, BS, mask=m, workspace=z((1 << 20,), F32))


def test_small_calls_check_their_buffers():
    nb8 = 4   # grid (4, 8, 8), bs 64
    reaches_device_check(V.vsa_pattern_mask, (4, 8, 8), 64, V.VSA_PATTERN_SPATIAL, 1, out=z((nb8, nb8), U8))
    shape_error(V.vsa_pattern_mask, (4, 8, 8), 64, V.VSA_PATTERN_SPATIAL, 1, out=z((nb8, nb8 - 1), U8))
    shape_error(V.vsa_pattern_mask, (4, 8, 8), 64, V.VSA_PATTERN_SPATIAL, 1, out=z((nb8 * nb8,), U8))
    shape_error(V.vsa_cube_block_len, (4, 8, 8), out=z((3,), I32))
    # permutation: row counts of src / out for each kind and direction
    x = z((1, 2, 256, 128))
    reaches_device_check(V.vsa_permute, x, (4, 8, 8), V.VSA_PERM_FRAME_MAJOR)
    shape_error(V.vsa_permute, z((1, 2, 255, 128)), (4, 8, 8), V.VSA_PERM_FRAME_MAJOR)
    shape_error(V.vsa_permute, x, (4, 8, 8), V.VSA_PERM_FRAME_MAJOR, out=z((1, 2, 255, 128)))
    shape_error(V.vsa_permute, x, (4, 8, 8), V.VSA_PERM_FRAME_MAJOR, head_sel=[1])
    shape_error(V.vsa_permute, x, (5, 6, 9), V.VSA_PERM_CUBE4)             # N = 270 != 256
    slots = V.vsa_cube_dims((5, 6, 9))[1]
    shape_error(V.vsa_permute, z((1, 2, 270, 128)), (5, 6, 9), V.VSA_PERM_CUBE4, inverse=True)
    reaches_device_check(V.vsa_permute, z((1, 2, slots, 128)), (5, 6, 9), V.VSA_PERM_CUBE4, inverse=True)
    # pooled scores and selection
    q = z((1, 2, 300, 128))
    reaches_device_check(V.vsa_block_scores, q, q, 64)
    shape_error(V.vsa_block_scores, q, q, 64, blk_len=z((4,), I32))
    shape_error(V.vsa_block_scores, q, q, 64, out=(z((1, 2, 5, 5), F32), z((1, 2, 5, 64), F32),
                                                   z((1, 2, 5, 128), F32)))
    s = z((1, 2, 5, 5), F32)
    reaches_device_check(V.vsa_select_topk, s, 3, 0.9, forced=z((5, 5), U8))
    shape_error(V.vsa_select_topk, s, 3, 0.9, forced=z((1, 2, 5, 5), U8))
    shape_error(V.vsa_select_topk, s, 3, out=(z((1, 2, 5, 2), I32), z((1, 2, 5), I32)))
    # mask -> list
    reaches_device_check(V.vsa_mask_to_list, z((1, 2, 5, 5), U8))
    shape_error(V.vsa_mask_to_list, z((5, 5), U8))
    shape_error(V.vsa_mask_to_list, z((2, 5, 5), U8), head_mask_idx=[0, 2])
    shape_error(V.vsa_mask_to_list, z((1, 2, 5, 5), U8), out=(z((1, 2, 5, 4), I32), z((1, 2, 5), I32)))


def test_profiler_checks_masks_and_outputs():
    q, k, v = qkv()
    rows, cand = z((8,), I32), z((2, NB, NB), U8)
    reaches_device_check(V.vsa_profile_heads, q, k, v, GRID, BS, rows, cand, [0, 1])
    shape_error(V.vsa_profile_heads, q, k, v, GRID, BS, rows, z((2, NB + 1, NB + 1), U8), [0, 1])
    shape_error(V.vsa_profile_heads, q, k, v, GRID, BS, rows, cand, [0])
    shape_error(V.vsa_profile_heads, q, k, v, GRID, BS, z((8, 1), I32), cand, [0, 1])
    shape_error(V.vsa_profile_heads, q, k, v, GRID, BS, rows, cand, [0, 1],
                out=(z((B, H, 3), F32), z((B, H), I32)))
    shape_error(V.vsa_profile_heads, q, k, v, GRID, BS, rows, cand, [0, 1], workspace=z((16,), U8))


def test_semantic_calls_check_their_buffers():
    x = z((1, 2, 300, 128))
    reaches_device_check(V.vsa_kmeans, x, 7, 2)
    shape_error(V.vsa_kmeans, x, 7, 2, out=(z((1, 2, 7, 128), F32), z((1, 2, 300), I32), z((1, 2, 8), I32)))
    lab = z((1, 2, 300), I32)
    reaches_device_check(V.vsa_cluster_order, lab, 7)
    shape_error(V.vsa_cluster_order, lab, 7, out=(z((1, 2, 300), I32), z((1, 2, 7), I32)))
    reaches_device_check(V.vsa_gather_rows, x, lab)
    shape_error(V.vsa_gather_rows, x, z((1, 2, 299), I32))
    cq, ck, kn = z((1, 2, 7, 128), F32), z((1, 2, 9, 128), F32), z((1, 2, 9), I32)
    reaches_device_check(V.vsa_cluster_scores, cq, ck, kn)
    shape_error(V.vsa_cluster_scores, cq, z((1, 2, 9, 64), F32), kn)
    shape_error(V.vsa_cluster_scores, cq, ck, z((1, 2, 8), I32))
    qo, ko = z((1, 2, 8), I32), z((1, 2, 10), I32)
    reaches_device_check(V.vsa_varlen_sparse_attn_fwd, x, x, x, qo, ko, mask=z((1, 2, 7, 9), U8))
    shape_error(V.vsa_varlen_sparse_attn_fwd, x, x, x, qo, ko, mask=z((1, 2, 9, 7), U8))
    shape_error(V.vsa_varlen_sparse_attn_fwd, x, x, x, qo, ko, kv_idx=z((1, 2, 7, 3), I32), kv_cnt=z((1, 2, 9), I32))
    shape_error(V.vsa_varlen_sparse_attn_fwd, x, x, x, z((1, 1, 8), I32), ko, mask=z((1, 2, 7, 9), U8))


def test_fp8_calls_check_their_buffers():
    x = z((1, 2, 300, 128))
    reaches_device_check(V.vsa_fp8_quantize, x, V.VSA_FP8_ROWS)
    shape_error(V.vsa_fp8_quantize, x, V.VSA_FP8_VT, out=z((1, 2, 5, 128, 32), U8))
    shape_error(V.vsa_fp8_quantize, x, V.VSA_FP8_ROWS, scales=z((1, 2, 4), F32))
    q8, vt8 = z((1, 2, 300, 128), U8), z((1, 2, 5, 128, 64), U8)
    qs, vs = z((1, 2, 5), F32), z((1, 2, 128), F32)
    m = z((1, 2, 3, 3), U8)
    reaches_device_check(V.vsa_block_sparse_attn_fwd_fp8, q8, q8, vt8, qs, qs, vs, 128, mask=m)
    shape_error(V.vsa_block_sparse_attn_fwd_fp8, q8, q8, z((1, 2, 4, 128, 64), U8), qs, qs, vs, 128, mask=m)
    shape_error(V.vsa_block_sparse_attn_fwd_fp8, q8, q8, vt8, z((1, 2, 4), F32), qs, vs, 128, mask=m)
    shape_error(V.vsa_block_sparse_attn_fwd_fp8, q8, q8, vt8, qs, qs, vs, 128, mask=z((1, 2, 3, 2), U8))


def test_skiparse_calls_check_their_buffers():
    grid = (2, 9, 7)                       # N = 126
    n_slots, nb = V.vsa_skiparse_dims(grid, V.VSA_SKIPARSE_GROUP, 3, 64)
    x = z((1, 2, 126, 128))
    reaches_device_check(V.vsa_skiparse_permute, x, grid, V.VSA_SKIPARSE_GROUP, 3, 64)
    shape_error(V.vsa_skiparse_permute, z((1, 2, 125, 128)), grid, V.VSA_SKIPARSE_GROUP, 3, 64)
    shape_error(V.vsa_skiparse_permute, x, grid, V.VSA_SKIPARSE_GROUP, 3, 64, out=z((1, 2, n_slots - 1, 128)))
    shape_error(V.vsa_skiparse_permute, x, grid, V.VSA_SKIPARSE_GROUP, 3, 64, inverse=True)
    reaches_device_check(V.vsa_skiparse_permute, z((1, 2, n_slots, 128)), grid, V.VSA_SKIPARSE_GROUP, 3, 64,
                         inverse=True)
    shape_error(V.vsa_skiparse_block_len, grid, V.VSA_SKIPARSE_GROUP, 3, 64, out=z((nb + 1,), I32))
    shape_error(V.vsa_skiparse_mask, grid, V.VSA_SKIPARSE_GROUP, 3, 64, out=z((nb, nb + 1), U8))
    with pytest.raises(V.VsaError):
        V.vsa_skiparse_dims(grid, 2, 3, 64)
    with pytest.raises(V.VsaError):
        V.vsa_skiparse_dims(grid, V.VSA_SKIPARSE_TOKEN, 9, 64)
