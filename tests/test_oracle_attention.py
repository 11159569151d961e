"""Pins for oracle.attention: a library special case, closed forms, invariants and
brute force on tiny inputs. CPU only."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as A


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N,bs,D", [(256, 64, 64), (200, 64, 32), (130, 128, 16)])
def test_all_ones_mask_equals_torch_sdpa(N, bs, D):
    """Library special case: with every block kept the result is dense attention,
    which torch's scaled_dot_product_attention computes in fp64 on the CPU."""
    q, k, v = rnd((2, 3, N, D), 1), rnd((2, 3, N, D), 2), rnd((2, 3, N, D), 3)
    nb = -(-N // bs)
    o, lse = A.block_sparse_attention(q, k, v, np.ones((nb, nb), np.uint8), bs)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.abs(o - ref).max() <= 1e-12
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(D)
    assert np.abs(lse - logsumexp(s, axis=-1)).max() <= 1e-12


def test_token_mask_special_case_matches_sdpa_boolean_mask():
    """bs = 1 turns the block mask into a token mask; torch SDPA with a boolean
    attn_mask is the library routine for that."""
    N, D = 40, 8
    q, k, v = rnd((1, 2, N, D), 4), rnd((1, 2, N, D), 5), rnd((1, 2, N, D), 6)
    m = (np.random.default_rng(7).random((2, N, N)) < 0.3).astype(np.uint8)
    m[:, np.arange(N), np.arange(N)] = 1
    o, _ = A.block_sparse_attention(q, k, v, m, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(m.astype(bool))[None]).numpy()
    assert np.abs(o - ref).max() <= 1e-12


def brute_force(q, k, v, mask, bs, scale):
    """Definition written out with scalar loops (tiny inputs only)."""
    B, H, N, D = q.shape
    o = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if mask[h][i // bs][j // bs]]
                if not keys:
                    continue
                s = {j: scale * sum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in keys}
                m = max(s.values())
                z = sum(math.exp(s[j] - m) for j in keys)
                for d in range(D):
                    o[b, h, i, d] = sum(math.exp(s[j] - m) / z * v[b, h, j, d] for j in keys)
                lse[b, h, i] = m + math.log(z)
    return o, lse


def test_brute_force_tiny_with_ragged_tail_and_empty_row():
    N, D, bs = 14, 3, 4               # 4 blocks, last one holds 2 tokens
    q, k, v = rnd((1, 2, N, D), 8), rnd((1, 2, N, D), 9), rnd((1, 2, N, D), 10)
    mask = np.array([[[1, 0, 1, 0], [0, 1, 0, 1], [0, 0, 0, 0], [1, 1, 1, 1]],
                     [[0, 0, 0, 1], [1, 1, 0, 0], [1, 0, 1, 0], [0, 1, 0, 1]]], np.uint8)
    o, lse = A.block_sparse_attention(q, k, v, mask, bs, scale=0.7)
    ob, lb = brute_force(q, k, v, mask, bs, 0.7)
    assert np.abs(o - ob).max() <= 1e-12
    fin = np.isfinite(lb)
    assert (fin == np.isfinite(lse)).all()
    assert np.abs(lse[fin] - lb[fin]).max() <= 1e-12
    # the empty row of head 0 (query block 2) is zero with lse = -inf
    assert (o[0, 0, 8:12] == 0).all() and np.isneginf(lse[0, 0, 8:12]).all()


def test_probability_rows_sum_to_one_and_vanish_off_mask():
    N, D, bs = 96, 16, 32
    q, k, v = rnd((1, 1, N, D), 11), rnd((1, 1, N, D), 12), rnd((1, 1, N, D), 13)
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8)
    _, _, p = A.block_sparse_attention(q, k, v, mask, bs, return_probs=True)
    assert np.abs(p.sum(-1) - 1).max() <= 1e-12
    blk = np.arange(N) // bs
    off = mask[blk[:, None], blk[None, :]] == 0
    assert (p[0, 0][off] == 0).all()


def test_constant_v_gives_that_constant():
    N, D, bs = 128, 8, 32
    q, k = rnd((1, 2, N, D), 14), rnd((1, 2, N, D), 15)
    v = np.broadcast_to(np.arange(D, dtype=np.float64), (1, 2, N, D)).copy()
    mask = (np.random.default_rng(16).random((2, 4, 4)) < 0.5).astype(np.uint8)
    mask[:, np.arange(4), np.arange(4)] = 1
    o, _ = A.block_sparse_attention(q, k, v, mask, bs)
    assert np.abs(o - v).max() <= 1e-12


def test_zero_queries_average_the_kept_values():
    N, D, bs = 100, 4, 32            # ragged last block of 4 tokens
    k, v = rnd((1, 1, N, D), 17), rnd((1, 1, N, D), 18)
    q = np.zeros((1, 1, N, D))
    mask = np.array([[1, 0, 0, 1], [0, 1, 1, 0], [1, 1, 1, 1], [0, 0, 0, 1]], np.uint8)
    o, lse = A.block_sparse_attention(q, k, v, mask, bs)
    for qb in range(4):
        keys = np.concatenate([np.arange(kb * bs, min(kb * bs + bs, N)) for kb in np.nonzero(mask[qb])[0]])
        rows = np.arange(qb * bs, min(qb * bs + bs, N))
        assert np.abs(o[0, 0, rows] - v[0, 0, keys].mean(0)).max() <= 1e-12
        assert np.abs(lse[0, 0, rows] - math.log(keys.size)).max() <= 1e-12


def test_single_kept_key_copies_its_value():
    N, D = 12, 5
    q, k, v = rnd((1, 1, N, D), 19), rnd((1, 1, N, D), 20), rnd((1, 1, N, D), 21)
    mask = np.zeros((N, N), np.uint8)
    target = np.random.default_rng(22).integers(0, N, N)
    mask[np.arange(N), target] = 1
    o, _ = A.block_sparse_attention(q, k, v, mask, 1)
    assert np.abs(o[0, 0] - v[0, 0, target]).max() <= 1e-12


def test_value_scaling_is_linear():
    N, D, bs = 64, 8, 16
    q, k, v = rnd((1, 1, N, D), 23), rnd((1, 1, N, D), 24), rnd((1, 1, N, D), 25)
    mask = (np.random.default_rng(26).random((4, 4)) < 0.6).astype(np.uint8)
    mask[np.arange(4), np.arange(4)] = 1
    o1, _ = A.block_sparse_attention(q, k, v, mask, bs)
    o2, _ = A.block_sparse_attention(q, k, 3.5 * v, mask, bs)
    assert np.abs(o2 - 3.5 * o1).max() <= 1e-12


def test_blk_len_equals_attention_over_the_compacted_valid_tokens():
    """Cube-style padding: a block's invalid slots are absent keys and zero outputs."""
    bs, D = 8, 6
    blk_len = np.array([8, 3, 5, 1])
    N = bs * blk_len.size
    q, k, v = rnd((1, 2, N, D), 27), rnd((1, 2, N, D), 28), rnd((1, 2, N, D), 29)
    mask = np.array([[1, 1, 0, 1], [0, 1, 1, 0], [1, 0, 1, 1], [1, 1, 1, 1]], np.uint8)
    o, lse = A.block_sparse_attention(q, k, v, mask, bs, blk_len)
    valid = np.concatenate([np.arange(b * bs, b * bs + n) for b, n in enumerate(blk_len)])
    blk = valid // bs
    oc, lc = A.masked_attention(q[:, :, valid], k[:, :, valid], v[:, :, valid], mask, blk, blk)
    assert np.abs(o[:, :, valid] - oc).max() <= 1e-12
    assert np.abs(lse[:, :, valid] - lc).max() <= 1e-12
    pad = np.setdiff1d(np.arange(N), valid)
    assert (o[:, :, pad] == 0).all() and np.isneginf(lse[:, :, pad]).all()


def test_rows_subset_matches_full():
    N, D, bs = 200, 8, 64
    q, k, v = rnd((1, 2, N, D), 30), rnd((1, 2, N, D), 31), rnd((1, 2, N, D), 32)
    mask = np.array([[1, 0, 1, 0], [1, 1, 0, 0], [0, 0, 1, 1], [1, 0, 0, 1]], np.uint8)
    o, lse = A.block_sparse_attention(q, k, v, mask, bs)
    rows = np.array([0, 5, 63, 64, 190, 199])
    o2, l2 = A.block_sparse_attention(q, k, v, mask, bs, rows=rows)
    # same arithmetic, different GEMM shapes: equal up to summation order
    assert np.abs(o[:, :, rows] - o2).max() <= 1e-14 and np.abs(lse[:, :, rows] - l2).max() <= 1e-14


def test_kept_flops_counts_valid_pairs():
    mask = np.array([[1, 0], [1, 1]], np.uint8)
    # N = 100, bs = 64: blocks of 64 and 36 tokens
    f = A.kept_flops(mask, 64, 100, 8)
    assert f == 4 * 8 * (64 * 64 + 36 * 64 + 36 * 36)
