"""Pins of the Skiparse-2D oracle (OSP-Next page, "Method"; the reading is in
oracle/skiparse.py): hand-worked subsets and layout, a coordinate-by-coordinate
brute force of the pattern, exact pair counts, the two patterns composed over
two layers reaching every pair, dense attention at k = 1, attention to itself
alone when a subset holds one token per frame and one frame, and the padded
block-diagonal layout computing the same attention."""
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import skiparse as SK

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def golden_lines(kind):
    for line in open(os.path.join(GOLD, "skiparse_small.txt")):
        if line.startswith(kind + " "):
            yield [f.split() for f in line.split("|")]


def test_golden_subsets():
    n = 0
    for head, ids in golden_lines("subsets"):
        mode, k, T, Hh, W = head[1], *map(int, head[2:])
        got = SK.subset_ids((T, Hh, W), k, mode)
        assert got.tolist() == [int(x) for x in ids], (mode, k, T, Hh, W)
        n += 1
    assert n == 5


def test_golden_layout():
    (head, slots, blk, ns), = list(golden_lines("layout"))
    mode, k, T, Hh, W, bs = head[1], *map(int, head[2:])
    slot, blk_len, n_slots = SK.layout((T, Hh, W), k, mode, bs)
    assert slot.tolist() == [int(x) for x in slots]
    assert blk_len.tolist() == [int(x) for x in blk]
    assert n_slots == int(ns[0])


@pytest.mark.parametrize("grid,k", [((2, 6, 8), 2), ((1, 9, 10), 3), ((3, 5, 7), 2), ((2, 4, 4), 4)])
@pytest.mark.parametrize("mode", SK.MODES)
def test_pattern_equals_coordinate_brute_force(grid, k, mode):
    N = int(np.prod(grid))
    sid = SK.subset_ids(grid, k, mode)
    A = sid[:, None] == sid[None, :]
    for i in range(N):
        for j in range(N):
            assert A[i, j] == SK.pair_allowed(grid, k, mode, i, j)
    assert SK.kept_pairs(grid, k, mode) == int(A.sum())


@pytest.mark.parametrize("mode,grid,k", [("token", (3, 6, 8), 2), ("token", (2, 9, 12), 3),
                                         ("group", (3, 8, 12), 2), ("group", (1, 18, 9), 3)])
def test_exact_density_on_divisible_grids(mode, grid, k):
    """Spatial extents divisible by k (token-wise) or k^2 (group-wise): k^2 equal
    subsets, so exactly N^2 / k^2 pairs are kept."""
    N = int(np.prod(grid))
    assert (np.bincount(SK.subset_ids(grid, k, mode)) == N // (k * k)).all()
    assert SK.kept_pairs(grid, k, mode) * k * k == N * N


@pytest.mark.parametrize("grid,k", [((2, 4, 4), 2), ((1, 9, 9), 3), ((2, 5, 7), 2)])
def test_token_then_group_reaches_every_pair(grid, k):
    """Composed over two layers (token-wise, then group-wise) every query reaches
    every key when both spatial extents are at least k^2; a single pattern alone
    does not (k > 1)."""
    a_tok = SK.subset_ids(grid, k, "token")
    a_grp = SK.subset_ids(grid, k, "group")
    At = (a_tok[:, None] == a_tok[None, :]).astype(np.int64)
    Ag = (a_grp[:, None] == a_grp[None, :]).astype(np.int64)
    assert ((At @ Ag) > 0).all()
    assert not At.all() and not Ag.all()


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_k1_is_dense_attention():
    grid = (2, 3, 5)
    q, k, v = (rand((1, 2, 30, 16), s) for s in range(3))
    for mode in SK.MODES:
        o, _ = SK.attention(q, k, v, grid, 1, mode)
        ref = torch.nn.functional.scaled_dot_product_attention(*(torch.tensor(x) for x in (q, k, v))).numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_single_frame_token_subsets_of_one_token_return_v():
    """T = 1, Hh = W = k, token-wise: every subset holds one token, so each query
    attends to itself alone and o = v; group-wise on the same grid is one patch,
    i.e. dense attention."""
    k = 3
    grid = (1, k, k)
    q, kk, v = (rand((1, 1, 9, 8), s + 10) for s in range(3))
    o, lse = SK.attention(q, kk, v, grid, k, "token")
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], (q[0, 0] * kk[0, 0]).sum(1) / np.sqrt(8), atol=1e-12)
    o2, _ = SK.attention(q, kk, v, grid, k, "group")
    np.testing.assert_allclose(o2, OA.dense_attention(q, kk, v)[0], atol=1e-12)


@pytest.mark.parametrize("grid,k,bs", [((3, 6, 10), 2, 16), ((2, 9, 7), 3, 8), ((2, 8, 8), 2, 64)])
@pytest.mark.parametrize("mode", SK.MODES)
def test_padded_block_diagonal_layout_is_the_same_attention(grid, k, mode, bs):
    """Moving Q, K, V to the padded subset-major layout, attending under the
    block-diagonal mask with the blocks' valid lengths, and moving O back gives
    the natural-coordinate result; the layout is a bijection onto the valid slots
    and the round trip is the identity."""
    N = int(np.prod(grid))
    q, kk, v = (rand((1, 2, N, 8), s + 20) for s in range(3))
    slot, blk_len, n_slots = SK.layout(grid, k, mode, bs)
    assert len(set(slot.tolist())) == N and n_slots % bs == 0 and blk_len.sum() == N
    valid = np.arange(n_slots) % bs < blk_len[np.arange(n_slots) // bs]
    assert sorted(slot.tolist()) == np.nonzero(valid)[0].tolist()
    sid = SK.subset_ids(grid, k, mode)
    for c in range(k * k):                              # a subset's tokens in natural order
        assert (np.diff(slot[sid == c]) == 1).all()
    qs, ks, vs = (SK.permute(x, grid, k, mode, bs) for x in (q, kk, v))
    np.testing.assert_array_equal(SK.permute(qs, grid, k, mode, bs, inverse=True), q)
    mask = SK.block_mask(grid, k, mode, bs)
    os_, _ = OA.block_sparse_attention(qs, ks, vs, mask, bs, blk_len)
    o = SK.permute(os_, grid, k, mode, bs, inverse=True)
    ref, _ = SK.attention(q, kk, v, grid, k, mode)
    np.testing.assert_allclose(o, ref, atol=1e-12)
