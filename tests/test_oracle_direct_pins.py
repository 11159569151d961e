"""Direct pins of oracle helpers that the other pins reach only through their
callers: each against a closed form, a plain recomputation from its definition
in other terms, or torch autograd."""
import numpy as np
import pytest
import torch

from oracle import attention_bwd as OB
from oracle import fp8 as OF
from oracle import layout as OL
from oracle import semantic as OS
from oracle import skiparse as SK


@pytest.mark.parametrize("grid,k,bs", [((2, 9, 7), 3, 8), ((3, 6, 10), 2, 16), ((1, 5, 5), 1, 4), ((2, 8, 12), 4, 6)])
@pytest.mark.parametrize("mode", SK.MODES)
def test_block_subset_is_the_subset_of_every_token_in_the_block(grid, k, bs, mode):
    slot, blk_len, n_slots = SK.layout(grid, k, mode, bs)
    sub = SK.subset_ids(grid, k, mode)
    bsub = SK.block_subset(grid, k, mode, bs)
    assert bsub.size == n_slots // bs == blk_len.size
    assert np.array_equal(bsub[slot // bs], sub)          # a block holds tokens of one subset only
    assert (blk_len > 0).all()                             # and no block is empty
    assert np.all(np.diff(bsub) >= 0)                      # subsets in id order


def test_dequantise_channels_is_exact_on_the_e4m3_grid():
    """Values drawn from the e4m3 grid times a power-of-two scale per channel, with
    each channel's largest magnitude at 448 times its scale: the quantiser picks
    that scale, so codes and scales reproduce the values exactly."""
    g = np.random.default_rng(3)
    grid_vals = OF.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid_vals = grid_vals[np.isfinite(grid_vals)]
    B, H, N, D = 1, 2, 37, 8
    pick = g.integers(0, grid_vals.size, (B, H, N, D))
    base = grid_vals[pick]
    base[:, :, 0, :] = 448.0 * np.where(g.random((B, H, D)) < 0.5, -1.0, 1.0)
    scale = 2.0 ** g.integers(-6, 4, (B, H, 1, D)).astype(np.float64)
    x = (base * scale).astype(np.float32)
    codes, sc = OF.quantise_channels(x)
    assert np.array_equal(sc, scale[:, :, 0, :].astype(np.float32))
    assert np.array_equal(OF.dequantise_channels(codes, sc), x.astype(np.float64))


def test_dequantise_channels_error_within_half_a_step():
    g = np.random.default_rng(4)
    x = g.standard_normal((2, 3, 50, 16)).astype(np.float32)
    codes, sc = OF.quantise_channels(x)
    y = OF.dequantise_channels(codes, sc)
    # e4m3 has 3 mantissa bits: half a step is 2^-4 of the value for normals, and
    # 2^-10 of the scale unit (448 ↔ amax) in the subnormal range
    s = sc[:, :, None, :].astype(np.float64)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(y - x) <= bound).all()


def test_kmeans_update_closed_form():
    x = np.array([[0.0, 0.0], [2.0, 2.0], [1.0, -1.0], [3.0, 5.0], [-4.0, 2.0], [7.0, 7.0]])
    labels = np.array([0, 0, 1, 1, 1, 3])
    cent = np.array([[9.0, 9.0], [9.0, 9.0], [-1.5, 2.5], [9.0, 9.0]])
    out, counts = OS.update(x, labels, cent)
    assert counts.tolist() == [2, 3, 0, 1]
    assert np.array_equal(out[0], [1.0, 1.0])
    assert np.array_equal(out[1], [0.0, 2.0])
    assert np.array_equal(out[2], [-1.5, 2.5])            # empty cluster keeps its centroid
    assert np.array_equal(out[3], [7.0, 7.0])


def test_kmeans_heads_is_kmeans_of_every_head():
    x = np.random.default_rng(5).standard_normal((2, 3, 40, 4))
    cent, labels, counts = OS.kmeans_heads(x, 5, 3)
    for b in range(2):
        for h in range(3):
            c1, l1, n1 = OS.kmeans(x[b, h], 5, 3)
            assert np.array_equal(cent[b, h], c1) and np.array_equal(labels[b, h], l1)
            assert np.array_equal(counts[b, h], n1)


def test_masked_attention_bwd_through_a_layout_map_matches_autograd():
    """Query and key blocks read through the frame-major map (blocks are runs of
    the map, not of natural order) and a ragged valid set: the general form of the
    gradients against torch autograd of the token-level masked softmax (fp64)."""
    T, Hh, W, bs = 3, 4, 5, 8
    N = T * Hh * W
    g = np.random.default_rng(6)
    B, H, D = 1, 2, 8
    q, k, v, do = (g.standard_normal((B, H, N, D)) for _ in range(4))
    blk = OL.frame_major_map(T, Hh, W) // bs
    nb = int(blk.max()) + 1
    mask = (g.random((H, nb, nb)) < 0.45).astype(np.uint8)
    mask[:, 0, :] = 0                                       # a block row that keeps nothing
    valid = np.ones(N, bool)
    valid[g.choice(N, 7, replace=False)] = False
    scale = 0.3
    dq, dk, dv = OB.masked_attention_bwd(q, k, v, do, mask, blk, blk, scale, q_valid=valid, k_valid=valid)

    tm = mask[:, blk][:, :, blk].astype(bool) & valid[None, None, :] & valid[None, :, None]
    qt, kt, vt = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    s = scale * (qt @ kt.transpose(-1, -2))
    m = torch.tensor(tm[None])
    s = s.masked_fill(~m, float("-inf"))
    has = m.any(-1, keepdim=True)
    p = torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=-1) * has
    (p @ vt * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-10)
