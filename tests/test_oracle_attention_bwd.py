"""Pins of the oracle's block-sparse attention gradients against results fixed
independently of it: torch autograd of a dense softmax attention with a token
mask (fp64, CPU), torch's scaled_dot_product_attention autograd for the all-ones
mask, central finite differences, and the softmax-Jacobian invariants."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import attention_bwd as OB


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def token_mask(mask, bs, N, valid):
    """[H, N, N] bool: query i may see key j."""
    pos = np.arange(N)
    tm = mask[:, pos // bs][:, :, pos // bs].astype(bool)
    return tm & valid[None, :, None] & valid[None, None, :]


def autograd_ref(q, k, v, do, tm, scale):
    """Plain masked softmax attention differentiated by torch autograd in fp64.
    Rows with no visible key are dropped (their output is defined as 0)."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (qt @ kt.transpose(-1, -2))
    m = torch.tensor(tm[None])
    s = s.masked_fill(~m, float("-inf"))
    has = m.any(-1, keepdim=True)
    s = torch.where(has, s, torch.zeros_like(s))
    p = torch.softmax(s, dim=-1) * has
    o = p @ vt
    (o * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("N,bs,H,D,density,seed", [(40, 8, 2, 16, 0.4, 1), (37, 8, 3, 8, 0.3, 2), (64, 16, 1, 32, 0.6, 3)])
def test_bwd_matches_autograd_of_masked_softmax(N, bs, H, D, density, seed):
    nb = -(-N // bs)
    q, k, v, do = (rand((1, H, N, D), seed * 10 + i) for i in range(4))
    mask = (np.random.default_rng(seed).random((H, nb, nb)) < density).astype(np.uint8)
    mask[0, 0, :] = 0                                     # a query block with nothing kept
    scale = 1.0 / np.sqrt(D)
    dq, dk, dv = OB.block_sparse_attention_bwd(q, k, v, do, mask[None], bs)
    rq, rk, rv = autograd_ref(q[0], k[0], v[0], do[0], token_mask(mask, bs, N, np.ones(N, bool)), scale)
    np.testing.assert_allclose(dq[0], rq, atol=1e-11)
    np.testing.assert_allclose(dk[0], rk, atol=1e-11)
    np.testing.assert_allclose(dv[0], rv, atol=1e-11)
    assert (dq[0, 0, :bs] == 0).all()                     # the empty query block gets nothing


def test_bwd_all_ones_equals_sdpa_autograd():
    H, N, D = 2, 48, 16
    q, k, v, do = (rand((1, H, N, D), 40 + i) for i in range(4))
    dq, dk, dv = OB.block_sparse_attention_bwd(q, k, v, do, np.ones((1, H, 3, 3), np.uint8), 16)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)


def test_bwd_finite_differences():
    """L = sum(o * do); every gradient entry against a central difference of the
    oracle's own forward (a different code path: no Jacobian written out)."""
    H, N, D, bs = 1, 6, 4, 2
    q, k, v, do = (rand((1, H, N, D), 70 + i) for i in range(4))
    mask = np.array([[[1, 0, 1], [1, 1, 0], [0, 1, 1]]], np.uint8)[None]
    dq, dk, dv = OB.block_sparse_attention_bwd(q, k, v, do, mask, bs)
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = OA.block_sparse_attention(qq, kk, vv, mask, bs)
        return float((o * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, err_msg=name)


def test_bwd_softmax_invariants_and_padding():
    """Per head: sum over keys of dk is 0 (each row of ds sums to 0); sum over keys
    of dv equals the sum of do over rows that keep any key; invalid positions
    (blk_len) get and give nothing."""
    H, N, D, bs = 2, 32, 8, 8
    q, k, v, do = (rand((1, H, N, D), 90 + i) for i in range(4))
    mask = (np.random.default_rng(9).random((1, H, 4, 4)) < 0.5).astype(np.uint8)
    mask[..., np.arange(4), np.arange(4)] = 1
    blk_len = np.array([8, 5, 8, 3])
    dq, dk, dv = OB.block_sparse_attention_bwd(q, k, v, do, mask, bs, blk_len=blk_len)
    valid = OA.block_valid(N, bs, blk_len)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    rows_with_keys = valid.copy()                          # every valid row keeps its own (diagonal) block
    np.testing.assert_allclose(dv.sum(axis=2), do[:, :, rows_with_keys].sum(axis=2), atol=1e-11)
    for g in (dq, dk, dv):
        assert (g[:, :, ~valid] == 0).all()
    # padding contents do not matter
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for t in (q2, k2, v2, do2):
        t[:, :, ~valid] = 1e3
    g2 = OB.block_sparse_attention_bwd(q2, k2, v2, do2, mask, bs, blk_len=blk_len)
    for a, b_ in zip((dq, dk, dv), g2):
        np.testing.assert_allclose(a[:, :, valid], b_[:, :, valid], atol=1e-11)


def test_bwd_flop_count():
    mask = np.ones((1, 1, 2, 2), np.uint8)
    assert OB.kept_flops_bwd(mask, 4, 8, 16) == 10 * 16 * 64


def test_bwd_rows_matches_autograd_at_selected_positions():
    """The sampled form (used at full video sizes) against torch autograd of the
    dense masked softmax, with padding (blk_len) and a key block nobody keeps."""
    H, N, D, bs = 2, 45, 8, 8
    nb = -(-N // bs)
    q, k, v, do = (rand((1, H, N, D), 110 + i) for i in range(4))
    mask = (np.random.default_rng(11).random((H, nb, nb)) < 0.45).astype(np.uint8)
    mask[:, :, 3] = 0
    blk_len = np.array([8, 6, 8, 8, 2, 5])
    valid = OA.block_valid(N, bs, blk_len)
    q_rows = np.array([0, 7, 9, 14, 20, 33, 44])
    k_rows = np.array([1, 8, 13, 25, 30, 34, 40, 44])
    dq, dk, dv = OB.block_sparse_attention_bwd_rows(q, k, v, do, mask[None], bs, q_rows, k_rows, blk_len=blk_len)
    rq, rk, rv = autograd_ref(q[0], k[0], v[0], do[0], token_mask(mask, bs, N, valid), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(dq[0], rq[:, q_rows], atol=1e-11)
    np.testing.assert_allclose(dk[0], rk[:, k_rows], atol=1e-11)
    np.testing.assert_allclose(dv[0], rv[:, k_rows], atol=1e-11)
    assert (dk[0][:, [3]] == 0).all() and (dv[0][:, [3]] == 0).all()      # key 25 sits in block 3
