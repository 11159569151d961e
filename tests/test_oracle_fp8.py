"""Pins of the FP8 oracle: the e4m3 codec against torch's float8_e4m3fn cast (an
independent implementation of the OCP format), hand-worked codes, the
quantiser's error bound and exact cases, the transposed-V tile layout, and
attention on inputs that quantise exactly."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import fp8 as OF


def torch_codes(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = OF.e4m3_decode(codes)
    assert ((np.isnan(ref) & np.isnan(got)) | (ref == got)).all()


def test_encode_matches_torch_on_random_ties_subnormals_and_range_edges():
    g = np.random.default_rng(0)
    grid = OF.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2                      # exact ties
    x = np.concatenate([g.standard_normal(20000) * 10.0, g.standard_normal(5000) * 1e-3, mids, -mids, grid, -grid,
                        [0.0, -0.0, 463.9, 464.0, 464.1, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    x = x.astype(np.float32)
    assert (OF.e4m3_encode(x) == torch_codes(x)).all()


def test_hand_worked_codes():
    # 1.0 = 0 0111 000; 448 = 0 1111 110; 2^-9 = smallest subnormal 0 0000 001;
    # 1.0625 is halfway between 1.0 and 1.125 and goes to the even mantissa (1.0)
    assert OF.e4m3_encode([1.0, 448.0, 2.0 ** -9, 1.0625, -2.0]).tolist() == [0x38, 0x7E, 0x01, 0x38, 0xC0]


def test_quantise_rows_error_bound_and_amax_code():
    g = np.random.default_rng(1)
    x = OF.e4m3_decode(np.zeros(1)) + g.standard_normal((1, 2, 200, 128)) * np.exp(g.standard_normal((1, 2, 200, 1)))
    codes, s = OF.quantise_rows(x)
    assert s.shape == (1, 2, 4)
    deq = OF.dequantise_rows(codes, s)
    # within half a step: 2^-4 relative in the normal range, 2^-10 s below it
    y = np.abs(x.astype(np.float32))
    bound = np.maximum(y * 2.0 ** -4, np.repeat(s, 64, axis=2)[:, :, :200, None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - x.astype(np.float32)) <= bound).all()
    # the largest element of every block becomes +-448 exactly
    for b in range(4):
        blk = np.abs(x[0, 0, 64 * b:64 * b + 64].astype(np.float32))
        i = np.unravel_index(blk.argmax(), blk.shape)
        assert OF.e4m3_decode(codes[0, 0, 64 * b + i[0], i[1]]) in (448.0, -448.0)


def test_zero_block_and_channel_scales():
    x = np.zeros((1, 1, 70, 128))
    x[0, 0, 64:, 3] = 2.0
    codes, s = OF.quantise_rows(x)
    assert s[0, 0, 0] == 0 and (codes[0, 0, :64] == 0).all()
    assert s[0, 0, 1] == np.float32(2.0) / np.float32(448.0)
    vc, vs = OF.quantise_channels(x)
    assert vs[0, 0, 3] == np.float32(2.0) / np.float32(448.0) and vs[0, 0, 0] == 0
    assert (OF.e4m3_decode(vc[0, 0, 64:, 3]) == 448.0).all()


def test_vt_tile_layout():
    """Column of key k = 32 st + 8 g + 4 h + e is 32 h + 16 st + 4 g + e: a bijection
    of the 64 keys; every key lands where the 32x32 accumulator's element
    x = 4 g + e of half-wave h, sub-tile st lives (byte 16 st + x of that half)."""
    cols = OF.vt_column(np.arange(64))
    assert sorted(cols.tolist()) == list(range(64))
    for st in range(2):
        for h in range(2):
            for x in range(16):
                key = 32 * st + 8 * (x >> 2) + 4 * h + (x & 3)       # accumulator row of element x
                assert cols[key] == 32 * h + 16 * st + x
    c = np.random.default_rng(2).integers(0, 255, (1, 2, 100, 128)).astype(np.uint8)
    t = OF.vt_tiles(c)
    assert t.shape == (1, 2, 2, 128, 64)
    for n in (0, 5, 63, 64, 99):
        assert (t[:, :, n // 64, :, cols[n % 64]] == c[:, :, n, :]).all()
    assert (t[:, :, 1][..., cols[36:]] == 0).all()               # keys past N


def test_attention_on_exactly_quantisable_inputs_equals_bf16_oracle():
    """Values on the e4m3 grid with every block's amax 448 (and every channel's for
    V): quantisation is exact, so the FP8 oracle equals plain attention."""
    g = np.random.default_rng(3)
    grid = OF.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    shape = (1, 2, 192, 128)
    q, k, v = (grid[g.integers(0, 127, shape)] * np.where(g.random(shape) < 0.5, -1, 1) for _ in range(3))
    for x in (q, k):
        x[:, :, ::64, 0] = 448.0
    v[:, :, 0, :] = 448.0
    mask = (g.random((1, 2, 3, 3)) < 0.6).astype(np.uint8)
    mask[..., np.arange(3), np.arange(3)] = 1
    scale = 1e-4
    o8, l8, _ = OF.attention_fp8(q, k, v, mask, 64, scale=scale)
    o, l = OA.block_sparse_attention(q, k, v, mask, 64, scale=scale)
    np.testing.assert_allclose(o8, o, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(l8, l, rtol=1e-12)


def _dequantised(q, k, v):
    return (OF.dequantise_rows(*OF.quantise_rows(q)), OF.dequantise_rows(*OF.quantise_rows(k)),
            OF.dequantise_channels(*OF.quantise_channels(v)))


def test_rounded_p_against_torch_cast_of_the_oracle_probabilities():
    """The rounded-P attention recomputed another way: the plain oracle's
    normalised probabilities p over the dequantised inputs, scaled so that the
    row's largest is 1 (P = p / max p, whose sum is 1 / max p), rounded by torch's
    float8_e4m3fn cast, times V, divided by that sum."""
    g = np.random.default_rng(11)
    B, H, N, D, bs = 1, 2, 150, 16, 32
    q, k, v = (g.standard_normal((B, H, N, D)) * 2.0 for _ in range(3))
    mask = (g.random((H, 5, 5)) < 0.6).astype(np.uint8)
    mask[0, 2] = 0                                          # a query block that keeps nothing
    o, lse = OF.attention_fp8_rounded_p(q, k, v, mask, bs)
    qd, kd, vd = _dequantised(q, k, v)
    _, l_ref, p = OA.block_sparse_attention(qd, kd, vd, mask, bs, return_probs=True)
    pmax = p.max(axis=-1, keepdims=True)
    ok = pmax > 0
    P = np.where(ok, p / np.where(ok, pmax, 1.0), 0.0)
    Pr = torch.tensor(P).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = np.einsum("bhij,bhjd->bhid", Pr, vd) * pmax
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=1e-12)
    assert (o[0, 0, 64:96] == 0).all() and np.isneginf(lse[0, 0, 64:96]).all()


def test_rounded_p_leaves_probabilities_on_the_e4m3_grid_unchanged():
    """Logits ln 2 * n with n a power of two (or 0) up to 8: every P = 2^(n - 8) is
    an e4m3 value (2^-8 a subnormal), so rounding changes nothing and the result is
    the unrounded FP8 oracle's."""
    g = np.random.default_rng(12)
    B, H, N, D = 1, 1, 128, 4
    q = np.zeros((B, H, N, D)); q[..., 0] = 1.0
    k = np.zeros((B, H, N, D)); k[..., 0] = g.choice([0.0, 1.0, 2.0, 4.0, 8.0], N)
    k[:, :, ::64, 0] = 8.0                                  # every 64-row block's amax is 8
    v = g.standard_normal((B, H, N, D))
    mask = np.ones((2, 2), np.uint8)
    o, lse = OF.attention_fp8_rounded_p(q, k, v, mask, 64, scale=np.log(2.0))
    o_u, lse_u, _ = OF.attention_fp8(q, k, v, mask, 64, scale=np.log(2.0))
    np.testing.assert_allclose(o, o_u, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(lse, lse_u, rtol=1e-12)


def test_rounded_p_within_half_a_step_of_the_unrounded_result():
    """|o_rounded - o| <= sum_j |e4m3(P_j) - P_j| |v_j| / sum_j P_j, with the
    rounding of each P at most half a step: 2^-4 P for normals (P >= 2^-6) and
    2^-10 below; and the rounding does change the result on random inputs."""
    g = np.random.default_rng(13)
    B, H, N, D, bs = 1, 1, 96, 8, 32
    q, k, v = (g.standard_normal((B, H, N, D)) * 1.5 for _ in range(3))
    mask = np.ones((3, 3), np.uint8)
    o, _ = OF.attention_fp8_rounded_p(q, k, v, mask, bs)
    o_u, _, _ = OF.attention_fp8(q, k, v, mask, bs)
    qd, kd, vd = _dequantised(q, k, v)
    s = (qd[0, 0] @ kd[0, 0].T) / np.sqrt(D)
    P = np.exp(s - s.max(axis=1, keepdims=True))
    half = np.maximum(P * 2.0 ** -4, 2.0 ** -10)
    bound = (half @ np.abs(vd[0, 0])) / P.sum(axis=1, keepdims=True)
    assert (np.abs(o[0, 0] - o_u[0, 0]) <= bound * (1 + 1e-9)).all()
    assert np.abs(o - o_u).max() > 1e-4
