"""FP8 (e4m3) block-sparse attention (test infrastructure only).

Sparse Video-Gen page ("Key results"; also the Sparse VideoGen2 and USV pages'
speed-ups) reports further gains when the attention runs in FP8. The page fixes
no quantisation scheme; the plainest reading, used here:

* Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals, largest finite 448, codes 0x7F / 0xFF are NaN, no
  infinities; round to nearest, ties to even.
* Q and K: one scale per (b, h, block of 64 positions): s = amax / 448 with amax
  the largest |x| over the block's rows and channels (fp32), code =
  e4m3(x * (448 / amax)), both products in fp32; a block of zeros has s = 0 and
  codes 0.
* V: one scale per (b, h, channel) over all positions, same rule.
* The attention is then plain block-sparse attention on the dequantised values
  code * s (``oracle.attention``). ``attention_fp8_rounded_p`` adds the usual FP8
  attention practice of rounding the probabilities to e4m3 before they multiply
  V: with m_i the row's largest kept logit, P_ij = exp(s_ij - m_i), o_i =
  sum_j e4m3(P_ij) v_j / sum_j P_ij and lse_i = m_i + log sum_j P_ij. A kernel
  with a lazily moved offset forms the same P whenever its offset is the row
  maximum (e.g. when the maximum lies in the first kept tile); fp32 sums are
  covered by the test tolerance.
* V is stored transposed in tiles of 64 keys: [B, H, ceil(N / 64), D, 64], key
  k = 32 st + 8 g + 4 h + e (st, h in {0, 1}; g, e in [0, 4)) of a tile at column
  32 h + 16 st + 4 g + e, keys past N zero. (This is the order in which the
  score accumulator of the 32x32 MFMA holds a lane's keys.)
"""
from __future__ import annotations

import numpy as np

from .attention import block_sparse_attention

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code (ties to even); |x| beyond the rounding range of 448 and
    NaN give NaN (0x7F with the sign)."""
    x = np.asarray(x, np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    # all 127 non-negative finite codes, ascending
    grid = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    idx = np.searchsorted(grid, a, side="left")           # grid[idx-1] < a <= grid[idx]
    idx = np.clip(idx, 1, 126)
    lo, hi = grid[idx - 1], grid[idx]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((idx & 1) == 0))
    code = np.where(pick_hi, idx, idx - 1).astype(np.int64)
    code = np.where(a <= grid[0], 0, code)
    # past 448: above the midpoint 464 to the next (missing) step, rounding leaves the
    # range; 464 itself ties to the even code 448
    code = np.where(a > 464.0, 0x7F, code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code.astype(np.uint8) | sign)


def _quantise(x32: np.ndarray, amax: np.ndarray):
    amax = amax.astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / np.where(amax > 0, amax, np.float32(1)), np.float32(0))
    y = (x32 * inv.astype(np.float32)).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y), scale


def quantise_rows(x, block: int = 64):
    """x [B, H, N, D] -> (codes uint8 [B, H, N, D], scales fp32 [B, H, ceil(N / block)])."""
    x32 = np.asarray(x, np.float32)
    B, H, N, D = x32.shape
    nb = -(-N // block)
    pad = np.zeros((B, H, nb * block, D), np.float32)
    pad[:, :, :N] = x32
    blocks = pad.reshape(B, H, nb, block, D)
    amax = np.abs(blocks).max(axis=(3, 4))
    codes, scale = _quantise(blocks, amax[..., None, None])
    return codes.reshape(B, H, nb * block, D)[:, :, :N], scale[..., 0, 0]


def quantise_channels(x):
    """x [B, H, N, D] -> (codes uint8 [B, H, N, D], scales fp32 [B, H, D])."""
    x32 = np.asarray(x, np.float32)
    amax = np.abs(x32).max(axis=2)
    codes, scale = _quantise(x32, amax[:, :, None, :])
    return codes, scale[:, :, 0, :]


def dequantise_rows(codes, scales, block: int = 64):
    B, H, N, D = codes.shape
    s = np.repeat(np.asarray(scales, np.float64), block, axis=2)[:, :, :N]
    return e4m3_decode(codes) * s[..., None]


def dequantise_channels(codes, scales):
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, :, None, :]


def vt_column(k: np.ndarray) -> np.ndarray:
    """Column of key k (0..63) in a transposed V tile."""
    k = np.asarray(k)
    st, g, h, e = k >> 5, (k >> 3) & 3, (k >> 2) & 1, k & 3
    return 32 * h + 16 * st + 4 * g + e


def vt_tiles(codes) -> np.ndarray:
    """codes [B, H, N, D] -> [B, H, ceil(N / 64), D, 64] (see the module text)."""
    B, H, N, D = codes.shape
    nt = -(-N // 64)
    out = np.zeros((B, H, nt, D, 64), np.uint8)
    k = np.arange(64)
    col = vt_column(k)
    for t in range(nt):
        rows = np.arange(t * 64, min(N, t * 64 + 64))
        out[:, :, t][..., col[:rows.size]] = np.transpose(codes[:, :, rows, :], (0, 1, 3, 2))
    return out


def attention_fp8(q, k, v, mask, bs: int, blk_len=None, scale=None):
    """(o, lse, parts): block-sparse attention on the dequantised Q, K, V."""
    qc, qs = quantise_rows(q)
    kc, ks = quantise_rows(k)
    vc, vs = quantise_channels(v)
    qd, kd, vd = dequantise_rows(qc, qs), dequantise_rows(kc, ks), dequantise_channels(vc, vs)
    if scale is None:
        scale = 1.0 / np.sqrt(np.asarray(q).shape[-1])
    o, lse = block_sparse_attention(qd, kd, vd, mask, bs, blk_len, scale)
    return o, lse, dict(q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs)


def attention_fp8_rounded_p(q, k, v, mask, bs: int, scale=None, rows=None):
    """(o, lse) of the natural blocked layout (position i in block i // bs, the
    last block ragged): attention on the dequantised Q, K, V with the
    probabilities rounded to e4m3 before they multiply V (module text); mask
    [nqb, nkb] | [H, nqb, nkb] | [B, H, nqb, nkb]. Rows that keep nothing get
    o = 0 and lse = -inf."""
    qd = dequantise_rows(*quantise_rows(q))
    kd = dequantise_rows(*quantise_rows(k))
    vd = dequantise_channels(*quantise_channels(v))
    B, H, N, D = qd.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    m4 = np.asarray(mask)
    m4 = np.broadcast_to(m4, (B, H) + m4.shape[-2:]) if m4.ndim < 4 else m4
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((B, H, rows.size, D))
    lse = np.full((B, H, rows.size), -np.inf)
    for b in range(B):
        for h in range(H):
            for qb in np.unique(rows // bs):
                sel = np.nonzero(rows // bs == qb)[0]
                keys = np.concatenate([np.arange(kb * bs, min(N, (kb + 1) * bs))
                                       for kb in np.nonzero(m4[b, h, qb])[0]] + [np.zeros(0, np.int64)])
                if keys.size == 0:
                    continue
                s = scale * (qd[b, h, rows[sel]] @ kd[b, h, keys].T)
                m = s.max(axis=1, keepdims=True)
                pr = np.exp(s - m)
                l = pr.sum(axis=1, keepdims=True)
                o[b, h, sel] = (e4m3_decode(e4m3_encode(pr)) @ vd[b, h, keys]) / l
                lse[b, h, sel] = (m + np.log(l))[:, 0]
    return o, lse
