"""Skiparse-2D fixed spatial patterns (test infrastructure only).

OSP-Next page, "Method": the sparse half of the model's hybrid attention uses
fixed token-wise and group-wise patterns along the spatial dimensions, chosen so
that they keep locality and run on FlashAttention-style kernels. The page says
nothing more; the reading used here, for an integer factor k >= 1:

* token-wise: token (t, y, x) belongs to subset (y mod k, x mod k): the tokens
  of a subset sit k apart along both spatial axes (a strided sample of every
  frame);
* group-wise: the frame is tiled by contiguous k x k patches; token (t, y, x) lies
  in patch (y div k, x div k) and belongs to subset ((y div k) mod k,
  (x div k) mod k): whole patches, k patches apart along both axes;
* a query attends, with one softmax, to every key of its own subset in every
  frame (the temporal axis stays dense); subset (a, b) has id a k + b.

Each pattern keeps about 1/k^2 of the pairs. Stored subset by subset, each
subset is one dense attention of its own, i.e. a block-diagonal mask, which is
what makes it FlashAttention-compatible. The layout used for that: subsets in id
order, each padded to a whole number of bs-slot blocks, a subset's tokens in its
first slots in natural order.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention
from .layout import grid_coords

MODES = ("token", "group")


def subset_ids(grid, k: int, mode: str) -> np.ndarray:
    """Subset id of every token in natural order (int64, length N)."""
    T, Hh, W = grid
    if k < 1 or mode not in MODES:
        raise ValueError("k >= 1 and mode 'token' or 'group'")
    _, y, x = grid_coords(T, Hh, W)
    if mode == "token":
        a, b = y % k, x % k
    else:
        a, b = (y // k) % k, (x // k) % k
    return a * k + b


def pair_allowed(grid, k: int, mode: str, i: int, j: int) -> bool:
    """Whether query i may attend to key j, stated on the coordinates of the two
    tokens (no subset ids): the two conditions along y and x."""
    T, Hh, W = grid
    yi, xi = (i // W) % Hh, i % W
    yj, xj = (j // W) % Hh, j % W
    if mode == "token":
        return (yi - yj) % k == 0 and (xi - xj) % k == 0
    return (yi // k - yj // k) % k == 0 and (xi // k - xj // k) % k == 0


def attention(q, k_, v, grid, k: int, mode: str, scale=None, rows=None):
    """Skiparse-2D attention in natural coordinates: (o [B,H,R,D], lse [B,H,R]).
    The subset id is the block id on both sides and the mask is the identity over
    subsets, so query i attends exactly to the keys of its subset."""
    sid = subset_ids(grid, k, mode)
    mask = np.eye(k * k, dtype=np.uint8)
    return masked_attention(q, k_, v, mask, sid, sid, scale, rows=rows)


def layout(grid, k: int, mode: str, bs: int):
    """Padded subset-major layout: (slot [N], blk_len [nb], n_slots) with slot[n]
    the position of natural token n and blk_len the valid slots of each block."""
    sid = subset_ids(grid, k, mode)
    N = sid.size
    n_sub = k * k
    counts = np.bincount(sid, minlength=n_sub)
    blocks = -(-counts // bs)                          # whole blocks per subset
    start = np.concatenate([[0], np.cumsum(blocks * bs)])[:-1]
    order = np.lexsort((np.arange(N), sid))            # by subset, then natural order
    rank = np.empty(N, np.int64)
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]
    rank[order] = np.arange(N) - first[sid[order]]
    slot = start[sid] + rank
    n_slots = int(blocks.sum() * bs)
    blk_len = np.zeros(n_slots // bs, np.int64)
    for c in range(n_sub):
        for i in range(blocks[c]):
            blk_len[start[c] // bs + i] = min(bs, counts[c] - i * bs)
    return slot, blk_len, n_slots


def block_subset(grid, k: int, mode: str, bs: int) -> np.ndarray:
    """Subset id of every block of the padded layout."""
    sid = subset_ids(grid, k, mode)
    counts = np.bincount(sid, minlength=k * k)
    return np.repeat(np.arange(k * k), -(-counts // bs))


def block_mask(grid, k: int, mode: str, bs: int) -> np.ndarray:
    """Block-diagonal block mask [nb, nb] of the padded layout: a block attends
    to the blocks of its own subset."""
    b = block_subset(grid, k, mode, bs)
    return (b[:, None] == b[None, :]).astype(np.uint8)


def permute(x, grid, k: int, mode: str, bs: int, inverse: bool = False) -> np.ndarray:
    """[B, H, N, D] -> [B, H, n_slots, D] (pads zero), or back with inverse."""
    slot, _, n_slots = layout(grid, k, mode, bs)
    x = np.asarray(x)
    if inverse:
        return x[:, :, slot]
    out = np.zeros(x.shape[:2] + (n_slots,) + x.shape[3:], x.dtype)
    out[:, :, slot] = x
    return out


def kept_pairs(grid, k: int, mode: str) -> int:
    """Number of (query, key) pairs the pattern keeps: sum of squared subset sizes."""
    c = np.bincount(subset_ids(grid, k, mode), minlength=k * k)
    return int((c.astype(np.int64) ** 2).sum())
