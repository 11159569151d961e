"""Token orders of a T x Hh x W video grid and the permutations between them.

Natural order lists tokens frame by frame, row by row: position n holds the token
(t, y, x) with n = (t*Hh + y)*W + x.

* Frame-major order (Sparse Video-Gen page, "Approach": the token-major to
  frame-major layout transformation that makes temporal sparsity contiguous):
  all frames of one spatial position (y, x) sit next to each other, ordered by t,
  and positions follow raster order of (y, x). The oracle builds it by sorting
  tokens on the key (y, x, t), not from a closed-form index map.
* Cube order (USV page, Figure 2 caption: the tokens of Q, K and V grouped into
  small spatio-temporal cubes): cubes of c x c x c tokens in raster order of their
  (t/c, y/c, x/c) index, each owning c^3 slots; a cube's valid tokens fill its
  first slots in (t, y, x) raster order and the rest are zero padding. The oracle
  builds it by a stable sort of tokens on their cube id.
"""
from __future__ import annotations

import numpy as np


def grid_coords(T: int, Hh: int, W: int):
    """(t, y, x) of every token in natural order, as int64 arrays of length N."""
    t = np.repeat(np.arange(T), Hh * W)
    y = np.tile(np.repeat(np.arange(Hh), W), T)
    x = np.tile(np.arange(W), T * Hh)
    return t, y, x


def frame_major_map(T: int, Hh: int, W: int) -> np.ndarray:
    """pi[n] = position in frame-major order of the token at natural position n."""
    t, y, x = grid_coords(T, Hh, W)
    order = np.lexsort((t, x, y))      # sequence of natural ids sorted by (y, x, t)
    pi = np.empty(order.size, np.int64)
    pi[order] = np.arange(order.size)
    return pi


def cube_map(T: int, Hh: int, W: int, c: int = 4):
    """Cube layout of the grid.

    Returns (slot, blk_len, n_slots): slot[n] is the padded position of natural
    token n, blk_len[cube] its number of valid tokens, n_slots = n_cubes * c^3.
    """
    t, y, x = grid_coords(T, Hh, W)
    ct, cy, cx = -(-T // c), -(-Hh // c), -(-W // c)
    cube = ((t // c) * cy + (y // c)) * cx + (x // c)
    n_cubes = ct * cy * cx
    N = t.size
    order = np.lexsort((np.arange(N), cube))   # by cube, then natural (raster) order
    counts = np.bincount(cube, minlength=n_cubes)
    starts = np.cumsum(counts) - counts
    rank = np.empty(N, np.int64)
    rank[order] = np.arange(N) - starts[cube[order]]
    slot = cube * c ** 3 + rank
    return slot, counts.astype(np.int64), n_cubes * c ** 3


def permute(x: np.ndarray, grid, kind: str, inverse: bool = False, head_sel=None) -> np.ndarray:
    """Apply a layout change to x of shape [B, H, N, D] (or [B, H, slots, D] for an
    inverse cube move).

    kind "frame_major": forward dst[pi(n)] = src[n]; inverse dst[n] = src[pi(n)].
      Only heads with head_sel[h] != 0 move (None = all); the others are copied.
      Sparse Video-Gen page, "Approach": the transformation serves temporal heads.
    kind "cube4": forward scatters tokens to their cube slots and zero-fills pads;
      inverse gathers each natural token back from its slot (pads are dropped).
    """
    T, Hh, W = grid
    if kind == "frame_major":
        pi = frame_major_map(T, Hh, W)
        out = np.array(x, copy=True)
        heads = range(x.shape[1]) if head_sel is None else [h for h in range(x.shape[1]) if head_sel[h]]
        for h in heads:
            if inverse:
                out[:, h] = x[:, h][:, pi]
            else:
                out[:, h][:, pi] = x[:, h]
        return out
    if kind == "cube4":
        if head_sel is not None:
            raise ValueError("cube layout moves every head")
        slot, _, n_slots = cube_map(T, Hh, W, 4)
        B, H, _, D = x.shape
        if inverse:
            return np.array(x[:, :, slot, :], copy=True)
        out = np.zeros((B, H, n_slots, D), x.dtype)
        out[:, :, slot, :] = x
        return out
    raise ValueError(kind)
