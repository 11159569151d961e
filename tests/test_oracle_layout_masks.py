"""Pins for oracle.layout and oracle.masks: hand-worked values, closed forms,
invariants and brute force over token pairs. CPU only."""
import numpy as np
import pytest

from oracle import layout as L
from oracle import masks as M
from workloads import WAN480, HUNYUAN720, LONG126


def test_frame_major_hand_worked_values_4x8x8():
    """On the 4x8x8 grid, natural n = 64 t + 8 y + x goes to (8 y + x) * 4 + t."""
    pi = L.frame_major_map(4, 8, 8)
    assert pi[64] == 1        # (t=1, y=0, x=0)
    assert pi[1] == 4         # (t=0, y=0, x=1)
    assert pi[255] == 255     # (t=3, y=7, x=7)
    assert pi[0] == 0
    assert pi[8] == 32        # (t=0, y=1, x=0)


@pytest.mark.parametrize("grid", [(4, 8, 8), (5, 3, 7), (21, 30, 52), (1, 4, 4), (3, 1, 1)])
def test_frame_major_is_bijection_with_contiguous_position_runs(grid):
    T, Hh, W = grid
    pi = L.frame_major_map(*grid)
    N = T * Hh * W
    assert np.array_equal(np.sort(pi), np.arange(N))
    t, y, x = L.grid_coords(*grid)
    # each spatial position's T frames form one contiguous run, in frame order
    s = y * W + x
    for sp in np.random.default_rng(0).choice(Hh * W, size=min(20, Hh * W), replace=False):
        run = np.sort(pi[s == sp])
        assert np.array_equal(run, run[0] + np.arange(T))
        assert np.array_equal(pi[s == sp], run)            # t ascending -> position ascending
    # closed form, checked against the sort-built map everywhere
    assert np.array_equal(pi, s * T + t)


def test_permute_roundtrip_and_head_select():
    grid = (3, 4, 5)
    N = 60
    x = np.random.default_rng(1).standard_normal((2, 3, N, 4))
    sel = [1, 0, 1]
    y = L.permute(x, grid, "frame_major", False, sel)
    assert np.array_equal(y[:, 1], x[:, 1])                 # unselected head copied
    assert not np.array_equal(y[:, 0], x[:, 0])
    assert np.array_equal(L.permute(y, grid, "frame_major", True, sel), x)
    pi = L.frame_major_map(*grid)
    assert np.array_equal(y[:, 0, pi], x[:, 0])


def test_cube_counts_on_the_wan_grid():
    """21x30x52 in 4x4x4 cubes: 6*8*13 = 624 cubes; by extents (4 or 1 frames) x
    (4 or 2 rows) x 4 columns the valid sizes are 64 (455), 32 (65), 16 (91), 8 (13)."""
    slot, counts, n_slots = L.cube_map(21, 30, 52, 4)
    assert counts.size == 624 and n_slots == 39936
    vals, freq = np.unique(counts, return_counts=True)
    assert dict(zip(vals.tolist(), freq.tolist())) == {8: 13, 16: 91, 32: 65, 64: 455}
    assert counts.sum() == 32760


@pytest.mark.parametrize("grid", [(4, 8, 8), (5, 6, 7), (21, 30, 52)])
def test_cube_slots_valid_prefix_raster_order(grid):
    T, Hh, W = grid
    slot, counts, n_slots = L.cube_map(T, Hh, W, 4)
    N = T * Hh * W
    assert np.unique(slot).size == N and slot.max() < n_slots
    cube, rank = slot // 64, slot % 64
    assert np.array_equal(np.bincount(cube, minlength=counts.size), counts)
    assert (rank < counts[cube]).all()                      # valid tokens form a prefix
    t, y, x = L.grid_coords(T, Hh, W)
    assert np.array_equal(cube, ((t // 4) * (-(-Hh // 4)) + y // 4) * (-(-W // 4)) + x // 4)
    # inside each cube, rank follows natural (t, y, x) raster order
    for c in np.random.default_rng(2).choice(counts.size, size=min(30, counts.size), replace=False):
        members = np.nonzero(cube == c)[0]
        assert np.array_equal(rank[members], np.arange(members.size))


def test_cube_permute_roundtrip_zero_pads():
    grid = (5, 6, 7)
    x = np.random.default_rng(3).standard_normal((1, 2, 210, 3))
    y = L.permute(x, grid, "cube4")
    slot, counts, n_slots = L.cube_map(*grid, 4)
    pad = np.setdiff1d(np.arange(n_slots), slot)
    assert (y[:, :, pad] == 0).all()
    assert np.array_equal(L.permute(y, grid, "cube4", inverse=True), x)


@pytest.mark.parametrize("grid,bs,kind,w", [
    ((4, 8, 8), 64, "spatial", 0), ((4, 8, 8), 64, "spatial", 1),
    ((4, 8, 8), 64, "temporal", 0), ((4, 8, 8), 16, "temporal", 3),
    ((5, 6, 7), 16, "spatial", 1), ((5, 6, 7), 16, "temporal", 2),    # ragged last block
    ((7, 9, 11), 64, "spatial", 2), ((7, 9, 11), 64, "temporal", 5),
    ((6, 12, 10), 128, "temporal", 0), ((3, 5, 5), 8, "spatial", 0),
])
def test_interval_rule_matches_brute_force(grid, bs, kind, w):
    assert np.array_equal(M.pattern_mask(grid, bs, kind, w), M.pattern_mask_bruteforce(grid, bs, kind, w))


def test_densities_and_row_counts_at_full_shapes():
    """Block densities and kept-per-row ranges of the video-shaped workloads."""
    ms = M.pattern_mask(WAN480.grid, 128, "spatial", 1)
    mt = M.pattern_mask(WAN480.grid, 128, "temporal", 0)
    assert round(ms.mean(), 4) == 0.1448 and (ms.sum(1).min(), ms.sum(1).max()) == (25, 50)
    assert round(mt.mean(), 4) == 0.0113 and (mt.sum(1).min(), mt.sum(1).max()) == (2, 3)
    assert round(M.pattern_mask(HUNYUAN720.grid, 128, "spatial", 2).mean(), 4) == 0.1476
    assert round(M.pattern_mask(HUNYUAN720.grid, 128, "temporal", 276).mean(), 4) == 0.1500
    ml = M.pattern_mask(LONG126.grid, 128, "spatial", 1)
    assert round(ml.mean(), 4) == 0.0249
    # a same-frame window always keeps the diagonal; so does a same-position band
    assert ms.diagonal().all() and mt.diagonal().all() and ml.diagonal().all()


def test_mask_list_roundtrip():
    m = (np.random.default_rng(4).random((2, 3, 7, 9)) < 0.4).astype(np.uint8)
    idx, cnt = M.mask_to_list(m)
    assert np.array_equal(M.list_to_mask(idx, cnt, 9), m)
    for r, c in zip(idx.reshape(-1, 9), cnt.reshape(-1)):
        assert (np.diff(r[:c]) > 0).all() and (r[c:] == -1).all()
