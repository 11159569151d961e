"""Pins for oracle.profile and oracle.pipeline: equivariance between the moved and
the pulled-back forms, the all-rows special case, ties, and recovery of a
planted head type by a strong generator. CPU only."""
import numpy as np

from oracle import attention as A
from oracle import layout as L
from oracle import masks as M
from oracle import pipeline as PL
from oracle import profile as P
from oracle import scores as S
from oracle import select as SEL
from workloads import WAN480, make_qkv, planted_head_type


def small(grid, H=4, amplitude=0.5, seed=11, D=128):
    w = WAN480.scaled(name="small", T=grid[0], Hh=grid[1], W=grid[2], H=H,
                      amplitude=amplitude, seed=seed, D=D)
    return w, make_qkv(w)


def test_frame_major_candidate_equals_moved_tensors():
    """Evaluating a frame-major mask through the layout map equals permuting Q, K, V,
    attending under the mask in frame-major order, and permuting back."""
    grid, bs = (4, 6, 10), 32
    w, (q, k, v) = small(grid, H=2)
    mt = M.pattern_mask(grid, bs, "temporal", 3)
    blk = P.layout_blocks(grid, bs, 1)
    o_pull, l_pull = A.masked_attention(q, k, v, mt, blk, blk)
    qm, km, vm = (L.permute(x, grid, "frame_major") for x in (q, k, v))
    o_mv, l_mv = A.block_sparse_attention(qm, km, vm, mt, bs)
    o_back = L.permute(o_mv, grid, "frame_major", inverse=True)
    pi = L.frame_major_map(*grid)
    assert np.abs(o_pull - o_back).max() <= 1e-12
    assert np.abs(l_pull - l_mv[:, :, pi]).max() <= 1e-12


def test_all_rows_profile_equals_full_error_argmin():
    grid, bs = (4, 6, 10), 32
    w, (q, k, v) = small(grid, H=4)
    N = w.N
    cands = np.stack([M.pattern_mask(grid, bs, "spatial", 0), M.pattern_mask(grid, bs, "temporal", 2)])
    err, choice = P.profile_heads(q, k, v, grid, bs, np.arange(N), cands, [0, 1])
    od, _ = A.dense_attention(q, k, v)
    os_, _ = A.block_sparse_attention(q, k, v, cands[0], bs)
    blk = L.frame_major_map(*grid) // bs
    ot, _ = A.masked_attention(q, k, v, cands[1], blk, blk)
    e_ref = np.stack([((os_ - od) ** 2).sum((-1, -2)), ((ot - od) ** 2).sum((-1, -2))], -1)
    assert np.abs(err - e_ref).max() <= 1e-9 * max(1.0, e_ref.max())
    assert np.array_equal(choice, np.argmin(e_ref, -1))


def test_identical_candidates_tie_to_the_first():
    grid, bs = (3, 4, 8), 16
    w, (q, k, v) = small(grid, H=2)
    m = M.pattern_mask(grid, bs, "spatial", 0)
    err, choice = P.profile_heads(q, k, v, grid, bs, np.arange(0, w.N, 5), np.stack([m, m]), [0, 0])
    assert (err[..., 0] == err[..., 1]).all() and (choice == 0).all()


def test_strong_generator_recovers_planted_head_types():
    """With the positional signal at amplitude 2.0 each head's planted type
    (even spatial, odd temporal) is what the 1 % profiler picks on >= 90 % of heads."""
    grid, bs = (8, 12, 16), 64
    w, (q, k, v) = small(grid, H=8, amplitude=2.0, seed=5)
    N = w.N
    rows = np.sort(np.random.default_rng([5, 3]).choice(N, size=max(16, N // 100), replace=False))
    cands = np.stack([M.pattern_mask(grid, bs, "spatial", 0), M.pattern_mask(grid, bs, "temporal", 8)])
    _, choice = P.profile_heads(q, k, v, grid, bs, rows, cands, [0, 1])
    assert (choice[0] == planted_head_type(8)).mean() >= 0.9


def test_cube_pipeline_equals_moved_cube_layout():
    """Scores, selection and attention in cube layout (tensors moved, blk_len
    validity) equal the natural-coordinate pipeline."""
    grid = (5, 6, 9)
    w, (q, k, v) = small(grid, H=2, seed=3)
    nc_slot, counts, n_slots = L.cube_map(*grid, 4)
    o_nat, l_nat, idx, cnt = PL.cube_pipeline(q, k, v, grid, k_max=5, top_p=0.9)
    qc, kc, vc = (L.permute(x, grid, "cube4") for x in (q, k, v))
    Sc = S.block_scores(qc, kc, 64, counts)[0]
    assert np.abs(Sc - PL.cube_scores(q, k, grid)).max() <= 1e-12
    idx2, cnt2 = SEL.select(Sc, None, 5, 0.9)
    assert np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2)
    mask = M.list_to_mask(idx2, cnt2, counts.size)
    oc, lc = A.block_sparse_attention(qc, kc, vc, mask, 64, counts)
    assert np.abs(L.permute(oc, grid, "cube4", inverse=True) - o_nat).max() <= 1e-12
    assert np.abs(lc[:, :, nc_slot] - l_nat).max() <= 1e-12


def test_long_pipeline_keeps_local_window_and_budget():
    grid, bs = (6, 4, 8), 16
    w, (q, k, v) = small(grid, H=2, seed=4)
    o, lse, idx, cnt = PL.long_pipeline(q, k, v, grid, bs, 1, 8)
    forced = M.pattern_mask(grid, bs, "spatial", 1)
    assert forced.sum(1).max() <= 8 < forced.shape[0]
    m = M.list_to_mask(idx, cnt, forced.shape[0])
    assert (m[..., forced == 1] == 1).all()
    assert (cnt == 8).all()
    # the long-range part is the best-scoring non-forced blocks
    Sc = S.block_scores(q, k, bs)[0]
    for h in range(2):
        for qb in range(forced.shape[0]):
            extra = np.nonzero((m[0, h, qb] == 1) & (forced[qb] == 0))[0]
            rest = np.nonzero((m[0, h, qb] == 0) & (forced[qb] == 0))[0]
            if rest.size:
                assert Sc[0, h, qb, extra].min() >= Sc[0, h, qb, rest].max()
    o2, l2 = A.block_sparse_attention(q, k, v, m, bs)
    assert np.abs(o2 - o).max() <= 1e-12


def test_svg_pipeline_matches_per_head_moved_form():
    grid, bs = (4, 6, 10), 32
    w, (q, k, v) = small(grid, H=2, seed=6)
    choice = np.array([[0, 1]])
    o, lse = PL.svg_pipeline(q, k, v, grid, bs, choice, 0, 2)
    ms = M.pattern_mask(grid, bs, "spatial", 0)
    mt = M.pattern_mask(grid, bs, "temporal", 2)
    o0, _ = A.block_sparse_attention(q[:, :1], k[:, :1], v[:, :1], ms, bs)
    sel = [0, 1]
    qm, km, vm = (L.permute(x, grid, "frame_major", False, sel) for x in (q, k, v))
    o1m, _ = A.block_sparse_attention(qm[:, 1:], km[:, 1:], vm[:, 1:], mt, bs)
    o1 = L.permute(o1m, grid, "frame_major", True)
    assert np.abs(o[:, :1] - o0).max() <= 1e-12
    assert np.abs(o[:, 1:] - o1).max() <= 1e-12
