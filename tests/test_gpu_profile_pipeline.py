"""GPU parity of vsa_profile_heads and of the three end-to-end flows against the
oracle (pipelines compared in natural coordinates on sampled rows)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from oracle import attention as OA
from oracle import layout as OL
from oracle import masks as OM
from oracle import pipeline as OP
from oracle import profile as OPR
from oracle import scores as OS
from tests.gpu_util import announce, assert_close_bf16, dev, dev_i32, dev_u8, host
from tests.selection_rules import check_selection
from workloads import WAN480, WAN480_CUBE, LONG126, make_qkv, profile_rows, sample_rows

pytestmark = pytest.mark.gpu

ERR_REL = 1e-3      # error allowed on each candidate's profile error, relative to the decision's scale
GAP_MIN = 1e-4      # choices must agree wherever the oracle's relative gap reaches this


def bf16(x):
    """fp32 array rounded to bf16 values (the inputs the GPU sees), as float64."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def check_profile(err_g, ch_g, err_r, ch_r, what):
    """A candidate's error is compared at the scale of the head's decision: the
    second-smallest oracle error e2 (a candidate with a larger error, at its own
    size). With every candidate off by at most rel.max() of that scale, a head
    whose relative gap (e2 - e1) / e2 exceeds twice rel.max() cannot change its
    choice, so the choice must match there."""
    e = np.sort(err_r, axis=-1)
    e2 = e[..., 1] if err_r.shape[-1] > 1 else e[..., 0]
    scale = np.maximum(np.maximum(np.abs(err_r), e2[..., None]), 1e-30)
    rel = np.abs(err_g - err_r) / scale
    assert rel.max() <= ERR_REL, f"{what}: profile error off by {rel.max():.2e} (relative)"
    gap = (e[..., 1] - e[..., 0]) / np.maximum(e[..., 1], 1e-30) if err_r.shape[-1] > 1 else np.ones(ch_r.shape)
    clear = gap >= max(GAP_MIN, 2 * rel.max())
    assert np.array_equal(ch_g[clear], ch_r[clear]), f"{what}: choice differs where the gap is clear"
    own = np.abs(err_g - err_r) / np.maximum(np.abs(err_r), 1e-30)
    print(f"[{what}] max rel err {rel.max():.2e} (own scale {own.max():.2e}), choices {ch_g.ravel().tolist()} vs "
          f"oracle {ch_r.ravel().tolist()}, min gap {gap.min():.2e}, unchecked {int((~clear).sum())}")
    return gap


def small(grid, H, amplitude, seed, bs=64):
    w = WAN480.scaled(name="small", T=grid[0], Hh=grid[1], W=grid[2], H=H, amplitude=amplitude, seed=seed, bs=bs)
    return w, make_qkv(w)


@pytest.mark.parametrize("amplitude", [0.5, 2.0])
def test_profile_small_grid(amplitude):
    grid, bs = (8, 12, 16), 64
    announce(f"profile small amp={amplitude}")
    w, (q, k, v) = small(grid, 8, amplitude, 5, bs)
    N = w.N
    rows = np.sort(np.random.default_rng([5, 3]).choice(N, size=64, replace=False)).astype(np.int32)
    cands = np.stack([OM.pattern_mask(grid, bs, "spatial", 0), OM.pattern_mask(grid, bs, "temporal", 8)])
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), grid, bs, dev_i32(rows), dev_u8(cands), [0, 1])
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, [0, 1])
    check_profile(host(err), host(ch), er, cr, f"small amp {amplitude}")
    if amplitude == 2.0:
        from workloads import planted_head_type
        assert (host(ch)[0] == planted_head_type(8)).mean() >= 0.9


@pytest.mark.parametrize("P", [1, 3, 4])
def test_profile_candidate_counts_and_identical_candidates(P):
    grid, bs = (6, 8, 10), 64
    announce(f"profile P={P}")
    w, (q, k, v) = small(grid, 3, 0.5, 9, bs)
    rows = np.arange(0, w.N, 7).astype(np.int32)
    base = [OM.pattern_mask(grid, bs, "spatial", 0), OM.pattern_mask(grid, bs, "temporal", 4),
            OM.pattern_mask(grid, bs, "spatial", 1), OM.pattern_mask(grid, bs, "temporal", 4)]
    lay = [0, 1, 0, 1][:P]
    cands = np.stack(base[:P])
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), grid, bs, dev_i32(rows), dev_u8(cands), lay)
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, lay)
    ge = host(err)
    check_profile(ge, host(ch), er, cr, f"P={P}")
    if P == 4:
        assert np.array_equal(ge[..., 1], ge[..., 3])      # identical candidates, identical errors


def test_profile_large_logits_and_rows_a_candidate_keeps_nothing():
    """Scores with a spread of about 35 (Q and K scaled by 6): the running offset
    must keep every exp2 finite. One candidate keeps no key at all for one query
    block, so its output there is 0 and its error is the dense output's square."""
    grid, bs, H = (6, 10, 12), 64, 2
    announce("profile large logits")
    g = np.random.default_rng([31, 1])
    N = grid[0] * grid[1] * grid[2]
    q, k = (bf16((6.0 * g.standard_normal((1, H, N, 128))).astype(np.float32)) for _ in range(2))
    v = bf16(g.standard_normal((1, H, N, 128)).astype(np.float32))
    rows = np.sort(g.choice(N, size=48, replace=False)).astype(np.int32)
    c0 = OM.pattern_mask(grid, bs, "spatial", 0)
    qb = int(rows[5]) // bs
    c0[qb, :] = 0                                           # the sampled row 5 keeps nothing under candidate 0
    cands = np.stack([c0, OM.pattern_mask(grid, bs, "temporal", 2)])
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), grid, bs, dev_i32(rows), dev_u8(cands), [0, 1])
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, [0, 1])
    assert np.isfinite(host(err)).all()
    check_profile(host(err), host(ch), er, cr, "large logits")


def test_profile_two_batch_entries():
    """B = 2: every (b, h) pair profiled on the shared rows, against the oracle;
    the second batch entry holds different inputs (a different seed)."""
    grid, bs = (6, 10, 12), 64
    announce("profile B=2")
    w = WAN480.scaled(name="b2", T=grid[0], Hh=grid[1], W=grid[2], H=3, amplitude=2.0, seed=21, bs=bs)
    q1, k1, v1 = make_qkv(w)
    q2, k2, v2 = make_qkv(w.scaled(seed=22))
    q, k, v = (np.concatenate(p, axis=0) for p in ((q1, q2), (k1, k2), (v1, v2)))
    rows = np.sort(np.random.default_rng([21, 1]).choice(w.N, size=40, replace=False)).astype(np.int32)
    cands = np.stack([OM.pattern_mask(grid, bs, "spatial", 0), OM.pattern_mask(grid, bs, "temporal", 3)])
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), grid, bs, dev_i32(rows), dev_u8(cands), [0, 1])
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, [0, 1])
    assert host(err).shape == (2, 3, 2)
    check_profile(host(err), host(ch), er, cr, "B=2")


@pytest.mark.parametrize("bs,shuffle", [(48, True), (64, True), (40, False)])
def test_profile_ragged_blocks_and_unsorted_rows(bs, shuffle):
    """Blocks that are not a whole number of 32-key words (bit words built run
    by run), sampled rows in no particular order (each pass orders them by its
    layout), and candidates of both layouts, one natural one beyond the dense
    pass's own."""
    grid = (5, 9, 11)
    announce(f"profile ragged bs={bs} shuffle={shuffle}")
    w, (q, k, v) = small(grid, 3, 0.5, 13, bs)
    g = np.random.default_rng([13, bs])
    rows = g.choice(w.N, size=70, replace=False).astype(np.int32)
    if not shuffle:
        rows = np.sort(rows)
    cands = np.stack([OM.pattern_mask(grid, bs, "spatial", 0), OM.pattern_mask(grid, bs, "temporal", 2),
                      OM.pattern_mask(grid, bs, "spatial", 1)])
    lay = [0, 1, 0]
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), grid, bs, dev_i32(rows), dev_u8(cands), lay)
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, lay)
    check_profile(host(err), host(ch), er, cr, f"ragged bs={bs}")


@pytest.mark.parametrize("amplitude", [0.5, 4.0])
def test_profile_wan_full_shape(amplitude):
    """The benchmarked launch: Wan 480p, 12 heads, 1 % rows (328), spatial w=1 in
    natural order vs temporal w=0 in frame-major order. At amplitude 0.5 (the
    benchmark's generator) every head prefers the spatial pattern; at 4.0 the
    planted head types show (even heads spatial, odd heads temporal), so the
    choice is mixed and both outcomes are checked against the oracle at the full
    shape."""
    w = WAN480.scaled(name=f"wan480_amp{amplitude}", amplitude=amplitude)
    announce(f"profile wan full amp={amplitude}")
    q, k, v = make_qkv(w)
    rows = profile_rows(w)
    assert rows.size == 328
    cands = np.stack([OM.pattern_mask(w.grid, w.bs, "spatial", 1), OM.pattern_mask(w.grid, w.bs, "temporal", 0)])
    err, ch = V.vsa_profile_heads(dev(q), dev(k), dev(v), w.grid, w.bs, dev_i32(rows), dev_u8(cands), [0, 1])
    er, cr = OPR.profile_heads(q, k, v, w.grid, w.bs, rows, cands, [0, 1])
    gap = check_profile(host(err), host(ch), er, cr, f"wan full amp {amplitude}")
    if amplitude == 4.0:
        from workloads import planted_head_type
        assert np.array_equal(cr[0], planted_head_type(w.H)), "the oracle's choice follows the planted types"
        assert (gap >= GAP_MIN).all()
        assert np.array_equal(host(ch), cr)


def test_svg_pipeline_wan_full_shape():
    """Masks -> profiler -> frame-major permute of temporal heads -> lists ->
    attention -> inverse permute, against the oracle's pulled-back masks. The
    temporal path is forced on odd heads (choice given) so both branches run."""
    w = WAN480
    announce("svg pipeline wan full")
    q, k, v = make_qkv(w)
    choice = [h % 2 for h in range(w.H)]
    o, sel = PL.svg_layer(dev(q), dev(k), dev(v), w.grid, w.bs, 1, 0, None, choice=choice)
    # the fused kernel and the separate permute calls agree bit for bit
    o_sep, _ = PL.svg_layer(dev(q), dev(k), dev(v), w.grid, w.bs, 1, 0, None, choice=choice, fused=False)
    assert torch.equal(o, o_sep)
    rows = sample_rows(w.N, w.bs, 768, 11)
    ro, _ = OP.svg_pipeline(q, k, v, w.grid, w.bs, [choice], 1, 0, rows=rows)
    assert_close_bf16(host(o)[:, :, rows], ro, "svg pipeline")
    # and the profiler-driven path runs end to end
    rows_p = dev_i32(profile_rows(w))
    o2, sel2 = PL.svg_layer(dev(q), dev(k), dev(v), w.grid, w.bs, 1, 0, rows_p)
    ro2, _ = OP.svg_pipeline(q, k, v, w.grid, w.bs, [sel2], 1, 0, rows=rows)
    assert_close_bf16(host(o2)[:, :, rows], ro2, "svg pipeline (profiled)")


def test_svg_layer_two_batch_entries():
    """The profiled layer with B = 2 (different inputs per entry): every (b, h)
    gets its own choice on the device, the attention follows it, and the output
    equals the oracle's layer under the same choices at every row."""
    grid, bs, H = (4, 10, 12), 64, 3
    announce("svg layer B=2")
    w = WAN480.scaled(name="svg_b2", T=grid[0], Hh=grid[1], W=grid[2], H=H, amplitude=4.0, seed=41, bs=bs)
    q1, k1, v1 = make_qkv(w)
    q2, k2, v2 = make_qkv(w.scaled(seed=42))
    q, k, v = (np.concatenate(p, axis=0) for p in ((q1, q2), (k1, k2), (v1, v2)))
    rows = profile_rows(w)
    o, ch = PL.svg_layer(dev(q), dev(k), dev(v), grid, bs, 0, 2, dev_i32(rows))
    assert np.array(ch).shape == (2, H)
    cands = np.stack([OM.pattern_mask(grid, bs, "spatial", 0), OM.pattern_mask(grid, bs, "temporal", 2)])
    er, cr = OPR.profile_heads(q, k, v, grid, bs, rows, cands, [0, 1])
    e = np.sort(er, axis=-1)
    clear = (e[..., 1] - e[..., 0]) / np.maximum(e[..., 1], 1e-30) >= 2e-3
    assert np.array_equal(np.array(ch)[clear], cr[clear])
    ro, _ = OP.svg_pipeline(q, k, v, grid, bs, ch, 0, 2)
    assert_close_bf16(host(o), ro, "svg layer B=2")


def test_cube_pipeline_wan_full_shape():
    w = WAN480_CUBE
    announce("cube pipeline wan full")
    q, k, v = make_qkv(w)
    stats = {}
    o = PL.cube_layer(dev(q), dev(k), dev(v), w.grid, w.extra["k_frac"], w.extra["top_p"], stats=stats)
    gi, gc = host(stats["kv_idx"]), host(stats["kv_cnt"])
    # selection against the oracle's fp64 cube scores (gap rule)
    rS = OP.cube_scores(q, k, w.grid)
    n, exact, bad = check_selection(rS, None, 93, w.extra["top_p"], gi, gc)
    assert not bad, f"{len(bad)} of {n} rows beyond the gap rule"
    # attention under the GPU's selection, pulled back to natural coordinates
    slot, counts, _ = OL.cube_map(*w.grid, 4)
    cube = slot // 64
    mask = OM.list_to_mask(gi, gc, counts.size)
    rows = sample_rows(w.N, 64, 768, 12)
    ro, _ = OA.masked_attention(q, k, v, mask, cube, cube, rows=rows)
    assert_close_bf16(host(o)[:, :, rows], ro, "cube pipeline")


def test_long_pipeline_full_shape():
    w = LONG126
    H = 3
    announce("long pipeline full")
    q, k, v = make_qkv(w, H=H)
    stats = {}
    k_total = int(round(w.extra["density"] * w.nb))
    o = PL.long_layer(dev(q), dev(k), dev(v), w.grid, w.bs, 1, k_total, stats=stats)
    gi, gc = host(stats["kv_idx"]), host(stats["kv_cnt"])
    forced = OM.pattern_mask(w.grid, w.bs, "spatial", 1)
    rS, _, _ = OS.block_scores(q, k, w.bs)
    n, exact, bad = check_selection(rS, forced, k_total, 1.0, gi, gc)
    assert not bad
    mask = OM.list_to_mask(gi, gc, w.nb)
    rows = sample_rows(w.N, w.bs, 768, 13)
    ro, _ = OA.block_sparse_attention(q, k, v, mask, w.bs, rows=rows)
    assert_close_bf16(host(o)[:, :, rows], ro, "long pipeline")
