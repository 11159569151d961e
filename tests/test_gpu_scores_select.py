"""GPU parity of vsa_block_scores and vsa_select_topk against the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import layout as OL
from oracle import masks as OM
from oracle import scores as OS
from tests.gpu_util import announce, dev, dev_i32, dev_u8, host
from tests.selection_rules import check_selection
from workloads import WAN480_CUBE, LONG126, make_qkv

pytestmark = pytest.mark.gpu


def assert_scores_close(got, ref, what):
    d = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert d.max() <= 1e-4, f"{what}: score error {d.max():.2e}"


@pytest.mark.parametrize("N,bs,D,H", [(1000, 128, 128, 2), (700, 64, 128, 3), (333, 64, 64, 2)])
def test_block_scores_ragged(N, bs, D, H):
    announce(f"scores N={N} bs={bs} D={D}")
    rng = np.random.default_rng(N)
    qd = dev(rng.standard_normal((1, H, N, D)) + 0.3)
    kd = dev(rng.standard_normal((1, H, N, D)) - 0.2)
    S, qp, kp = V.vsa_block_scores(qd, kd, bs)
    rS, rq, rk = OS.block_scores(host(qd), host(kd), bs)
    assert np.abs(host(qp) - rq).max() <= 1e-5 and np.abs(host(kp) - rk).max() <= 1e-5
    assert_scores_close(host(S), rS, "ragged")


def test_block_scores_cube_layout_blk_len():
    w = WAN480_CUBE
    announce("scores cube layout wan 12 heads")
    q, k, _ = make_qkv(w)
    qc, kc = OL.permute(q, w.grid, "cube4"), OL.permute(k, w.grid, "cube4")
    _, counts, _ = OL.cube_map(*w.grid, 4)
    S, qp, kp = V.vsa_block_scores(dev(qc), dev(kc), 64, blk_len=dev_i32(counts))
    rS, rq, rk = OS.block_scores(qc, kc, 64, counts)
    assert np.abs(host(qp) - rq).max() <= 1e-5
    assert_scores_close(host(S), rS, "cube")


# nkb spans every register width of the one-wave kernel (4 ... 64 keys per lane,
# 4096 = the largest row); a quantum of 1000 makes every score of a row equal,
# so the order comes from the indices alone
@pytest.mark.parametrize("nkb,k_max,top_p,quant", [(10, 3, 1.0, 0.5), (10, 10, 0.6, None), (624, 93, 0.9, None),
                                                   (624, 93, 0.5, None), (300, 40, 1.0, 0.25), (1536, 154, 1.0, None),
                                                   (2048, 200, 0.95, None), (1, 1, 1.0, None), (5, 2, 0.3, 1.0),
                                                   (1000, 100, 0.9, None), (3000, 300, 0.8, None),
                                                   (4096, 4096, 0.5, None), (4096, 1, 1.0, 0.25),
                                                   (624, 93, 0.9, 1000.0), (1536, 154, 1.0, 1000.0)])
def test_select_topk_random_rows(nkb, k_max, top_p, quant):
    announce(f"select nkb={nkb} k={k_max} p={top_p}")
    rng = np.random.default_rng(nkb + k_max)
    S = (rng.standard_normal((1, 2, 24, nkb)) * 2.0).astype(np.float32)
    if quant:
        S = (np.round(S / quant) * quant).astype(np.float32)       # many exact ties
    Sd = torch.from_numpy(S).cuda()
    idx, cnt = V.vsa_select_topk(Sd, k_max, top_p)
    n, exact, bad = check_selection(S, None, k_max, top_p, host(idx), host(cnt))
    assert not bad, f"{len(bad)} rows outside the gap rule, e.g. {bad[:3]}"


def test_select_with_forced_local_window():
    announce("select forced local window nkb=300")
    grid, bs = (150, 4, 8), 16           # 300 blocks of half a frame; a +-1 frame window forces 4-6
    forced = OM.pattern_mask(grid, bs, "spatial", 1)
    nb = forced.shape[0]
    assert nb == 300 and forced.sum(1).max() < 30
    rng = np.random.default_rng(3)
    S = rng.standard_normal((1, 2, nb, nb)).astype(np.float32)
    idx, cnt = V.vsa_select_topk(torch.from_numpy(S).cuda(), 30, 1.0, forced=dev_u8(forced))
    gi, gc = host(idx), host(cnt)
    assert (gc == 30).all()
    n, exact, bad = check_selection(S, forced, 30, 1.0, gi, gc)
    assert not bad
    # every forced block is present
    sel = OM.list_to_mask(gi, gc, nb)
    assert (sel[..., forced == 1] == 1).all()
    # more forced blocks than room: the best-scoring forced blocks, capped
    idx, cnt = V.vsa_select_topk(torch.from_numpy(S).cuda(), 3, 1.0, forced=dev_u8(forced))
    n, exact, bad = check_selection(S, forced, 3, 1.0, host(idx), host(cnt))
    assert not bad


def test_cube_pipeline_selection_full_shape():
    """Wan 480p cube workload: pooled scores on the GPU, top-p 0.9 capped at 93
    of 624 cubes; the selection is checked against the oracle on those scores
    and on the oracle's own fp64 scores (gap rule)."""
    w = WAN480_CUBE
    announce("select cube wan full")
    q, k, _ = make_qkv(w)
    qc, kc = OL.permute(q, w.grid, "cube4"), OL.permute(k, w.grid, "cube4")
    _, counts, _ = OL.cube_map(*w.grid, 4)
    S, _, _ = V.vsa_block_scores(dev(qc), dev(kc), 64, blk_len=dev_i32(counts))
    k_max = int(np.floor(w.extra["k_frac"] * counts.size))
    assert k_max == 93
    idx, cnt = V.vsa_select_topk(S, k_max, w.extra["top_p"])
    gi, gc = host(idx), host(cnt)
    n, exact, bad = check_selection(host(S), None, k_max, w.extra["top_p"], gi, gc)
    assert not bad
    rS, _, _ = OS.block_scores(qc, kc, 64, counts)
    n, exact, bad = check_selection(rS, None, k_max, w.extra["top_p"], gi, gc)
    assert not bad, f"{len(bad)} of {n} rows differ from the fp64 selection beyond the gap rule"
    # with mean scale 0.5 the 15 % cap binds on most rows
    assert (gc == 93).mean() > 0.5


def test_long_horizon_selection_full_shape():
    w = LONG126
    H = 4
    announce("select long horizon")
    q, k, _ = make_qkv(w, H=H)
    S, _, _ = V.vsa_block_scores(dev(q), dev(k), w.bs)
    forced = OM.pattern_mask(w.grid, w.bs, "spatial", 1)
    k_total = int(round(w.extra["density"] * w.nb))
    idx, cnt = V.vsa_select_topk(S, k_total, 1.0, forced=dev_u8(forced))
    gi, gc = host(idx), host(cnt)
    assert (gc == k_total).all()
    rS, _, _ = OS.block_scores(q, k, w.bs)
    assert_scores_close(host(S), rS, "long")
    n, exact, bad = check_selection(rS, forced, k_total, 1.0, gi, gc)
    assert not bad, f"{len(bad)} of {n} rows beyond the gap rule"
