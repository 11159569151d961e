"""Hand-derived golden cases (tests/golden/) and the planted-outlier property of
the long-horizon generator. CPU only."""
import os

import numpy as np

from oracle import layout as L
from oracle import masks as M
from oracle import scores as S
from oracle import select as SEL
from workloads import LONG126, make_qkv, outlier_blocks

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_frame_major_golden():
    pi = L.frame_major_map(4, 8, 8)
    rows = np.loadtxt(os.path.join(GOLD, "frame_major_4x8x8.txt"), dtype=np.int64)
    for t, y, x, n, fm in rows:
        assert n == 64 * t + 8 * y + x
        assert pi[n] == fm


def test_top_p_golden():
    for line in open(os.path.join(GOLD, "top_p_cases.txt")):
        if line.startswith("#") or not line.strip():
            continue
        probs, top_p, k_max, kept = [f.strip() for f in line.split("|")]
        s = np.log(np.array([float(x) for x in probs.split(",")]))
        got = SEL.select_row(s, None, int(k_max), float(top_p))
        assert got.tolist() == [int(x) for x in kept.split(",")], line


def test_long_horizon_outliers_are_selected_everywhere():
    """Long-horizon generator: the planted outlier key blocks score about +3 logits
    above the rest, so with a local window forced and a 10 % budget every outlier
    block that is not already local is selected by every query block (two heads)."""
    w = LONG126
    q, k, _ = make_qkv(w, H=2)
    Sc = S.block_scores(q, k, w.bs)[0]
    forced = M.pattern_mask(w.grid, w.bs, "spatial", w.extra["w_local"])
    k_total = int(round(w.extra["density"] * w.nb))
    assert k_total == 154
    idx, cnt = SEL.select(Sc, forced, k_total, 1.0)
    outl = outlier_blocks(w)
    assert outl.size == 46
    sel = M.list_to_mask(idx, cnt, w.nb)
    for h in range(2):
        for qb in range(w.nb):
            need = outl[forced[qb, outl] == 0]
            assert sel[0, h, qb, need].all()
