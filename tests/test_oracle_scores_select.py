"""Pins for oracle.scores and oracle.select: closed forms, invariants, hand-worked
top-p cases and brute-force subset enumeration. CPU only."""
import itertools
import math

import numpy as np
import pytest

from oracle import scores as S
from oracle import select as SEL


def test_constant_blocks_pool_to_the_constant():
    bs, D, nb = 16, 4, 5
    vals = np.random.default_rng(0).standard_normal((1, 2, nb, D))
    x = np.repeat(vals, bs, axis=2)[:, :, :70]            # ragged last block of 6
    p = S.block_means(x, bs)
    assert np.abs(p - vals).max() <= 1e-15


def test_pool_brute_force_loops_and_blk_len():
    bs, D = 4, 3
    blk_len = np.array([4, 1, 3])
    x = np.random.default_rng(1).standard_normal((1, 1, 12, D))
    p = S.block_means(x, bs, blk_len)
    for b in range(3):
        for d in range(D):
            ref = sum(x[0, 0, b * bs + r, d] for r in range(blk_len[b])) / blk_len[b]
            assert abs(p[0, 0, b, d] - ref) <= 1e-15


def test_scores_linear_and_symmetric():
    bs = 8
    q = np.random.default_rng(2).standard_normal((1, 2, 40, 6))
    k = np.random.default_rng(3).standard_normal((1, 2, 40, 6))
    s1 = S.block_scores(q, k, bs)[0]
    s2 = S.block_scores(2.0 * q, k, bs)[0]
    assert np.abs(s2 - 2 * s1).max() <= 1e-14
    sq = S.block_scores(q, q, bs)[0]
    assert np.abs(sq - np.swapaxes(sq, -1, -2)).max() == 0
    # closed form for one entry, written out
    qm = q[0, 1, 8:16].mean(0)
    km = k[0, 1, 32:40].mean(0)
    assert abs(s1[0, 1, 1, 4] - float(qm @ km) / math.sqrt(6)) <= 1e-14


def test_top_p_hand_cases():
    """p = softmax(ln[.5,.3,.15,.05]) = [.5,.3,.15,.05]; cumulative .5,.8,.95,1."""
    s = np.log([0.5, 0.3, 0.15, 0.05])
    assert SEL.select_row(s, None, 4, 0.9).tolist() == [0, 1, 2]
    assert SEL.select_row(s, None, 4, 0.4).tolist() == [0]
    assert SEL.select_row(s, None, 4, 0.7).tolist() == [0, 1]
    assert SEL.select_row(s, None, 2, 0.9).tolist() == [0, 1]    # cap binds
    assert SEL.select_row(s[::-1], None, 4, 0.9).tolist() == [1, 2, 3]
    assert SEL.select_row(s, None, 4, 1.0).tolist() == [0, 1, 2, 3]   # top-p off


def test_ties_go_to_the_lower_index_and_output_is_ascending():
    s = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 0.0])
    assert SEL.select_row(s, None, 3, 1.0).tolist() == [1, 2, 3]
    assert SEL.select_row(s, None, 4, 1.0).tolist() == [1, 2, 3, 4]
    assert SEL.select_row(np.zeros(7), None, 3, 1.0).tolist() == [0, 1, 2]


def test_forced_blocks_are_kept_and_outrank_others():
    s = np.array([5.0, -1.0, 4.0, -2.0, 3.0])
    f = np.array([0, 1, 0, 1, 0])
    assert SEL.select_row(s, f, 3, 1.0).tolist() == [0, 1, 3]
    assert SEL.select_row(s, f, 4, 1.0).tolist() == [0, 1, 2, 3]
    assert SEL.select_row(s, f, 1, 1.0).tolist() == [1]          # more forced than room: best forced
    assert SEL.select_row(s, f, 2, 1.0).tolist() == [1, 3]


def brute_topk(s, k):
    """Every subset of size k; the max-sum one, lexicographically smallest on ties."""
    best, best_set = None, None
    for c in itertools.combinations(range(len(s)), k):
        tot = sum(s[j] for j in c)
        if best is None or tot > best + 1e-12:
            best, best_set = tot, c
    return list(best_set)


@pytest.mark.parametrize("seed", range(12))
def test_top_k_matches_subset_enumeration(seed):
    r = np.random.default_rng(seed)
    nkb = int(r.integers(2, 11))
    s = np.round(r.standard_normal(nkb), 1)          # rounding creates ties
    k = int(r.integers(1, nkb + 1))
    assert SEL.select_row(s, None, k, 1.0).tolist() == brute_topk(s, k)


@pytest.mark.parametrize("seed", range(8))
def test_top_p_keeps_the_shortest_prefix_reaching_p(seed):
    """Top-p by enumeration: among subsets in rank order, the first prefix whose
    probability mass reaches p, checked against a direct scan."""
    r = np.random.default_rng(100 + seed)
    nkb = 9
    s = r.standard_normal(nkb) * 2
    p = np.exp(s) / np.exp(s).sum()
    top_p = float(r.uniform(0.3, 0.95))
    got = SEL.select_row(s, None, nkb, top_p)
    mass = p[got].sum()
    assert mass >= top_p
    # removing the least probable kept block drops below top_p (shortest prefix)
    assert mass - p[got].min() < top_p
    # every kept block is at least as probable as every dropped one
    dropped = np.setdiff1d(np.arange(nkb), got)
    if dropped.size:
        assert p[got].min() >= p[dropped].max()


def test_select_batched_shapes_and_padding():
    s = np.random.default_rng(5).standard_normal((1, 2, 4, 6))
    idx, cnt = SEL.select(s, None, 3, 1.0)
    assert idx.shape == (1, 2, 4, 3) and (cnt == 3).all()
    idx, cnt = SEL.select(s, None, 5, 0.5)
    assert ((cnt >= 1) & (cnt <= 5)).all()
    for i, c in zip(idx.reshape(-1, 5), cnt.reshape(-1)):
        assert (i[c:] == -1).all() and (np.diff(i[:c]) > 0).all()
