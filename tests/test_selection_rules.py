"""The gap rule used to accept fp32 selections must excuse only near-boundary
differences. CPU only."""
import numpy as np

from oracle.select import select_row
from tests.selection_rules import row_matches


def test_exact_match_accepted_and_clear_mismatch_rejected():
    s = np.array([3.0, 1.0, 2.0, 0.0, -1.0])
    assert row_matches(s, None, 2, 1.0, [0, 2])
    assert not row_matches(s, None, 2, 1.0, [0, 1])
    assert not row_matches(s, None, 2, 1.0, [0])


def test_near_tie_at_the_boundary_is_excused():
    s = np.array([3.0, 1.00002, 1.0, 0.0])
    assert select_row(s, None, 2, 1.0).tolist() == [0, 1]
    assert row_matches(s, None, 2, 1.0, [0, 2])            # 1.0 vs 1.00002: within 1e-4
    s2 = np.array([3.0, 1.001, 1.0, 0.0])
    assert not row_matches(s2, None, 2, 1.0, [0, 2])       # gap 1e-3: not excused


def test_top_p_count_off_by_one_only_at_the_mass_boundary():
    p = np.array([0.5, 0.4, 0.05, 0.05])
    s = np.log(p)
    # cumsum 0.5, 0.9, ... ; top_p 0.90003 keeps 3 in fp64, fp32 may stop at 2
    assert select_row(s, None, 4, 0.90003).tolist() == [0, 1, 2]
    assert row_matches(s, None, 4, 0.90003, [0, 1])
    # far from the boundary a different count is an error
    assert not row_matches(s, None, 4, 0.7, [0])
    assert not row_matches(s, None, 4, 0.7, [0, 1, 2])


def test_forced_blocks_must_be_present():
    s = np.array([0.0, 5.0, 4.0, 3.0])
    f = np.array([1, 0, 0, 0])
    assert row_matches(s, f, 2, 1.0, [0, 1])
    assert not row_matches(s, f, 2, 1.0, [1, 2])
