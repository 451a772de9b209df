"""Pins of the oracle's held-out comparison (oracle.heldout_compare) against values the pages
print and values the definition fixes by hand, so that a dropped term, a swapped policy, a wrong
sign or an off-by-one in the resampling or the percentile fails one of them."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "heldout_proxy.json")


def test_pages_effect_is_pooled_minus_minimax_and_counts_cover_the_sample():
    """The printed effect is the pooled macro minus the minimax macro (same sign, 4 digits), the
    relative results are those macros' ratios, and wins + ties + losses is the sample size.  A
    two-group version of the same data gives the oracle's sign and direction."""
    g = json.load(open(GOLD))
    assert round(g["macro_pooled"] - g["macro_minimax"], 9) == pytest.approx(g["effect_vs_pooled"], abs=5e-10)
    assert g["effect_ci95"][0] < g["effect_vs_pooled"] < g["effect_ci95"][1]
    assert g["wins"] + g["ties"] + g["losses"] == g["groups"]
    assert round(100 * (1 - g["macro_minimax"] / g["macro_pooled"]), 2) == g["relative_vs_pooled_percent"]
    assert round(100 * (1 - g["macro_minimax"] / g["macro_absmax"]), 1) == g["relative_vs_absmax_percent"]
    # one module per policy value: the oracle's effect is B - A with A the minimax policy
    counts, eff, _, _ = oracle.heldout_compare([g["macro_minimax"]], [g["macro_pooled"]], [0, 1],
                                               np.zeros((0, 1), np.int32))
    assert eff == g["macro_pooled"] - g["macro_minimax"]
    assert list(counts) == [1, 0, 0]


def test_hand_example():
    pa = np.array([1.0, 2.0, 3.0, 4.0])
    pb = np.array([1.0, 3.0, 2.0, 5.0])
    off = np.array([0, 2, 4])
    idx = np.array([[0, 1, 2, 3], [1, 1, 3, 3]], np.int32)
    counts, eff, reps, (lo, hi) = oracle.heldout_compare(pa, pb, off, idx)
    assert list(counts) == [2, 1, 1]          # wins (2 < 3, 4 < 5), tie (1 == 1), loss (3 > 2)
    assert eff == 0.25                          # modules: mean(0, 1) = 0.5, mean(-1, 1) = 0
    assert list(reps) == [0.25, 1.0]            # identity draw; all-second draws (1, 1), (1, 1)
    assert lo == 0.25 + 0.75 * 0.025 and hi == 0.25 + 0.75 * 0.975


def test_macro_weights_modules_not_groups():
    """A module of one group counts as much as a module of three."""
    pa = np.zeros(4)
    pb = np.array([4.0, 0.0, 0.0, 0.0])
    _, eff, _, _ = oracle.heldout_compare(pa, pb, [0, 1, 4], np.zeros((0, 4), np.int32))
    assert eff == 2.0                           # (4 + 0) / 2, not 4 / 4


def test_identity_draws_reproduce_the_point_effect():
    rng = np.random.default_rng(3)
    off = np.array([0, 5, 12, 13, 30])
    pa, pb = rng.random(30), rng.random(30)
    idx = np.tile(np.arange(30, dtype=np.int32), (7, 1))
    _, eff, reps, (lo, hi) = oracle.heldout_compare(pa, pb, off, idx)
    assert np.all(reps == eff) and lo == eff and hi == eff


def test_constant_difference_is_exact():
    """Every difference 2^-5 in power-of-two modules: every sum is exact, so every replicate and
    both bounds are 2^-5 bit for bit."""
    off = np.array([0, 4, 8, 16])
    pa = np.linspace(0, 1, 16)
    pb = pa + 2.0 ** -5
    pb = pa + (pb - pa)  # the difference as stored
    diff = pb - pa
    assert np.all(diff == diff[0])
    idx = W.bootstrap_indices(off, 50, seed=1)
    _, eff, reps, (lo, hi) = oracle.heldout_compare(pa, pb, off, idx)
    assert eff == diff[0] and np.all(reps == diff[0]) and lo == diff[0] and hi == diff[0]


def test_single_group_modules_have_no_resampling_spread():
    rng = np.random.default_rng(4)
    pa, pb = rng.random(6), rng.random(6)
    off = np.arange(7)
    idx = W.bootstrap_indices(off, 20, seed=2)
    assert np.all(idx == np.arange(6))          # each module can only draw its own group
    _, eff, reps, _ = oracle.heldout_compare(pa, pb, off, idx)
    assert np.all(reps == eff)


def test_percentile_positions_on_known_replicates():
    """One module of n groups with differences 0..n-1; replicate r draws group r throughout, so its
    effect is r.  Replicates 0..B-1 in shuffled order: the bounds are q (B-1) exactly."""
    n = B = 41
    pa = np.zeros(n)
    pb = np.arange(n, dtype=np.float64)
    perm = np.random.default_rng(5).permutation(B)
    idx = np.repeat(perm[:, None], n, axis=1).astype(np.int32)
    _, _, reps, (lo, hi) = oracle.heldout_compare(pa, pb, [0, n], idx, alpha=0.1)
    assert list(reps) == list(range(B))
    assert lo == pytest.approx(0.05 * 40, abs=1e-12) and hi == pytest.approx(0.95 * 40, abs=1e-12)


def test_swapping_the_policies_flips_everything():
    rng = np.random.default_rng(6)
    off = np.array([0, 9, 20])
    pa, pb = rng.random(20), rng.random(20)
    pb[3] = pa[3]
    idx = W.bootstrap_indices(off, 33, seed=3)
    c1, e1, r1, (l1, h1) = oracle.heldout_compare(pa, pb, off, idx)
    c2, e2, r2, (l2, h2) = oracle.heldout_compare(pb, pa, off, idx)
    assert list(c1) == [c2[2], c2[1], c2[0]] and c1[1] == 1
    assert e1 == -e2 and np.all(r1 == -r2[::-1])
    assert l1 == pytest.approx(-h2, abs=1e-15) and h1 == pytest.approx(-l2, abs=1e-15)


def test_bad_draws_and_empty_modules_give_nan():
    pa, pb = np.zeros(4), np.ones(4)
    idx = np.array([[0, 1, 2, 3], [2, 1, 2, 3]], np.int32)  # replicate 1 draws group 2 for module 0
    _, eff, reps, (lo, hi) = oracle.heldout_compare(pa, pb, [0, 2, 4], idx)
    assert eff == 1.0 and reps[0] == 1.0 and np.isnan(reps[1]) and np.isnan(lo) and np.isnan(hi)
    _, eff, _, _ = oracle.heldout_compare(pa, pb, [0, 2, 2, 4], idx)
    assert np.isnan(eff)


def test_bootstrap_indices_stay_in_their_module_and_cover_it():
    off = np.array([0, 3, 3, 10, 11])
    idx = W.bootstrap_indices(off, 2000, seed=4)
    for m in range(4):
        lo, hi = off[m], off[m + 1]
        blk = idx[:, lo:hi]
        assert np.all((blk >= lo) & (blk < hi))
        if hi > lo:
            assert set(np.unique(blk)) == set(range(lo, hi))
