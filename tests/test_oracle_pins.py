"""Pins on the CPU oracle: what the pages and the mathematics fix, independent of the oracle.

Each test names the fact it checks.  None of them re-types the oracle's own
formula: they use closed forms, library routines (numpy's float16), exact
rational arithmetic, invariances and hand-computed values.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import exact_rational as X
import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _grid_values():
    return np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- P1: admissible set
def test_fp16_grid_matches_ieee_binary16():
    """Every positive finite binary16 value, decoded by the oracle, equals numpy's decoding;
    31,743 of them, strictly increasing in bit order, from 2^-24 to 65504."""
    g = json.load(open(os.path.join(GOLDEN, "fp16_grid.json")))
    vals = np.array([oracle.fp16_value(b) for b in range(g["first_bits"], g["last_bits"] + 1)])
    assert vals.size == g["count"] == oracle.N_SCALES
    np.testing.assert_array_equal(vals, _grid_values())
    assert np.all(np.diff(vals) > 0)
    assert vals[0] == g["first_value"] == 2.0 ** -24 and vals[-1] == g["last_value"]
    assert oracle.fp16_value(g["smallest_normal_bits"]) == g["smallest_normal_value"]


def test_fp16_round_matches_numpy():
    """Nearest binary16 with ties to even (oracle) equals numpy's float32 -> float16 cast."""
    xs = np.concatenate([
        RNG.lognormal(-3, 4, 3000).astype(np.float32),
        # exact midpoints between neighbours, subnormal and normal, and the overflow edge
        ((_grid_values()[:-1] + _grid_values()[1:]) / 2)[::97].astype(np.float32),
        np.array([0.0, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 65504, 65519.99, 65520, 1e9],
                 dtype=np.float32)])
    for x in xs:
        with np.errstate(over="ignore"):
            ref = int(np.float32(x).astype(np.float16).view(np.uint16))
        assert oracle.fp16_round(x) == ref, x


# ---------------------------------------------------------------- P7: the code function
def test_codes_match_exact_rational():
    """q = clip(round-half-even(w/s), -8, 7) with an fp32 quotient equals the exact-rational
    rule, on random pairs and on constructed exact half-integer quotients."""
    bits = RNG.integers(1, 0x7C00, 400)
    for b in bits:
        s = Fraction(float(np.uint16(b).view(np.float16)))
        # weights near every half-integer m*s, exactly on it, and random
        mids = [(m + Fraction(1, 2)) * s for m in range(-9, 9)]
        ws = [float(np.float32(float(v))) for v in mids]
        ws += list(RNG.normal(0, 10 * float(s), 20).astype(np.float32))
        w32 = np.array(ws, dtype=np.float32)
        got = oracle.codes_at(w32, int(b))
        want = [X.code(Fraction(float(x)), s) for x in w32]
        assert list(got) == want, hex(b)


def test_code_rounding_and_clipping_cases():
    """Round half to even first, then clip: 2.5->2, 3.5->4, -0.5->0, 6.5->6, 7.5->7 (8 clipped),
    -7.5->-8, -8.5->-8, 100->7, -100->-8 (scale 1.0 is binary16 0x3C00)."""
    w = np.array([2.5, 3.5, -0.5, 0.5, 6.5, 7.5, -7.5, -8.5, 100.0, -100.0, 0.0], np.float32)
    assert list(oracle.codes_at(w, 0x3C00)) == [2, 4, 0, 0, 6, 7, -8, -8, 7, -8, 0]


def test_codes_monotone_in_scale():
    """q_i(s) is monotone in s with at most 7 change points (w > 0) or 8 (w < 0); in the
    subnormal range one step of the grid can move a code by more than one."""
    ws = np.concatenate([RNG.normal(0, 0.05, 6), [1e-6, -1e-6, 3000.0, -3000.0]]).astype(np.float32)
    allq = np.stack([oracle.codes_at(ws, b) for b in range(1, 0x7C00)], axis=1)  # [n, 31743]
    for w, q in zip(ws, allq):
        dq = np.diff(q.astype(np.int64))
        if w > 0:
            assert np.all(dq <= 0) and q[0] == 7 and np.count_nonzero(dq) <= 7
        else:
            assert np.all(dq >= 0) and q[0] == -8 and np.count_nonzero(dq) <= 8
        assert q[-1] == 0 or abs(w) > 1000.0


# ---------------------------------------------------------------- P2: exact brute force
def _tiny_group(ws, ds):
    w = np.zeros((1, 128), np.float32)
    d = np.zeros((1, len(ds), 128), np.float32)
    w[0, :len(ws)] = ws
    d[0, :, :len(ws)] = ds
    return w, d


def _check_against_exact(ws, ds, qmin=-8, qmax=7, G=128, pos=None):
    """The oracle on the group zero-padded to G (weights at positions `pos`, default the first
    ones) against the exact brute force: minimax and pooled argmin bits where the exact runner-up
    gap exceeds 1e-12, and both minima to binary64 rounding."""
    ex = X.solve(ws, ds, qmin, qmax)
    pos = list(range(len(ws))) if pos is None else list(pos)
    w = np.zeros((1, G), np.float32)
    d = np.zeros((1, len(ds), G), np.float32)
    w[0, pos] = ws
    d[0][:, pos] = np.asarray(ds, np.float32)
    # diagonals of the zero weights are arbitrary: a zero weight adds 0 at every scale
    d[0][:, [i for i in range(G) if i not in pos]] = 3.0
    r = oracle.solve(w, d, qmin=qmin, qmax=qmax)
    for name, bits, v1, v2, got_bits, got_v1 in (
            ("minimax", ex.mm_bits, ex.F1, ex.F2, r.mm_bits[0], r.mm_F1[0]),
            ("pooled", ex.pl_bits, ex.P1, ex.P2, r.pl_bits[0], r.pl_P1[0])):
        exact_gap = float((v2 - v1) / v1) if v1 else (0.0 if v2 == 0 else np.inf)
        if exact_gap > 1e-12:
            assert int(got_bits) == bits, name
        assert got_v1 == pytest.approx(float(v1), rel=1e-13, abs=0), name
    return ex


def test_pages_example_matches_exact_rational():
    """The README's four-weight, two-environment example: oracle argmin == exact argmin, for the
    minimax and the pooled policy (which differ here: 0x31E8 and 0x31E0)."""
    g = json.load(open(os.path.join(GOLDEN, "pages_example.json")))
    w, d = workloads.pages_example()
    assert np.array_equal(w[0, :4], np.float32(g["weights"]))
    assert np.array_equal(d[0, :, :4], np.float32(g["environment_diagonals"]))
    ex = _check_against_exact(g["weights"], g["environment_diagonals"])
    assert ex.mm_bits != ex.pl_bits


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_tiny_groups_match_exact_rational(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 5))
    E = int(rng.integers(1, 4))
    ws = workloads.round_bf16(rng.normal(0, 0.05, n).astype(np.float32))
    ds = rng.lognormal(0, 1, (E, n)).astype(np.float32)
    _check_against_exact(list(ws), ds.tolist())


def test_pooled_policy_matches_exact_rational_with_three_environments():
    """Pooled objective pinned where it differs from every single environment's choice: three
    environments that each weigh a different weight, so the average's argmin is none of the
    per-environment argmins and a pooled sum that drops or misweighs an environment picks
    another scale."""
    ws = [0.8125, -0.296875, 0.1484375]
    ds = [[4.0, 0.25, 0.5], [0.25, 4.0, 0.5], [0.5, 0.25, 4.0]]
    ex = _check_against_exact(ws, ds)
    singles = {X.solve(ws, [row]).mm_bits for row in ds}
    assert ex.pl_bits not in singles


# ---------------------------------------------------------------- other quantizer ranges and lengths
@pytest.mark.parametrize("qmin,qmax,G,pos", [
    (-4, 3, 64, (0, 21, 40, 63)),        # signed 3-bit, groups of 64
    (-2, 1, 32, (3, 17, 31)),            # signed 2-bit, groups of 32
    (-128, 127, 256, (5, 129, 200, 255)),  # signed 8-bit, groups of 256 (weights past index 128)
    (0, 15, 128, (1, 64, 127)),          # unsigned 4-bit: negative weights take code 0
])
def test_quantizer_spec_matches_exact_rational(qmin, qmax, G, pos):
    """The README's solver takes a quantizer specification (qmin, qmax) and a group of any length
    (its example has four weights).  Tiny groups placed at scattered positions of longer groups,
    two environments: oracle against the exact brute force with the same code range."""
    rng = np.random.default_rng(qmax * 1000 + G)
    ws = workloads.round_bf16(rng.normal(0, 0.05, len(pos)).astype(np.float32))
    ws[0] = abs(ws[0]) * 3
    ds = rng.lognormal(0, 1, (2, len(pos))).astype(np.float32)
    _check_against_exact(list(ws), ds.tolist(), qmin, qmax, G, pos)


def test_groups_of_other_lengths_are_laid_out_back_to_back():
    """Three groups of 64 weights in one call, [n_groups][64] and diagonals [n_groups][E][64]: an
    all-zero group (pattern 0x0001), then single weights whose winners are known in closed form
    (the smallest binary16 scale at which the weight is an admissible code exactly)."""
    G = 64
    w = np.zeros((3, G), np.float32)
    w[1, 10] = 0.75
    w[2, 60] = -0.3125
    d = np.ones((3, 2, G), np.float32)
    r = oracle.solve(w, d, qmin=-4, qmax=3)
    assert r.mm_bits[0] == 0x0001
    # 0.75 = 3 * 0.25 (code 3, the largest); -0.3125 = -4 * 0.078125 (code -4, the smallest)
    assert r.mm_bits[1] == int(np.float16(0.25).view(np.uint16))
    assert r.mm_bits[2] == int(np.float16(0.078125).view(np.uint16))
    assert r.mm_F1[1] == 0.0 and r.mm_F1[2] == 0.0
    assert list(r.codes[1, 9:12]) == [0, 3, 0] and r.codes[2, 60] == -4


def test_code_range_cases():
    """Round half to even first, then clip to the range: at scale 1, [-2, 1] maps 1.5 -> 2 -> 1,
    -2.5 -> -2, -3 -> -2; [0, 15] maps every negative weight to 0 and 15.5 -> 16 -> 15;
    [-128, 127] maps 126.5 -> 126, 127.5 -> 128 -> 127, -128.5 -> -128."""
    w = np.array([1.5, -2.5, -3.0, 0.5], np.float32)
    assert list(oracle.codes_at(w, 0x3C00, -2, 1)) == [1, -2, -2, 0]
    w = np.array([-0.75, -100.0, 15.5, 14.5, 2.5], np.float32)
    assert list(oracle.codes_at(w, 0x3C00, 0, 15)) == [0, 0, 15, 14, 2]
    w = np.array([126.5, 127.5, -128.5, -127.5], np.float32)
    assert list(oracle.codes_at(w, 0x3C00, -128, 127)) == [126, 127, -128, -128]


# ---------------------------------------------------------------- P3: E=1 closed form
def _bracket(s):
    g = _grid_values()
    j = np.searchsorted(g, s)
    return {int(k) + 1 for k in (j - 1, j) if 0 <= k < g.size}


@pytest.mark.parametrize("seed", range(4))
def test_single_env_closed_form(seed):
    """E=1: with codes frozen at the winner's codes q*, the objective is the quadratic
    sum d (w - s q*)^2 whose minimiser is s* = sum d w q* / sum d q*^2; the winning scale
    must be a grid neighbour of s*."""
    rng = np.random.default_rng(100 + seed)
    w = workloads.round_bf16(rng.normal(0, 0.02, (4, 128)).astype(np.float32))
    d = rng.lognormal(0, 1, (4, 1, 128)).astype(np.float32)
    r = oracle.solve(w, d)
    for g in range(4):
        q = oracle.codes_at(w[g], int(r.mm_bits[g])).astype(np.float64)
        dd, ww = d[g, 0].astype(np.float64), w[g].astype(np.float64)
        s_star = (dd * ww * q).sum() / (dd * q * q).sum()
        assert int(r.mm_bits[g]) in _bracket(s_star) or r.mm_gap[g] < 1e-12


def test_winner_is_local_min_of_frozen_code_envelope():
    """General E: F(s) <= max_e sum d_e (w - s q*)^2 for every s, with equality at the winner;
    so the winner's grid neighbours cannot be better under frozen codes (exact arithmetic)."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    r = oracle.solve(w[:3], d, p)
    for g in range(3):
        b = int(r.mm_bits[g])
        ws = [Fraction(float(x)) for x in w[g]]
        ds = [[Fraction(float(x)) for x in row] for row in d[g % p]]
        qs = [int(v) for v in oracle.codes_at(w[g], b)]

        def frozen(bits):
            s = Fraction(float(np.uint16(bits).view(np.float16)))
            return max(sum(dd * (x - s * q) ** 2 for x, dd, q in zip(ws, de, qs)) for de in ds)
        f0 = frozen(b)
        assert float(f0) == pytest.approx(r.mm_F1[g], rel=1e-13)
        for nb in (b - 1, b + 1):
            assert frozen(nb) >= f0 * (1 - Fraction(1, 10 ** 12))


def test_single_environment_pooled_equals_minimax_bit_for_bit():
    """E = 1: P(s) = F_0(s) / 1 = F(s) exactly, so both policies pick the same pattern with the
    same minimum and runner-up, bit for bit."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    r = oracle.solve(w[:12], d[:, 1:2], p, n_threads=8)
    np.testing.assert_array_equal(r.pl_bits, r.mm_bits)
    np.testing.assert_array_equal(r.pl_P1, r.mm_F1)
    np.testing.assert_array_equal(r.pl_P2, r.mm_F2)


def test_pooled_policy_is_minimax_on_the_mean_diagonal():
    """sum_e F_e(s) / E is the single-environment objective with the mean diagonal (1/E) sum_e d_e,
    exactly in real arithmetic.  The mean diagonal rounded to binary32 moves the objective by at
    most 2^-24 relative, so wherever both gaps exceed 1e-6 the pooled pick equals the E = 1
    minimax pick on the mean diagonal, and its objective matches to 1e-6."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w = w[:24]
    dbar = d.astype(np.float64).mean(axis=1, keepdims=True).astype(np.float32)
    a = oracle.solve(w, d, p, n_threads=8)
    b = oracle.solve(w, dbar, p, n_threads=8)
    sure = (a.pl_gap > 1e-6) & (b.mm_gap > 1e-6)
    assert sure.sum() >= 12
    np.testing.assert_array_equal(a.pl_bits[sure], b.mm_bits[sure])
    np.testing.assert_allclose(a.pl_P1, b.mm_F1, rtol=1e-6)
    assert np.any(a.pl_bits != a.mm_bits)  # the pooled policy differs from the minimax one here


# ---------------------------------------------------------------- P4: dominance
def test_dominance_over_baselines():
    """minimax F <= F at the AbsMax and pooled scales; pooled P <= P at the minimax scale."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w = w[:24]
    r = oracle.solve(w, d, p, n_threads=8)
    ab = oracle.absmax_bits(w)
    F_ab = oracle.objective(w, d, ab, p)
    F_pl = oracle.objective(w, d, r.pl_bits, p)
    assert np.all(r.mm_F1 <= F_ab) and np.all(r.mm_F1 <= F_pl)
    assert np.all(oracle.objective(w, d, r.mm_bits, p) == r.mm_F1)
    Fe_mm = oracle.env_errors(w, d, r.mm_bits, p)
    P_mm = np.array([sum(row[1:], row[0]) for row in Fe_mm]) / d.shape[1]
    assert np.all(r.pl_P1 <= P_mm)
    assert np.any(r.mm_bits != ab)  # the policies do differ


# ---------------------------------------------------------------- P5: constructed ties
def test_all_zero_group_takes_lowest_pattern():
    w = np.zeros((1, 128), np.float32)
    d = np.ones((1, 3, 128), np.float32)
    r = oracle.solve(w, d)
    assert r.mm_bits[0] == 0x0001 and r.mm_F1[0] == 0.0 and r.mm_F2[0] == 0.0
    assert r.pl_bits[0] == 0x0001 and np.all(r.codes == 0)


@pytest.mark.parametrize("c_exp", [5, 7, 10])
def test_symmetric_pair_tie_takes_half_unit(c_exp):
    """Weights +-c*n (n in {1,2,3}, each present): F = 0 exactly at s = c and s = c/2 only,
    so the lower pattern, c/2 = 2^-(k+1), wins with an exact zero tie."""
    c = 2.0 ** -c_exp
    mult = np.array([1, 2, 3] + [1, 2, 3, 2] * 15 + [3], np.float64)  # 64 multiples
    w = np.concatenate([mult * c, -mult * c]).astype(np.float32)[None, :]
    d = RNG.lognormal(0, 1, (1, 4, 128)).astype(np.float32)
    d[0, 1] = d[0, 0]
    r = oracle.solve(w, d)
    half = int(np.float16(c / 2).view(np.uint16))
    assert int(r.mm_bits[0]) == half and r.mm_F1[0] == 0.0 and r.mm_F2[0] == 0.0
    F, _ = oracle.curve(w[0], d[0])
    assert set(np.nonzero(F == 0.0)[0] + 1) == {half, int(np.float16(c).view(np.uint16))}


@pytest.mark.parametrize("wv", [0.75, -0.75, 0.3125, -1.5, 3.0, 2.0 ** -20])
def test_single_weight_takes_smallest_exact_scale(wv):
    """One nonzero weight: F = 0 exactly where w/s is an integer code; the smallest such
    binary16 s (largest admissible |code|) wins."""
    w = np.zeros((1, 128), np.float32)
    w[0, 5] = wv
    d = np.ones((1, 2, 128), np.float32)
    r = oracle.solve(w, d)
    W = Fraction(float(np.float32(wv)))
    qs = range(1, 8) if wv > 0 else range(-8, 0)
    exact = []
    for q in qs:
        s = W / q
        h = np.float16(float(s))
        if np.isfinite(h) and h > 0 and Fraction(float(h)) == s:
            exact.append(int(h.view(np.uint16)))
    assert int(r.mm_bits[0]) == min(exact) and r.mm_F1[0] == 0.0


def _top_pattern(w):
    """Smallest pattern whose binary16 value is >= 2 max|w|, or None when 2 max|w| > 65504."""
    grid = _grid_values()
    t = 2.0 * float(np.max(np.abs(w.astype(np.float64))))
    j = int(np.searchsorted(grid, t, side="left"))
    return None if j == grid.size else j + 1


@pytest.mark.parametrize("case", ["config0", "large", "subnormal"])
def test_scales_above_twice_max_weight_tie_exactly(case):
    """From the first scale >= 2 max|w| on, |w/s| <= 1/2 rounds every code to 0, so the
    objective is max_e sum_i d w^2 (the pooled one its mean) at every larger pattern, bitwise
    the same value: the lower-bit-pattern rule never picks a pattern above that first one.
    The exhaustive sweep stops there."""
    if case == "config0":
        w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
        groups = [(w[g], d[g % p]) for g in (0, 17, 100)]
    elif case == "large":   # 2 max|w| = 3e4 lies inside the grid's last binade
        rng = np.random.default_rng(4)
        w = rng.normal(0, 2000, 128).astype(np.float32)
        w[3] = 15000.0
        groups = [(w, rng.lognormal(0, 1, (3, 128)).astype(np.float32))]
    else:                   # 2 max|w| inside the subnormal range
        rng = np.random.default_rng(5)
        w = (rng.uniform(-1, 1, 128) * 1e-6).astype(np.float32)
        groups = [(w, rng.lognormal(0, 1, (2, 128)).astype(np.float32))]
    for wg, dg in groups:
        bt = _top_pattern(wg)
        assert bt is not None
        F, P = oracle.curve(wg, dg)
        assert np.all(F[bt - 1:] == F[bt - 1]) and np.all(P[bt - 1:] == P[bt - 1])
        # closed form of the all-zero-code objective
        w64 = wg.astype(np.float64)
        Fe = [math.fsum(float(x) for x in dg[e].astype(np.float64) * w64 * w64) for e in range(dg.shape[0])]
        assert F[bt - 1] == pytest.approx(max(Fe), rel=1e-13)
        assert np.all(oracle.codes_at(wg, bt) == 0)
        assert bt == 1 or np.any(oracle.codes_at(wg, bt - 1) != 0)
        r = oracle.solve(wg[None, :], dg[None, :])
        assert int(r.mm_bits[0]) <= bt and int(r.pl_bits[0]) <= bt


def test_no_top_pattern_when_twice_max_weight_exceeds_the_grid():
    """2 max|w| > 65504: no binary16 scale zeroes every code and the sweep covers the grid."""
    w = np.zeros(128, np.float32)
    w[0] = 40000.0
    assert _top_pattern(w) is None
    assert np.any(oracle.codes_at(w, 0x7BFF) != 0)


# ---------------------------------------------------------------- P6: invariances
def test_environment_invariances():
    """Permuting, duplicating or adding a pointwise-dominated environment, and scaling every
    diagonal by 2^k, leave the minimax pick unchanged bit for bit."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w, d = w[:6], d[np.arange(6) % p]
    base = oracle.solve(w, d)
    variants = [d[:, ::-1], np.concatenate([d, d[:, :1]], axis=1),
                np.concatenate([d, d[:, 2:3] * np.float32(0.5)], axis=1),
                d * np.float32(2.0 ** 7), d * np.float32(2.0 ** -9)]
    for dv in variants:
        r = oracle.solve(w, np.ascontiguousarray(dv))
        np.testing.assert_array_equal(r.mm_bits, base.mm_bits)


def test_weight_power_of_two_scaling_shifts_exponent():
    """w -> 2w maps the winning scale s -> 2s exactly (binary16 exponent + 1 = bits + 0x400)."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w, d = w[:6], d[np.arange(6) % p]
    a = oracle.solve(w, d)
    b = oracle.solve(w * np.float32(2.0), d)
    np.testing.assert_array_equal(b.mm_bits.astype(np.int64), a.mm_bits.astype(np.int64) + 0x400)
    np.testing.assert_array_equal(b.mm_F1, a.mm_F1 * 4.0)


def test_weight_permutation_invariance():
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w, d = w[:6], d[np.arange(6) % p]
    perm = RNG.permutation(128)
    a = oracle.solve(w, d)
    b = oracle.solve(w[:, perm], d[:, :, perm])
    sure = a.mm_gap > 1e-9
    np.testing.assert_array_equal(a.mm_bits[sure], b.mm_bits[sure])
    np.testing.assert_allclose(b.mm_F1, a.mm_F1, rtol=1e-13)


# ---------------------------------------------------------------- AbsMax
def test_absmax_policy_cases():
    """fp16(fl32(max|w|/7)) by numpy's cast; zero group -> 0x0001; overflow -> 0x7BFF."""
    w = np.zeros((5, 128), np.float32)
    w[0, 3] = -0.7
    w[1, :] = RNG.normal(0, 0.02, 128).astype(np.float32)
    w[3, 0] = 1e6
    w[4, 9] = 1e-9
    got = oracle.absmax_bits(w)
    for g in (0, 1):
        m = np.float32(np.abs(w[g]).max())
        assert got[g] == int((m / np.float32(7)).astype(np.float16).view(np.uint16))
    assert got[2] == 0x0001 and got[3] == 0x7BFF and got[4] == 0x0001
    # another code range: the largest magnitude maps to the largest positive code, max|w| / qmax
    for qmax in (1, 3, 127):
        got = oracle.absmax_bits(w[:2], qmax=qmax)
        m = np.float32(np.abs(w[1]).max())
        assert got[1] == int((m / np.float32(qmax)).astype(np.float16).view(np.uint16))
        assert got[0] == int((np.float32(0.7) / np.float32(qmax)).astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------- GPTQ-v1 packing
def test_pack_hand_values():
    """Nibble j of qweight[r, o] holds code[o, 8r+j] + 8 (low nibble first); scales transpose."""
    out, inp = 3, 256
    codes = np.tile((np.arange(inp) % 8 - 8).astype(np.int8), (out, 1))
    codes[1] = -8
    codes[2] = 7
    sb = np.arange(out * 2, dtype=np.uint16).reshape(out, 2) + 0x3C00
    qw, sc = oracle.pack_gptq_v1(codes, sb, out, inp)
    assert qw.shape == (32, 3) and qw.dtype == np.int32
    assert np.all(qw[:, 0].view(np.uint32) == 0x76543210)
    assert np.all(qw[:, 1] == 0) and np.all(qw[:, 2] == -1)
    assert sc.shape == (2, 3) and sc[1, 2] == 0x3C05


def test_pack_round_trip():
    out, inp = 16, 384
    codes = RNG.integers(-8, 8, (out, inp)).astype(np.int8)
    sb = RNG.integers(1, 0x7C00, (out, inp // 128)).astype(np.uint16)
    c2, s2 = oracle.unpack_gptq_v1(*oracle.pack_gptq_v1(codes, sb, out, inp))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, sb)


@pytest.mark.parametrize("bits", [2, 8])
def test_pack_other_widths_hand_values_and_round_trip(bits):
    """bits = 2: sixteen 2-bit fields per int32, value code + 2; bits = 8: four bytes, code + 128;
    low field first, transposed to [in * bits / 32, out]."""
    per, zero = 32 // bits, 1 << (bits - 1)
    out, inp = 2, 128
    codes = np.zeros((out, inp), np.int8)
    codes[0] = (np.arange(inp) % per) % (1 << bits) - zero
    codes[1] = -zero
    sb = np.array([[0x3C00], [0x3C01]], np.uint16)
    qw, sc = oracle.pack_gptq_v1(codes, sb, out, inp, bits=bits)
    assert qw.shape == (inp // per, out)
    want0 = sum(((j % (1 << bits)) << (bits * j)) for j in range(per)) & 0xFFFFFFFF
    assert np.all(qw[:, 0].view(np.uint32) == want0) and np.all(qw[:, 1] == 0)
    assert list(sc[:, 1]) == [0x3C01]
    rng = np.random.default_rng(bits)
    codes = rng.integers(-zero, zero, (8, 256)).astype(np.int8)
    sb = rng.integers(1, 0x7C00, (8, 4)).astype(np.uint16)
    c2, s2 = oracle.unpack_gptq_v1(*oracle.pack_gptq_v1(codes, sb, 8, 256, bits=bits, group=64), bits=bits)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, sb)


# ---------------------------------------------------------------- proxy
def test_proxy_hand_values():
    """w = 0.375 at s = 0.25: q = round-half-even(1.5) = 2, error -0.125, squared 1/64.
    Diagonals 1 and 2 give per-env errors 1/64 and 2/64; worst env / 128 = 1/4096."""
    w = np.zeros((3, 128), np.float32)
    w[0, 0] = 0.375
    w[1, 0] = 0.375
    w[2, 7] = 0.375
    d = np.zeros((1, 2, 128), np.float32)
    d[0, 0, :] = 1.0
    d[0, 1, :] = 2.0
    bits = np.full(3, int(np.float16(0.25).view(np.uint16)), np.uint16)
    per, mod, macro = oracle.proxy(w, d, bits, [0, 1, 1], 2, d_period=1)
    assert list(per) == [1 / 4096] * 3
    assert list(mod) == [1 / 4096, 1 / 4096] and macro == 1 / 4096
    w[2, 7] = 0.0
    per, mod, macro = oracle.proxy(w, d, bits, [0, 1, 1], 2, d_period=1)
    assert list(mod) == [1 / 4096, 1 / 8192] and macro == (1 / 4096 + 1 / 8192) / 2


def test_proxy_divides_by_the_group_length_and_empty_module_is_nan():
    """Groups of 64: w = 0.375 at s = 0.25 gives error 1/64 per unit diagonal, so with diagonals 1
    and 2 the worst environment's mean square is (2/64)/64 = 1/2048.  A module with no groups has
    no mean (NaN), and neither has the macro over modules."""
    w = np.zeros((2, 64), np.float32)
    w[:, 0] = 0.375
    d = np.zeros((1, 2, 64), np.float32)
    d[0, 0, :] = 1.0
    d[0, 1, :] = 2.0
    bits = np.full(2, int(np.float16(0.25).view(np.uint16)), np.uint16)
    per, mod, macro = oracle.proxy(w, d, bits, [0, 2], 3, d_period=1)
    assert list(per) == [1 / 2048] * 2
    assert mod[0] == 1 / 2048 and np.isnan(mod[1]) and mod[2] == 1 / 2048
    assert np.isnan(macro)


def test_minimax_proxy_not_worse_than_baselines_on_calibration_diagonals():
    """With the calibration diagonals as d_eval, every group's minimax proxy is <= both baselines."""
    w, d, p = workloads.matrix_groups(*workloads.make_matrix(0, 0))
    w = w[:16]
    r = oracle.solve(w, d, p, n_threads=8)
    mods = np.zeros(16, np.int64)
    pm = oracle.proxy(w, d, r.mm_bits, mods, 1, p)[0]
    pa = oracle.proxy(w, d, oracle.absmax_bits(w), mods, 1, p)[0]
    pp = oracle.proxy(w, d, r.pl_bits, mods, 1, p)[0]
    assert np.all(pm <= pa) and np.all(pm <= pp)


def test_binary32_quotient_decides_like_exact_rational_near_every_half_integer():
    """For every binary16 scale s and half-integer h in 0.5..8.5, weights 1-3 binary32 ulps either
    side of h*s: round-half-even of the binary32 quotient equals the exact decision."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    s = bits.view(np.float16).astype(np.float32)
    for h2 in range(1, 18, 2):
        hs = (s * np.float32(h2 / 2)).astype(np.float32)
        for k in (1, 2, 3):
            for direction in (np.inf, -np.inf):
                w = hs.copy()
                for _ in range(k):
                    w = np.nextafter(w, np.float32(direction))
                got = np.array([oracle.codes_at(w[j:j + 1], int(bits[j]))[0] for j in range(0, w.size, 997)])
                below = (w.astype(np.float64) < hs.astype(np.float64))[::997]
                want = np.clip(np.where(below, h2 // 2, h2 // 2 + 1), -8, 7)
                np.testing.assert_array_equal(got, want)
