"""The binary32 screen of the full-grid search and its error bound, checked on the CPU.

The full grid forms, for every scale, each environment's error in binary32 from weights and scales
pre-scaled by the same power of two: x = RN(w' r) with r the reciprocal of s' (within one binary32
rounding), q = rint(x) clipped, e = fma(-s', q, w'), then e^2 and the environment's running fma.
Its exactness argument bounds that value against the definition's:
    (1 - (G+3) u) F  <=  F~ / 2^(2k)  <=  (1 + (G+3) u)(1 + 16.001 u X) F,   u = 2^-24,
X = max(-qmin, qmax) + 1/2, and the pooled sum meets E - 1 more roundings.  Every pattern within
the ratio of these bounds of the smallest screened value is rescored in binary64, so the answer
is exact as long as the bound holds.  Here the same binary32 operations run in numpy (every
operation rounded once, the fmas through binary64, where the products are exact) on seeded
groups, including outlier, tiny, clipped and short groups and other code ranges, at scales spread
over the whole grid; the values must sit inside the bound around the oracle's binary64 errors,
and a zero screened value must mean a zero error."""
import numpy as np
import pytest

import oracle
import workloads as W

U = 2.0 ** -24
GRID = np.arange(1, 0x7C00, dtype=np.uint16)


def _fma32(a, b, c):
    # a * b is exact in binary64 (24 x 24 bits); the sum is rounded once to binary32 unless it
    # also needs more than binary64's 53 bits, which the bound's margin covers
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _screen(w, d, bits, qmin, qmax):
    """Binary32 screen values (minimax, pooled) of groups w [n, G] with d [n, E, G] at one scale
    pattern per group, as the full grid forms them, on the pre-scaled values."""
    n, G = w.shape
    E = d.shape[1]
    wmax = np.max(np.abs(w), axis=1).astype(np.float64)
    ex = np.frexp(np.where(wmax > 0, wmax, 1.0))[1]
    k = np.where(wmax > 0, np.clip(1 - ex, -100, 100), 0)
    pk = (2.0 ** k).astype(np.float32)
    wp = (w * pk[:, None]).astype(np.float32)
    sp = (np.asarray(bits, np.uint16).view(np.float16).astype(np.float32) * pk).astype(np.float32)
    r = (np.float32(1.0) / sp).astype(np.float32)           # a correctly rounded reciprocal
    x = (wp * r[:, None]).astype(np.float32)
    q = np.clip(np.rint(x), qmin, qmax).astype(np.float32)
    e = _fma32(np.broadcast_to(-sp[:, None], (n, G)), q, wp)
    e2 = (e * e).astype(np.float32)
    acc = np.zeros((n, E), np.float32)
    for i in range(G):
        acc = _fma32(d[:, :, i], np.broadcast_to(e2[:, i, None], (n, E)), acc)
    scale = pk.astype(np.float64) ** 2
    F = acc.max(axis=1).astype(np.float64) / scale
    p = acc[:, 0].copy()
    for j in range(1, E):
        p = (p + acc[:, j]).astype(np.float32)
    return F, p.astype(np.float64) / scale


def _groups(kind, n, G, E, rng):
    w = rng.normal(0, 0.02, (n, G))
    if kind == "outliers":
        w *= np.where(rng.random((n, G)) < 0.03, 8.0, 1.0)
    elif kind == "tiny":
        w *= 1e-3
    elif kind == "zeros":
        w[:, ::3] = 0.0
    w = W.round_bf16(w.astype(np.float32))
    d = rng.lognormal(0, 1, (n, E, G)).astype(np.float32)
    return w, d


CASES = [("outliers", 128, 4, -8, 7), ("plain", 128, 4, -8, 7), ("tiny", 128, 4, -8, 7), ("zeros", 128, 8, -8, 7),
         ("outliers", 64, 3, -4, 3), ("plain", 32, 2, -2, 1), ("outliers", 256, 4, -128, 127), ("plain", 100, 5, 0, 15)]


@pytest.mark.parametrize("kind,G,E,qmin,qmax", CASES, ids=[f"{c[0]}_G{c[1]}_E{c[2]}_q{c[3]}..{c[4]}" for c in CASES])
def test_screen_values_sit_inside_the_bound(kind, G, E, qmin, qmax):
    rng = np.random.default_rng(hash((kind, G, E, qmin)) & 0xFFFF)
    n = 8
    w, d = _groups(kind, n, G, E, rng)
    X = max(-qmin, qmax) + 0.5
    lo = 1 - (G + 3) * U
    hi = (1 + (G + 3) * U) * (1 + 16.001 * U * X)
    lo_p = 1 - (G + 3 + E - 1) * U
    hi_p = (1 + (G + 3 + E - 1) * U) * (1 + 16.001 * U * X)
    # every scale of the grid (clipped, unclipped and all-zero-code ones), in seven interleaved parts
    for b0 in range(7):
        pats = GRID[b0::7]
        ww = np.repeat(w, pats.size, axis=0)
        dd = np.repeat(d, pats.size, axis=0)
        bits = np.tile(pats, n)
        Fe = oracle.env_errors(ww, dd, bits, ww.shape[0], 0, qmin, qmax)
        F = Fe.max(axis=1)
        Pe = Fe.sum(axis=1)
        Ft, Pt = _screen(ww, dd, bits, qmin, qmax)
        assert np.all(Ft >= lo * F * (1 - 1e-15)), "screened minimax value below its bound"
        assert np.all(Ft <= hi * F * (1 + 1e-15)), "screened minimax value above its bound"
        assert np.all(Pt >= lo_p * Pe * (1 - 1e-15)), "screened pooled sum below its bound"
        assert np.all(Pt <= hi_p * Pe * (1 + 1e-15)), "screened pooled sum above its bound"
        assert np.array_equal(Ft == 0, F == 0), "a zero screened value must mean a zero error"


def test_code_flips_near_half_integers_stay_inside_the_bound():
    """Weights placed within a few binary32 spacings of (k + 1/2) s for one scale s, where the
    screen's rounded quotient can pick the neighbouring code: the term then grows by at most the
    factor 1 + 16.001 u X, which the bound carries."""
    rng = np.random.default_rng(77)
    G, E, qmin, qmax = 128, 4, -8, 7
    X = max(-qmin, qmax) + 0.5
    lo, hi = 1 - (G + 3) * U, (1 + (G + 3) * U) * (1 + 16.001 * U * X)
    flips = 0
    for b in rng.integers(0x1800, 0x2C00, 12):
        b = int(b) | 1  # an odd significand: 1/s is not a binary32 number
        s = float(np.uint16(b).view(np.float16))
        k = rng.integers(-8, 8, (16, G)).astype(np.float64)
        eps = rng.uniform(-2, 2, (16, G)) * U
        w = ((k + 0.5) * s * (1 + eps)).astype(np.float32)
        d = rng.lognormal(0, 1, (16, E, G)).astype(np.float32)
        bits = np.full(16, b, np.uint16)
        Fe = oracle.env_errors(w, d, bits, 16)
        F = Fe.max(axis=1)
        Ft, _ = _screen(w, d, bits, qmin, qmax)
        assert np.all(Ft >= lo * F * (1 - 1e-15)) and np.all(Ft <= hi * F * (1 + 1e-15))
        # how often the screen's code differs from the definition's here (the case the factor covers)
        sp = np.float32(s)
        xs = (w * (np.float32(1.0) / sp)).astype(np.float32)
        flips += int(np.count_nonzero(np.clip(np.rint(xs), qmin, qmax) != oracle.codes_for(w, bits)))
    assert flips > 0, "no code flip was constructed; the case does not exercise the factor"
