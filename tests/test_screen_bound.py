"""The lower bounds that let the binary32 screen skip chunks of scales, checked by brute force.

For a chunk of consecutive binary16 scales [s_lo, s_hi] the screen bounds each environment's
objective F_e(s) = sum_i d_ei (w_i - s q_i(s))^2 from below by Z + C, where Z sums d w^2 over the
weights whose clip key (w/6.5 for w > 0, |w|/7.5 otherwise) is at most s_lo/15 (code 0 at every
scale >= s_lo), and C sums d (|w| - |q| s_hi)^2 over the weights whose clip key exceeds s_hi (code 7
or -8 at every scale <= s_hi) where that difference is positive.  Z does not decrease for later
chunks and bounds them too; C does not increase for later chunks and bounds every earlier one.
These tests evaluate every objective exactly (binary64, the definition's codes) at every pattern
up to the first scale >= 2 max|w| and check all three statements on seeded groups, including
groups whose optimum lies far from max|w|/7.  Parity of the screen itself is checked on the GPU.
"""
import numpy as np
import pytest

import workloads as W

CHUNK = 128
GRID = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


def _objectives(w, d, top):
    """F[e, k] at pattern k + 1, k < top: codes clip(rne(w/s), -8, 7), binary64."""
    s = GRID[:top]
    q = np.clip(np.rint(w[None, :] / s[:, None]), -8, 7)
    r2 = (w[None, :] - s[:, None] * q) ** 2            # [top, 128]
    return d @ r2.T                                     # [E, top]


def _bounds(w, d, lo, hi):
    a = np.abs(w)
    key = np.where(w > 0, w / 6.5, a / 7.5)
    qa = np.where(w > 0, 7.0, 8.0)
    z = d @ np.where(key <= lo / 15.0, a * a, 0.0)
    t = np.where(key > hi, np.maximum(0.0, a - qa * hi), 0.0)
    c = d @ (t * t)
    return z, c


def _groups():
    rng = np.random.default_rng(5)
    out = []
    w1, d1, p1 = W.matrix_groups(*W.make_matrix(1, 0))
    for g in rng.choice(w1.shape[0], 6, replace=False):
        out.append((w1[g].astype(np.float64), d1[g % p1].astype(np.float64)))
    x = rng.normal(0, 0.01, 128)
    x[9] = 1.0
    dd = rng.lognormal(0, 0.5, (4, 128))
    dd[:, 9] = 1e-6
    out.append((x, dd))                                 # optimum clips the large weight
    x = rng.normal(0, 0.02, 128)
    x[50] = 0.75
    dd = np.full((4, 128), 1e-6)
    dd[:, 50] = 1.0
    out.append((x, dd))                                 # optimum above max|w|/7
    x = np.zeros(128)
    x[3] = -0.3
    out.append((x, rng.lognormal(0, 1, (2, 128))))      # a lone weight
    out.append((rng.standard_t(3, 128) * 0.02, rng.lognormal(0, 1, (8, 128))))
    return out


@pytest.mark.parametrize("j", range(10))
def test_chunk_bounds_hold_at_every_scale(j):
    w, d = _groups()[j]
    top = int(np.searchsorted(GRID, 2.0 * np.abs(w).max(), side="left")) + 1
    F = _objectives(w, d, top)
    nch = (top - 1) // CHUNK + 1
    zs, cs, mins = [], [], []
    for c in range(nch):
        k0, k1 = c * CHUNK, min(c * CHUNK + CHUNK, top)
        z, cc = _bounds(w, d, GRID[k0], GRID[k1 - 1])
        fmin = F[:, k0:k1].min(axis=1)
        assert np.all(z + cc <= fmin * (1 + 1e-12)), c
        zs.append(z); cs.append(cc); mins.append(fmin)
    zs, cs, mins = np.array(zs), np.array(cs), np.array(mins)   # [nch, E]
    for c in range(nch):
        # Z of chunk c bounds every later chunk, C of chunk c every earlier one
        assert np.all(zs[c][None, :] <= mins[c:] * (1 + 1e-12)), c
        assert np.all(cs[c][None, :] <= mins[:c + 1] * (1 + 1e-12)), c
    # the bound is informative: on typical groups most chunks are skippable against the optimum
    opt = F.max(axis=0).min()
    skippable = ((zs + cs).max(axis=1) > 1.001 * opt).mean()
    if j < 6:
        assert skippable > 0.5


@pytest.mark.parametrize("j", range(10))
def test_candidate_window_drops_only_scales_above_the_probe(j):
    """The candidate solver ignores every scale s <= lo, lo = max_i (|w_i| - sqrt(1.0001 U /
    max_e d_ei)) / |q_i| (q_i = 7 for w_i > 0, else -8), with U = max_e F_e at s_a = binary16(
    max|w|/9).  Below |w_i|/|q_i| weight i is clipped with residual |w_i| - |q_i| s, so every such
    scale has max_e F_e > 1.0001 U (checked exactly here at every pattern), and the optimum, at
    most U, lies above lo."""
    w, d = _groups()[j]
    a = np.abs(w)
    if a.max() == 0:
        return
    top = int(np.searchsorted(GRID, 2.0 * a.max(), side="left")) + 1
    F = _objectives(w, d, top).max(axis=0)
    sa = float(np.float16(a.max() / 9))
    qa_code = np.clip(np.rint(w / sa), -8, 7)
    U = (d @ ((w - sa * qa_code) ** 2)).max()
    qa = np.where(w > 0, 7.0, 8.0)
    dm = d.max(axis=0)
    lo = np.where(dm > 0, (a - np.sqrt(1.0001 * U / np.where(dm > 0, dm, 1.0))) / qa, -np.inf).max()
    below = GRID[:top] <= lo
    assert np.all(F[below] > 1.0001 * U * (1 - 1e-12))
    assert GRID[int(np.argmin(F))] > lo
    if j < 6:
        assert below.sum() > 0.4 * top  # on typical groups most of the grid is ruled out
