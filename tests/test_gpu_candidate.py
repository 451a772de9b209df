"""GPU parity of the candidate-set solver: against the oracle, and against the exhaustive sweep
at full size (the pages' solver-versus-exhaustive cross-check, CliffQuant README "Verification")."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import bits_np, check_minimax, dev, say, threads

pytestmark = pytest.mark.gpu


def _both(w, d, p):
    wt, dt = dev(w), dev(d)
    c = cq.quantize_groups(wt, dt, p, method="candidate")
    x = cq.quantize_groups(wt, dt, p, method="exhaustive")
    torch.cuda.synchronize()
    return c, x


def _agree(c, x, label):
    """Candidate and exhaustive pick the same scale, codes and objective on every group."""
    cb, xb = bits_np(c["scales"]), bits_np(x["scales"])
    co, xo = c["objective"].cpu().numpy(), x["objective"].cpu().numpy()
    diff = np.nonzero(cb != xb)[0]
    if diff.size:
        rel = np.abs(co[diff] - xo[diff]) / np.maximum(xo[diff], 1e-300)
        assert np.all(rel <= 1e-9), f"{label}: {diff.size} scale mismatches, worst objective gap {rel.max()}"
    same = cb == xb
    np.testing.assert_array_equal(co[same], xo[same])
    np.testing.assert_array_equal(c["codes"].cpu().numpy()[same], x["codes"].cpu().numpy()[same])
    flags = c["flags"].cpu().numpy()
    say(f"  {label}: {cb.size} groups, {diff.size} scale mismatches, "
        f"{int(np.count_nonzero(flags & cq.FLAG_FALLBACK))} handed to the exhaustive sweep")
    return flags


def test_candidate_config0_vs_oracle():
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    c, x = _both(w, d, p)
    sol = oracle.solve(w, d, p, n_threads=threads())
    check_minimax(w, d, p, c, sol)
    _agree(c, x, "config 0")


def test_candidate_pages_example():
    w, d = W.pages_example()
    sol = oracle.solve(w, d)
    scale, obj, codes = cq.solve_breakpoint_exact([0.9, -0.4, 0.2, -1.1],
                                                  [[1.0, 0.8, 0.5, 1.2], [0.6, 1.4, 0.9, 0.7]])
    assert scale == oracle.fp16_value(sol.mm_bits[0]) and obj == sol.mm_F1[0]
    assert codes == list(sol.codes[0, :4])


def test_candidate_matches_exhaustive_config1_full():
    """All 86,016 groups of config 1; the oracle checks a seeded sample of 96."""
    gids = W.sample_groups(1, 96, salt=3)
    m_idx, local = W.locate(1, gids)
    for m, mat in enumerate(W.config(1).matrices):
        w, d, p = W.matrix_groups(*W.make_matrix(1, m))
        c, x = _both(w, d, p)
        _agree(c, x, f"config 1 {mat.name}")
        sel = local[m_idx == m]
        ws, ds = w[sel], d[sel % p]
        sol = oracle.solve(ws, ds, ds.shape[0], n_threads=threads())
        sub = {k: (v[torch.from_numpy(sel).cuda()] if v is not None else None) for k, v in c.items()}
        check_minimax(ws, ds, ds.shape[0], sub, sol)


def test_candidate_config3_stress_sample():
    """Edge and tie stress (E=8, per-group diagonals): 48 groups of each category."""
    cats = W.config3_categories()
    rng = np.random.default_rng(2)
    idx = np.sort(np.concatenate([rng.choice(np.nonzero(cats == k)[0], 48, replace=False) for k in range(5)]))
    w, d, cat, ce = W.make_groups(3, idx)
    n = idx.size
    c, x = _both(w, d, n)
    flags = _agree(c, x, "config 3 sample")
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, c, sol)
    bits = bits_np(c["scales"])
    z = cat == W.CAT_ZERO
    assert np.all(bits[z] == 1)
    pt = cat == W.CAT_PAIR_TIE
    want = np.array([int(np.float16(W.pair_tie_unit(int(k)) / 2).view(np.uint16)) for k in ce[pt]])
    np.testing.assert_array_equal(bits[pt], want)
    assert np.all(flags[z | pt] & cq.FLAG_FALLBACK)   # exact ties go to the exhaustive check


def test_candidate_config4_sample_e16():
    gids = W.sample_groups(4, 48, salt=1)
    w, d, _ = W.gather_matrix_groups(4, gids)
    n = w.shape[0]
    c, x = _both(w, d, n)
    _agree(c, x, "config 4 sample")
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, c, sol)


def test_candidate_config2_matrices():
    """Two full matrices of config 2 (25,888 and 25,696 groups) against the exhaustive sweep."""
    for m in (0, 149):
        w, d, p = W.matrix_groups(*W.make_matrix(2, m))
        c, x = _both(w, d, p)
        _agree(c, x, f"config 2 matrix {m}")


def test_candidate_odd_env_counts():
    """E = 3 and E = 5 run padded kernels; the pick must not change."""
    rng = np.random.default_rng(9)
    for E in (1, 3, 5):
        w = W.round_bf16(rng.normal(0, 0.02, (24, 128)).astype(np.float32))
        d = rng.lognormal(0, 1, (24, E, 128)).astype(np.float32)
        c, x = _both(w, d, 24)
        sol = oracle.solve(w, d, 24, n_threads=threads())
        check_minimax(w, d, 24, c, sol)
        check_minimax(w, d, 24, x, sol)


def test_many_fallbacks_take_both_list_paths():
    """More tie groups than the sliced list path serves (256): all-zero and symmetric-pair
    groups mixed with ordinary ones; every group must still match the exhaustive sweep."""
    rng = np.random.default_rng(21)
    n = 900
    w = W.round_bf16(rng.normal(0, 0.02, (n, 128)).astype(np.float32))
    d = rng.lognormal(0, 1, (n, 4, 128)).astype(np.float32)
    zero = rng.random(n) < 0.4
    w[zero] = 0.0
    pairs = (~zero) & (rng.random(n) < 0.3)
    for j in np.nonzero(pairs)[0]:
        c = 2.0 ** -int(rng.integers(5, 11))
        mult = np.array([1, 2, 3] + list(rng.integers(1, 4, 61)), np.float64)
        w[j] = rng.permutation(np.concatenate([mult * c, -mult * c])).astype(np.float32)
        d[j, 1] = d[j, 0]
    c, x = _both(w, d, n)
    flags = _agree(c, x, "fallback mix")
    assert np.count_nonzero(flags & cq.FLAG_FALLBACK) > 256
    bits = bits_np(c["scales"])
    assert np.all(bits[zero] == 1)
    sel = np.nonzero(~zero)[0][:40]
    sol = oracle.solve(w[sel], d[sel], sel.size, n_threads=threads())
    sub = {k: (v[torch.from_numpy(sel).cuda()] if v is not None else None) for k, v in c.items()}
    check_minimax(w[sel], d[sel], sel.size, sub, sol)


def test_candidate_subnormal_scales():
    """Groups whose optimum lies among the subnormal binary16 scales (max|w| from 1e-7 to 1e-4,
    so that max|w|/7 < 2^-14) or straddles the smallest normal one, against the oracle and the
    full grid: the transition search converts patterns to values and back in that range."""
    rng = np.random.default_rng(33)
    n = 64
    mag = 10.0 ** rng.uniform(-7, -4, n)
    w = (rng.normal(0, 1, (n, 128)) * mag[:, None] * np.where(rng.random((n, 128)) < 0.03, 6.0, 1.0)).astype(np.float32)
    d = rng.lognormal(0, 1, (n, 4, 128)).astype(np.float32)
    c, x = _both(w, d, n)
    _agree(c, x, "subnormal scales")
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, c, sol)
    assert np.count_nonzero(bits_np(c["scales"]) < 0x0400) > n // 4
