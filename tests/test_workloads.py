"""The seeded synthetic inputs: shapes, determinism and the structure each config promises."""
import numpy as np
import torch

import oracle
import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).normal(0, 0.05, 100000).astype(np.float32)
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0]  # exact ties to even
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(W.round_bf16(x), ref)


def test_config_sizes():
    assert W.config(0).n_groups == 128
    assert W.config(1).n_groups == 86016
    assert W.config(2).n_groups == 3883008
    assert W.config(2).n_groups * 128 == 497025024
    assert W.config(3).n_groups == 262144
    assert W.config(4).n_groups == 1048576
    assert [W.config(k).E for k in range(5)] == [4, 4, 4, 8, 16]


def test_matrix_layout_and_determinism():
    A, da = W.make_matrix(0, 0)
    B, db = W.make_matrix(0, 0)
    assert A.shape == (64, 256) and da.shape == (4, 256)
    np.testing.assert_array_equal(A, B)
    np.testing.assert_array_equal(da, db)
    np.testing.assert_array_equal(W.round_bf16(A), A)         # bf16-valued
    np.testing.assert_allclose(da.astype(np.float64).mean(axis=1), 1.0, rtol=1e-6)
    w, d, p = W.matrix_groups(A, da)
    assert w.shape == (128, 128) and d.shape == (2, 4, 128) and p == 2
    g = 5 * 2 + 1                                             # row 5, second input chunk
    np.testing.assert_array_equal(w[g], A[5, 128:256])
    np.testing.assert_array_equal(d[g % p], da[:, 128:256])
    frac_out = np.mean(np.abs(A) > 0.08)
    assert 0.005 < frac_out < 0.03                            # ~1% outliers x8 (plus 4-sigma tail)


def test_gather_matches_matrix():
    gids = np.array([0, 127, 28672, 86015])
    w, d, m = W.gather_matrix_groups(1, gids)
    assert list(m) == [0, 0, 1, 2]
    A, da = W.make_matrix(1, 2)
    wg, dg, p = W.matrix_groups(A, da)
    np.testing.assert_array_equal(w[3], wg[-1])
    np.testing.assert_array_equal(d[3], dg[(wg.shape[0] - 1) % p])


def test_config3_categories_and_structure():
    cats = W.config3_categories()
    assert np.bincount(cats).tolist() == [104858, 52429, 26214, 26214, 52429]
    idx = np.arange(0, 262144, 2053)
    w, d, c, ce = W.make_groups(3, idx)
    for j in range(idx.size):
        if c[j] == W.CAT_ZERO:
            assert not np.any(w[j])
        elif c[j] == W.CAT_TINY:
            assert np.all(np.abs(w[j]) < 1e-5)
        elif c[j] == W.CAT_PAIR_TIE:
            u = W.pair_tie_unit(int(ce[j]))
            assert set(np.unique(np.abs(w[j]) / u)) == {1.0, 2.0, 3.0}
            np.testing.assert_array_equal(np.sort(w[j]), np.sort(-w[j]))
            np.testing.assert_array_equal(d[j, 0::2], d[j, 1::2])
        elif c[j] == W.CAT_ONE_CHANNEL:
            zero_rows = [e for e in range(8) if np.count_nonzero(d[j, e]) == 1]
            assert len(zero_rows) == 1 and d[j, zero_rows[0]].max() == 128.0
    # chunks regenerate identically when asked for alone
    w2, d2, _, _ = W.make_groups(3, idx[5:7])
    np.testing.assert_array_equal(w2, w[5:7])
    np.testing.assert_array_equal(d2, d[5:7])


def test_pair_tie_groups_have_exact_zero_ties():
    """A generated symmetric-pair group: the oracle picks c/2 with an exact zero tie."""
    cats = W.config3_categories()
    j = int(np.nonzero(cats == W.CAT_PAIR_TIE)[0][0])
    w, d, _, ce = W.make_groups(3, [j])
    r = oracle.solve(w, d)
    half = int(np.float16(W.pair_tie_unit(int(ce[0])) / 2).view(np.uint16))
    assert r.mm_bits[0] == half and r.mm_F1[0] == 0.0 and r.mm_F2[0] == 0.0


def test_config4_diagonal_permutation_structure():
    A, dm = W.make_matrix(4, 0)
    assert A.shape == (4096, 4096) and dm.shape == (16, 4096)
    # each env is a renormalised copy of one base row with 410 channels permuted
    same = np.isclose(dm[0] / dm[0].mean(), dm[1] / dm[1].mean(), rtol=1e-5)
    assert 4096 - 2 * 410 <= same.sum() <= 4096


def test_heldout_inputs_are_seeded_and_laid_out_by_module():
    a = W.heldout_sample(0, 50)
    b = W.heldout_sample(0, 50)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    w, d, de, off = a
    n = w.shape[0]
    assert d.shape == de.shape == (n, 4, 128) and d.dtype == de.dtype == np.float32
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) > 0)
    # held-out diagonals share the calibration base but not its perturbation
    assert not np.array_equal(d, de)
    r = np.log(de.astype(np.float64) / d.astype(np.float64))
    assert abs(float(np.median(r))) < 0.3 and float(np.std(r)) > 0.3


def test_bootstrap_indices_are_seeded():
    off = np.array([0, 5, 9, 20])
    assert np.array_equal(W.bootstrap_indices(off, 30, seed=1), W.bootstrap_indices(off, 30, seed=1))
    assert not np.array_equal(W.bootstrap_indices(off, 30, seed=1), W.bootstrap_indices(off, 30, seed=2))


def test_calibration_activations_are_seeded_bf16_with_the_diagonal_scale():
    x = W.calibration_activations(0, 0, 64)
    assert x.dtype == np.uint16 and x.shape == (4, 64, 256)
    assert np.array_equal(x, W.calibration_activations(0, 0, 64))
    v = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(v)) and np.all((x & 0x7F80) != 0x7F80)
