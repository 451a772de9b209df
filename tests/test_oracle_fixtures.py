"""The stored oracle samples (tests/golden/oracle_config*.npz, written by make_oracle_fixtures.py)
still agree with the oracle: a seeded draw of their groups is solved again and must give the same
bit patterns and the same runner-up-gap flags for both policies.  A fixture gone stale (a changed
oracle or input generator) fails here, on the CPU, before any GPU test reads it."""
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fixture(name):
    f = np.load(os.path.join(GOLDEN, name))
    n = f["mm_bits"].size
    out = {k: f[k] for k in f.files}
    out["mm_sure"] = np.unpackbits(out["mm_sure"])[:n].astype(bool)
    out["pl_sure"] = np.unpackbits(out["pl_sure"])[:n].astype(bool)
    return out


def _same(fx, pick, sol):
    np.testing.assert_array_equal(sol.mm_bits, fx["mm_bits"][pick])
    np.testing.assert_array_equal(sol.pl_bits, fx["pl_bits"][pick])
    np.testing.assert_array_equal(sol.mm_gap > 1e-9, fx["mm_sure"][pick])
    np.testing.assert_array_equal(sol.pl_gap > 1e-9, fx["pl_sure"][pick])


def test_config1_fixture_reproduces():
    fx = _fixture("oracle_config1_all.npz")
    assert fx["mm_bits"].size == 86016
    rng = np.random.default_rng(41)
    lo = 0
    for m in range(len(W.config(1).matrices)):
        w, d, p = W.matrix_groups(*W.make_matrix(1, m))
        pick = np.sort(rng.choice(w.shape[0], 24, replace=False))
        sol = oracle.solve(w[pick], d[pick % p], len(pick), n_threads=os.cpu_count() or 1)
        _same(fx, lo + pick, sol)
        lo += w.shape[0]


@pytest.mark.parametrize("name,k", [("oracle_config3_65536.npz", 3), ("oracle_config4_16384.npz", 4)])
def test_sample_fixture_reproduces(name, k):
    fx = _fixture(name)
    gids = fx["gids"]
    pick = np.sort(np.random.default_rng(42 + k).choice(gids.size, 32, replace=False))
    if k == 3:
        w, d, _, _ = W.make_groups(3, gids[pick])
    else:
        w, d, _ = W.gather_matrix_groups(4, gids[pick])
    sol = oracle.solve(w, d, w.shape[0], n_threads=os.cpu_count() or 1)
    _same(fx, pick, sol)
