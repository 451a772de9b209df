"""GPU parity on the oracle's protocol samples that take minutes of host brute force: all 86,016
groups of config 1, a seeded 65,536-group subsample of config 3 (E = 8, every stress category)
and a seeded 16,384-group sample of config 4 (E = 16).

The pages check their solver against exhaustive FP16 enumeration ("Verification" in the CliffQuant
README and the W4A16-G128 model card).  The oracle's winning bit patterns, and whether its runner-up
gap exceeds 1e-9, are stored in tests/golden/ by make_oracle_fixtures.py (which calls only the
oracle); the tests regenerate the same seeded inputs, run every method through the C ABI, and
apply the match criteria: bits equal where the gap exceeds 1e-9, else the GPU's objective within
1e-9 of the oracle's minimum; the GPU's binary64 objective equal to the oracle's at the GPU's own
scale, bit for bit; codes bit-exact."""
import os

import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import bits_np, check_policy, dev, pooled_at, say, threads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fixture(name):
    f = np.load(os.path.join(GOLDEN, name))
    n = f["mm_bits"].size
    out = {k: f[k] for k in f.files}
    out["mm_sure"] = np.unpackbits(out["mm_sure"])[:n].astype(bool)
    out["pl_sure"] = np.unpackbits(out["pl_sure"])[:n].astype(bool)
    return out


def _against(label, w, d, p, r, fx, lo, hi, pooled):
    """One method's result on groups [lo, hi) of the fixture."""
    nt = threads()
    bits = fx["mm_bits"][lo:hi]
    gap = np.where(fx["mm_sure"][lo:hi], np.inf, 0.0)
    F1 = oracle.objective(w, d, bits, p, nt)
    gb = bits_np(r["scales"])
    same, near = check_policy(f"{label} minimax", w, d, p, gb, r["objective"].cpu().numpy(), bits, F1, gap,
                              lambda b: oracle.objective(w, d, b, p, nt))
    if r.get("codes") is not None:
        diff = np.nonzero(np.any(r["codes"].cpu().numpy() != oracle.codes_for(w, gb), axis=1))[0]
        assert diff.size == 0, f"{label}: codes differ on groups {diff[:5]}"
    if pooled:
        pbits = fx["pl_bits"][lo:hi]
        pgap = np.where(fx["pl_sure"][lo:hi], np.inf, 0.0)
        check_policy(f"{label} pooled", w, d, p, bits_np(r["pooled_scales"]), r["pooled_objective"].cpu().numpy(),
                     pbits, pooled_at(w, d, p, pbits), pgap, lambda b: pooled_at(w, d, p, b))
    return same, near


def _all_methods(label, w, d, p, fx, lo, hi):
    wt, dt = dev(w), dev(d)
    for method in ("exhaustive", "bounded", "candidate"):
        pooled = method != "candidate"
        r = cq.quantize_groups(wt, dt, p, method=method, pooled=pooled)
        torch.cuda.synchronize()
        same, near = _against(f"{label} {method}", w, d, p, r, fx, lo, hi, pooled)
        say(f"  {label} {method}: bits equal {same}/{hi - lo}, oracle near ties {near}")


def test_config1_every_group_against_the_oracle():
    fx = _fixture("oracle_config1_all.npz")
    lo = 0
    for m in range(len(W.config(1).matrices)):
        w, d, p = W.matrix_groups(*W.make_matrix(1, m))
        hi = lo + w.shape[0]
        say(f"config 1 matrix {m}: groups {lo}..{hi - 1}")
        _all_methods(f"config 1 matrix {m}", w, d, p, fx, lo, hi)
        lo = hi
    assert lo == fx["mm_bits"].size == 86016


def test_config3_subsample_against_the_oracle():
    fx = _fixture("oracle_config3_65536.npz")
    gids = fx["gids"]
    assert np.array_equal(gids, W.sample_groups(3, 65536, salt=7))
    w, d, cat, _ = W.make_groups(3, gids)
    say(f"config 3 subsample: {w.shape[0]} groups, E=8, categories {np.bincount(cat, minlength=5)}")
    _all_methods("config 3", w, d, w.shape[0], fx, 0, w.shape[0])


def test_config4_sample_against_the_oracle():
    fx = _fixture("oracle_config4_16384.npz")
    gids = fx["gids"]
    assert np.array_equal(gids, W.sample_groups(4, 16384, salt=7))
    w, d, _ = W.gather_matrix_groups(4, gids)
    say(f"config 4 sample: {w.shape[0]} groups, E=16")
    _all_methods("config 4", w, d, w.shape[0], fx, 0, w.shape[0])
