"""GPU parity: the held-out comparison of two policies (cq_heldout_compare) against the oracle.

Both sides sum every mean left to right in binary64 and take the same bootstrap draws (from the
seeded input generator), so counts, effect, sorted replicates and interval must agree bit for
bit.  The end-to-end case runs each side's own pipeline (scales, held-out proxy, comparison) on a
seeded sample of config 2 and compares within the proxy's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import check_minimax, check_pooled, bits_np, dev, say, threads

pytestmark = pytest.mark.gpu


def _gpu(pa, pb, off, idx, alpha=0.05):
    c, e, b, ci = cq.heldout_compare(dev(pa), dev(pb), dev(off), dev(idx) if idx.shape[0] else None, alpha)
    torch.cuda.synchronize()
    return c.cpu().numpy(), e.cpu().item(), b.cpu().numpy(), ci.cpu().numpy()


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok]), (a[ok][a[ok] != b[ok]][:5], b[ok][a[ok] != b[ok]][:5])


@pytest.mark.parametrize("B,alpha", [(1000, 0.05), (2500, 0.1), (1, 0.05), (0, 0.05)])
def test_synthetic_values_bit_exact(B, alpha):
    rng = np.random.default_rng(40 + B)
    sizes = [1, 2, 7, 64, 300, 1, 33, 128]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    pa = rng.lognormal(-8, 1, n)
    pb = pa * (1 + rng.normal(0, 0.02, n))
    tie = rng.random(n) < 0.1
    pb[tie] = pa[tie]
    idx = W.bootstrap_indices(off, B, seed=B)
    say(f"held-out comparison: {n} groups, {len(sizes)} modules, {B} replicates")
    gc, ge, gb, gci = _gpu(pa, pb, off, idx, alpha)
    oc, oe, ob, oci = oracle.heldout_compare(pa, pb, off, idx, alpha)
    assert list(gc) == list(oc) and oc[1] == np.count_nonzero(tie)
    _same([ge], [oe])
    _same(gb, ob)
    _same(gci, oci)
    if B == 0:
        assert np.all(np.isnan(gci))


def test_bad_draws_and_empty_module_give_nan():
    pa, pb = np.zeros(6), np.ones(6)
    off = np.array([0, 2, 6], np.int64)
    idx = W.bootstrap_indices(off, 5, seed=9)
    idx[3, 0] = 4                           # replicate 3 draws outside module 0
    gc, ge, gb, gci = _gpu(pa, pb, off, idx)
    oc, oe, ob, oci = oracle.heldout_compare(pa, pb, off, idx)
    _same(gb, ob)
    assert np.isnan(gb[-1]) and np.all(np.isnan(gci)) and ge == 1.0
    off2 = np.array([0, 2, 2, 6], np.int64)  # an empty module
    _, ge2, _, _ = _gpu(pa, pb, off2, W.bootstrap_indices(off2, 5, seed=9))
    assert np.isnan(ge2)


def test_end_to_end_on_held_out_diagonals():
    """Config 2's held-out setting at a size the oracle solves in seconds: 512 groups sampled
    across all matrices, scales from the calibration diagonals, proxy and comparison on the
    held-out diagonals.  The GPU's scales meet the match criteria against the oracle's for both
    policies; then the oracle's proxy and comparison on the GPU's own scales must give the GPU's
    counts where the two policies' values differ beyond the proxy tolerance, and its effect and
    interval within that tolerance."""
    w, d, de, off = W.heldout_sample(2, 512)
    n = w.shape[0]
    idx = W.bootstrap_indices(off, 2000, seed=11)
    say(f"held-out end to end: {n} groups in {off.size - 1} modules")
    wt, dt, det = dev(w), dev(d), dev(de)
    r = cq.quantize_groups(wt, dt, n, method="exhaustive", pooled=True)
    sc = torch.stack((r["scales"], r["pooled_scales"]))
    pg, _, _ = cq.proxy_worst_env_wmse_multi(wt, det, sc, dev(off), n)
    gc, ge, gb, gci = _gpu_t(pg[0], pg[1], off, idx)
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, r, sol)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol)
    gm, gp = bits_np(r["scales"]), bits_np(r["pooled_scales"])
    mods = np.repeat(np.arange(off.size - 1), np.diff(off))
    pa = oracle.proxy(w, de, gm, mods, off.size - 1, n, threads())[0]
    pb = oracle.proxy(w, de, gp, mods, off.size - 1, n, threads())[0]
    oc, oe, ob, oci = oracle.heldout_compare(pa, pb, off, idx)
    pgn = pg.cpu().numpy()
    np.testing.assert_allclose(pgn[0], pa, rtol=1e-6, atol=0)
    np.testing.assert_allclose(pgn[1], pb, rtol=1e-6, atol=0)
    decisive = np.abs(pa - pb) > 1e-6 * np.maximum(pa, pb)
    assert np.array_equal(np.sign(pgn[0] - pgn[1])[decisive], np.sign(pa - pb)[decisive])
    assert np.all(pgn[0][gm == gp] == pgn[1][gm == gp])
    # equal scales give equal values on both sides, so ties agree exactly; wins and losses agree
    # up to groups whose two values lie within the proxy tolerance of each other
    assert gc[1] == oc[1]
    assert abs(int(gc[0]) - int(oc[0])) <= int(np.count_nonzero(~decisive & (gm != gp)))
    scale = max(abs(float(np.mean(pa))), 1e-300)
    assert abs(ge - oe) <= 1e-6 * scale
    assert np.all(np.abs(gci - np.asarray(oci)) <= 1e-6 * scale)
    say(f"  wins/ties/losses {list(gc)} (oracle on the same scales {list(oc)}), effect {ge:.4g} "
        f"(oracle {oe:.4g}), interval {gci} (oracle {oci})")


def _gpu_t(pa_t, pb_t, off, idx, alpha=0.05):
    c, e, b, ci = cq.heldout_compare(pa_t.contiguous(), pb_t.contiguous(), dev(off), dev(idx), alpha)
    torch.cuda.synchronize()
    return c.cpu().numpy(), e.cpu().item(), b.cpu().numpy(), ci.cpu().numpy()


def test_more_groups_than_the_lds_path_holds():
    """5,000 groups in 40 modules: the module means take the global-memory kernel."""
    rng = np.random.default_rng(77)
    sizes = rng.integers(1, 250, 40)
    sizes[-1] += 5000 - sizes.sum() if sizes.sum() < 5000 else 0
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    assert n > 4096
    pa = rng.lognormal(-8, 1, n)
    pb = pa * (1 + rng.normal(0, 0.02, n))
    idx = W.bootstrap_indices(off, 300, seed=77)
    say(f"held-out comparison, global path: {n} groups, {sizes.size} modules")
    gc, ge, gb, gci = _gpu(pa, pb, off, idx)
    oc, oe, ob, oci = oracle.heldout_compare(pa, pb, off, idx)
    assert list(gc) == list(oc)
    _same([ge], [oe])
    _same(gb, ob)
    _same(gci, oci)
