"""GPU parity on the oracle samples of the five synthetic configs, at the pages' protocol sizes.

The README and model card ("Verification") check the production solver against exhaustive FP16
enumeration on 10,000 solver cases; config 2 mirrors that with a seeded 10,000-group sample of its
3,883,008 groups.  Configs 3 and 4 (E = 8 and 16) are checked on seeded samples with the pooled
policy decided in the same pass, and the proxy on modules of a full config-1 matrix.  Each method
(full grid, bounded sweep, candidate solver) runs through the C ABI on the sample and is compared
with the oracle under the match criteria: scale bits equal where the oracle's runner-up gap exceeds
1e-9, else the objective within 1e-9; codes bit-exact; proxies within 1e-6."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import PROXY_TOL, bits_np, check_minimax, check_pooled, check_same_result, dev, say, threads

pytestmark = pytest.mark.gpu


def _methods(w, d, p, label, sol):
    """Every method on the same groups against the oracle; the full grid and the bounded sweep
    also bit for bit against each other, and the candidate solver against the full grid."""
    wt, dt = dev(w), dev(d)
    x = cq.quantize_groups(wt, dt, p, method="exhaustive", pooled=True)
    b = cq.quantize_groups(wt, dt, p, method="bounded", pooled=True)
    c = cq.quantize_groups(wt, dt, p, method="candidate")
    torch.cuda.synchronize()
    for name, r in (("exhaustive", x), ("bounded", b), ("candidate", c)):
        same, near = check_minimax(w, d, p, r, sol)
        if name != "candidate":
            check_pooled(w, d, p, r["pooled_scales"], r["pooled_objective"], sol)
        say(f"  {label} {name}: bits equal {same}/{w.shape[0]}, oracle near ties {near}")
    check_same_result(x, b, f"{label}: full grid against bounded")
    check_same_result(x, c, f"{label}: full grid against candidate", keys=("scales", "codes", "objective"))
    fl = c["flags"].cpu().numpy()
    say(f"  {label}: candidate fallbacks {int(np.count_nonzero(fl & cq.FLAG_FALLBACK))}, "
        f"full-grid binary64 sweeps {int(np.count_nonzero(x['flags'].cpu().numpy() & cq.FLAG_FP64_SWEEP))}")
    return x


def test_config2_ten_thousand_group_sample():
    """The pages' protocol: 10,000 seeded groups of config 2's 150 matrices."""
    gids = W.sample_groups(2, 10000)
    w, d, _ = W.gather_matrix_groups(2, gids)
    say(f"config 2 sample: {w.shape[0]} groups, E=4, oracle on {threads()} threads")
    sol = oracle.solve(w, d, w.shape[0], n_threads=threads())
    _methods(w, d, w.shape[0], "config 2 sample", sol)


def test_config3_stratified_sample():
    """Edge and tie stress (E = 8, per-group diagonals): 4,096 seeded groups, every category in its
    proportion (Student-t, tiny, all-zero, symmetric-pair ties, one-channel environments)."""
    cats = W.config3_categories()
    idx = W.sample_groups(3, 4096, salt=5)
    w, d, cat, ce = W.make_groups(3, idx)
    n = idx.size
    say(f"config 3 sample: {n} groups, E=8, categories {np.bincount(cat, minlength=5)}")
    sol = oracle.solve(w, d, n, n_threads=threads())
    x = _methods(w, d, n, "config 3 sample", sol)
    bits = bits_np(x["scales"])
    zero = cat == W.CAT_ZERO
    assert np.all(bits[zero] == 0x0001)
    pair = cat == W.CAT_PAIR_TIE
    half = np.array([int(np.float16(W.pair_tie_unit(int(k)) / 2).view(np.uint16)) for k in ce[pair]])
    assert np.array_equal(bits[pair], half)


def test_config4_sample():
    """Many environments (E = 16): 2,048 seeded groups of config 4's eight 4096 x 4096 matrices."""
    gids = W.sample_groups(4, 2048, salt=5)
    w, d, _ = W.gather_matrix_groups(4, gids)
    say(f"config 4 sample: {w.shape[0]} groups, E=16")
    sol = oracle.solve(w, d, w.shape[0], n_threads=threads())
    _methods(w, d, w.shape[0], "config 4 sample", sol)


def test_proxy_on_full_size_modules():
    """The proxy over config 1's gate matrix (28,672 groups): one module of all of them, and the
    same groups split into three uneven modules, for three policies; module means and macro within
    the proxy tolerance of the oracle's, every module compared."""
    w, d, p = W.matrix_groups(*W.make_matrix(1, 0))
    n = w.shape[0]
    wt, dt = dev(w), dev(d)
    r = cq.quantize_groups(wt, dt, p, method="bounded", pooled=True)
    ab = cq.baseline_scales(wt, dt, p, "absmax", codes=False, objective=False)
    sv = torch.stack((r["scales"], r["pooled_scales"], ab["scales"]))
    bits = bits_np(sv.reshape(-1)).reshape(3, n)
    for off in (np.array([0, n], np.int64), np.array([0, 5000, 5001, n], np.int64)):
        M = off.size - 1
        mods = np.repeat(np.arange(M), np.diff(off))
        pg, mm, macro = cq.proxy_worst_env_wmse_multi(wt, dt, sv, dev(off), p)
        torch.cuda.synchronize()
        for k in range(3):
            rp, rm, rmac = oracle.proxy(w, d, bits[k], mods, M, p, threads())
            np.testing.assert_allclose(pg[k].cpu().numpy(), rp, rtol=PROXY_TOL, atol=0)
            np.testing.assert_allclose(mm[k].cpu().numpy(), rm, rtol=PROXY_TOL, atol=0)
            assert abs(macro[k].item() - rmac) <= PROXY_TOL * rmac
        say(f"  proxy, {M} module(s) over {n} groups: macro {[float(x) for x in macro.cpu()]}")
