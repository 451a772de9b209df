"""GPU parity of the candidate-set solver for other quantizers (the README's "Use the solver"
takes a code range and a group of any length): code ranges with at most 8 codes on each side of
zero and groups of up to 128 weights, against the oracle run with the same quantizer and against
the full grid bit for bit.  Groups whose direct candidates tie go to the full grid's list mode
(flag CQ_FLAG_FALLBACK); a test with more of them than that launch has workgroups runs its
grid-stride loop.

Every call goes through the C ABI (libcq.so)."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import bits_np, check_minimax, check_same_result, dev, say, spec_groups, threads

pytestmark = pytest.mark.gpu

KEYS = ("scales", "codes", "objective")

# (qmin, qmax, group length, environments): signed 3- and 2-bit codes, unsigned and one-sided
# ranges, the widest accepted range, the pages' range on shorter groups, and E up to 16
SPECS = [(-4, 3, 64, 4), (-2, 1, 32, 3), (0, 7, 128, 2), (-8, 8, 128, 4), (-8, 7, 100, 5), (-8, 7, 4, 2),
         (-1, 1, 16, 1), (-3, 5, 128, 8), (0, 1, 77, 16), (-8, 0, 90, 2), (-4, 3, 64, 20)]


def _run(w, d, n, method, qmin, qmax):
    r = cq.quantize_groups(dev(w), dev(d), n, method=method, qmin=qmin, qmax=qmax)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("qmin,qmax,G,E", SPECS, ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in SPECS])
def test_candidate_spec_against_oracle_and_full_grid(qmin, qmax, G, E):
    n = 64
    w, d = spec_groups(qmin, qmax, G, E, n, seed=11000 + 7 * G + qmax - qmin)
    say(f"candidate, quantizer [{qmin}, {qmax}], G={G}, E={E}: {n} groups")
    c = _run(w, d, n, "candidate", qmin, qmax)
    sol = oracle.solve(w, d, n, n_threads=threads(), qmin=qmin, qmax=qmax)
    same, near = check_minimax(w, d, n, c, sol, qmin=qmin, qmax=qmax)
    f = _run(w, d, n, "exhaustive", qmin, qmax)
    check_same_result(c, f, f"[{qmin}, {qmax}] G={G} E={E}", KEYS)
    flags = c["flags"].cpu().numpy()
    # the all-zero group: every scale ties at 0, the full grid decides (lowest pattern)
    assert bits_np(c["scales"])[1] == 0x0001 and flags[1] & cq.FLAG_FALLBACK
    say(f"  bits equal {same}/{n}, near ties {near}, fallbacks {int(np.count_nonzero(flags & cq.FLAG_FALLBACK))}")


def test_candidate_spec_many_fallbacks_take_the_list_loop():
    """3,000 groups of [-4, 3] at G = 64, E = 4, a third of them all-zero (each ties at every scale
    and goes to the full grid's list mode, more entries than its launch has workgroups): the same
    scales, codes and objectives as the full grid, and the fallback flag exactly on the zero
    groups and the other tied ones."""
    qmin, qmax, G, E, n = -4, 3, 64, 4, 3000
    w, d = spec_groups(qmin, qmax, G, E, n, seed=12345)
    zero = np.zeros(n, bool)
    zero[::3] = True
    w[zero] = 0.0
    say(f"candidate [{qmin}, {qmax}] G={G}: {n} groups, {int(zero.sum())} all-zero")
    c = _run(w, d, n, "candidate", qmin, qmax)
    f = _run(w, d, n, "exhaustive", qmin, qmax)
    check_same_result(c, f, "list loop", KEYS)
    flags = c["flags"].cpu().numpy()
    fb = (flags & cq.FLAG_FALLBACK) != 0
    assert np.all(fb[zero]), "every all-zero group is decided by the full grid"
    assert np.all(bits_np(c["scales"])[zero] == 0x0001)
    # the fallback groups carry the full grid's own flags besides FALLBACK
    ff = f["flags"].cpu().numpy()
    assert np.array_equal(flags[fb] & ~np.uint8(cq.FLAG_FALLBACK), ff[fb])
    sub = np.nonzero(~zero)[0][:256]
    sol = oracle.solve(w[sub], d[sub], sub.size, n_threads=threads(), qmin=qmin, qmax=qmax)
    cs = {k: c[k][torch.from_numpy(sub).cuda()] for k in KEYS}
    same, near = check_minimax(w[sub], d[sub], sub.size, cs, sol, qmin=qmin, qmax=qmax)
    say(f"  fallbacks {int(fb.sum())}; oracle on 256 nonzero groups: bits equal {same}, near ties {near}")


@pytest.mark.parametrize("qmin,qmax,G", [(-4, 3, 64), (-2, 1, 32)])
def test_candidate_spec_equals_full_grid_at_matrix_size(qmin, qmax, G):
    """28,672 seeded groups (the size of a config-1 matrix), bf16-valued N(0, 0.02) weights with 1%
    outliers x8 and lognormal diagonals shared by every eighth group, E = 4: the candidate solver
    and the full grid return the same scales, codes and binary64 objectives in every group."""
    rng = np.random.default_rng(4000 + G)
    n, E = 28672, 4
    w = W.round_bf16((rng.normal(0, 0.02, (n, G)) * np.where(rng.random((n, G)) < 0.01, 8.0, 1.0))
                     .astype(np.float32))
    d = rng.lognormal(0, 1, (n // 8, E, G)).astype(np.float32)
    c = cq.quantize_groups(dev(w), dev(d), n // 8, method="candidate", qmin=qmin, qmax=qmax)
    f = cq.quantize_groups(dev(w), dev(d), n // 8, method="exhaustive", qmin=qmin, qmax=qmax)
    torch.cuda.synchronize()
    check_same_result(c, f, f"[{qmin}, {qmax}] G={G}, {n} groups", KEYS)
    fb = int(torch.count_nonzero(c["flags"] & cq.FLAG_FALLBACK).item())
    say(f"candidate [{qmin}, {qmax}] G={G}: {n} groups equal to the full grid, {fb} decided by its list mode")


def test_solver_call_defaults_to_the_candidate_solver_where_it_applies():
    """The README's four-weight call with code ranges the candidate solver takes and one it does
    not: the same answer as the oracle either way."""
    ws = [0.9, -0.4, 0.2, -1.1]
    ds = [[1.0, 0.8, 0.5, 1.2], [0.6, 1.4, 0.9, 0.7]]
    w = np.array([ws], np.float32)
    d = np.array([ds], np.float32)
    for qmin, qmax in ((-8, 7), (-4, 3), (-2, 1), (0, 7), (-128, 127)):
        sol = oracle.solve(w, d, qmin=qmin, qmax=qmax)
        scale, obj, codes = cq.solve_breakpoint_exact(ws, ds, qmin=qmin, qmax=qmax)
        assert scale == oracle.fp16_value(sol.mm_bits[0]) and obj == sol.mm_F1[0], (qmin, qmax)
        assert codes == list(sol.codes[0]), (qmin, qmax)
