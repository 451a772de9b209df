"""GPU parity of the full-grid exhaustive kernel (every scale, every weight): against the oracle,
against the bounded sweep bit for bit, and for other quantizers (the README's "Use the solver"
takes a code range and a group of any length) against the oracle run with the same quantizer.

Every call goes through the C ABI (libcq.so)."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import bits_np, check_minimax, check_pooled, check_same_result, dev, say, spec_groups, threads

pytestmark = pytest.mark.gpu


def _run(w, d, d_period, method="exhaustive", pooled=True, qmin=-8, qmax=7):
    r = cq.quantize_groups(dev(w), dev(d), d_period, method=method, pooled=pooled, qmin=qmin, qmax=qmax)
    torch.cuda.synchronize()
    return r


def test_full_grid_config0_all_groups():
    say("full grid, config 0: 128 groups, E=4, minimax + pooled")
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    r = _run(w, d, p)
    sol = oracle.solve(w, d, p, n_threads=threads())
    same, near = check_minimax(w, d, p, r, sol)
    check_pooled(w, d, p, r["pooled_scales"], r["pooled_objective"], sol)
    say(f"  bits equal {same}/128, near ties {near}")


def test_full_grid_equals_bounded_sweep_on_a_config1_matrix():
    """Config 1's gate matrix, all 28,672 groups: the full grid and the branch-and-bound sweep
    return the same scales, codes and binary64 objectives for both policies."""
    w, d, p = W.matrix_groups(*W.make_matrix(1, 0))
    say(f"full grid vs bounded: {w.shape[0]} groups")
    a = _run(w, d, p, "exhaustive")
    b = _run(w, d, p, "bounded")
    check_same_result(a, b, "config 1 gate")


# (qmin, qmax, group length, environments): signed 3-, 2- and 8-bit codes, unsigned 4-bit codes,
# the pages' range on longer, shorter and ragged groups
SPECS = [(-4, 3, 64, 4), (-2, 1, 32, 3), (-128, 127, 128, 4), (0, 15, 128, 2), (-8, 7, 256, 4),
         (-8, 7, 4, 2), (-8, 7, 100, 5), (-4, 3, 200, 1)]


@pytest.mark.parametrize("qmin,qmax,G,E", SPECS, ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in SPECS])
def test_quantizer_spec_against_oracle(qmin, qmax, G, E):
    n = 48
    w, d = spec_groups(qmin, qmax, G, E, n, seed=1000 + G + qmax)
    say(f"quantizer [{qmin}, {qmax}], G={G}, E={E}: {n} groups")
    r = _run(w, d, n, qmin=qmin, qmax=qmax)
    sol = oracle.solve(w, d, n, n_threads=threads(), qmin=qmin, qmax=qmax)
    same, near = check_minimax(w, d, n, r, sol, qmin=qmin, qmax=qmax)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol, qmin=qmin, qmax=qmax)
    bits = bits_np(r["scales"])
    assert bits[1] == 0x0001 and r["objective"].cpu().numpy()[1] == 0.0
    flags = r["flags"].cpu().numpy()
    assert flags[1] & cq.FLAG_EXACT_TIE
    say(f"  bits equal {same}/{n}, near ties {near}, flags {np.bincount(flags, minlength=32)[[0, 2, 6, 16, 18, 22]]}")


def test_pages_example_at_its_own_length_and_other_ranges():
    """The README's four-weight call with other code ranges: the group runs at length 4."""
    ws = [0.9, -0.4, 0.2, -1.1]
    ds = [[1.0, 0.8, 0.5, 1.2], [0.6, 1.4, 0.9, 0.7]]
    w = np.array([ws], np.float32)
    d = np.array([ds], np.float32)
    for qmin, qmax in ((-8, 7), (-4, 3), (-2, 1), (-128, 127), (0, 15)):
        sol = oracle.solve(w, d, qmin=qmin, qmax=qmax)
        scale, obj, codes = cq.solve_breakpoint_exact(ws, ds, qmin=qmin, qmax=qmax, method="exhaustive")
        assert scale == oracle.fp16_value(sol.mm_bits[0]) and obj == sol.mm_F1[0], (qmin, qmax)
        assert codes == list(sol.codes[0]), (qmin, qmax)


def test_spec_entry_with_the_pages_quantizer_is_the_plain_entry():
    """Group length 128 and [-8, 7] through the spec entry: the same results as cq_quantize_groups,
    for every method."""
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    wt, dt = dev(w), dev(d)
    n, E = w.shape[0], d.shape[1]
    for m in (cq.EXHAUSTIVE, cq.BOUNDED, cq.CANDIDATE):
        ws = torch.empty(cq.cq_workspace_size(m, E, n), dtype=torch.uint8, device="cuda")
        s1 = torch.empty(n, dtype=torch.int16, device="cuda")
        s2 = torch.empty(n, dtype=torch.int16, device="cuda")
        cq.cq_quantize_groups(wt, dt, p, E, n, m, s1, workspace=ws)
        cq.cq_quantize_groups_spec(wt, dt, 128, -8, 7, p, E, n, m, s2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2), m


SLICE_CASES = [(-8, 7, 128, 1), (-8, 7, 128, 2), (-8, 7, 128, 4), (-8, 7, 128, 8), (-8, 7, 128, 16),
               (-8, 7, 128, 32), (-4, 3, 64, 3)]


@pytest.mark.parametrize("qmin,qmax,G,E", SLICE_CASES, ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in SLICE_CASES])
def test_sliced_small_batches_equal_one_workgroup_per_group(qmin, qmax, G, E):
    """Below 1,024 groups a group's scales are split over several workgroups whose key lists are
    merged; from 1,024 groups on each group has one workgroup.  The same groups give the same
    scales, codes and binary64 objectives both ways, for both policies, and the same input and
    exact-tie flags (which groups the binary64 sweep settles may differ), including an
    all-zero group (zero rule), constructed ties, a non-finite input and a group outside the
    binary32 screen's range (binary64 sweep)."""
    n = 1040
    w, d = spec_groups(qmin, qmax, G, E, n, seed=2000 + E + G)
    w[4, 3] = np.nan
    d[5, 0, 0] = 2.0 ** 101
    say(f"slices vs one workgroup per group: [{qmin}, {qmax}], G={G}, E={E}, {n} groups")
    full = _run(w, d, n, qmin=qmin, qmax=qmax)
    keys = ("scales", "codes", "objective", "pooled_scales", "pooled_objective")
    mask = cq.FLAG_BAD_INPUT | cq.FLAG_EXACT_TIE
    for m in (1, 6, 300, 1023):
        sub = _run(np.ascontiguousarray(w[:m]), np.ascontiguousarray(d[:m]), m, qmin=qmin, qmax=qmax)
        check_same_result({k: full[k][:m] for k in keys}, sub, f"{m} groups", keys)
        fa, fb = full["flags"][:m].cpu().numpy() & mask, sub["flags"].cpu().numpy() & mask
        assert np.array_equal(fa, fb), f"{m} groups: flags differ on {np.nonzero(fa != fb)[0][:5]}"
    assert bits_np(full["scales"])[4] == 0 and full["flags"].cpu().numpy()[4] & cq.FLAG_BAD_INPUT


def test_flat_objectives_take_the_binary64_sweep():
    """Config 3's one-channel groups (one environment weighs a single channel): that environment's
    error is the same at every scale that rounds its weight to 0, and where the other environments
    stay below it the minimax objective is flat, with hundreds of patterns tied exactly.  The
    screen's shortlist overflows and the binary64 sweep decides; the result against the oracle."""
    w, d, cat, _ = W.make_groups(3, np.arange(8192))
    sel = np.nonzero(cat == W.CAT_ONE_CHANNEL)[0]
    r = _run(w[sel], d[sel], sel.size)
    swept = sel[np.nonzero(r["flags"].cpu().numpy() & cq.FLAG_FP64_SWEEP)[0]]
    say(f"one-channel groups {sel.size}, decided by the binary64 sweep {swept.size}")
    assert swept.size > 0
    ws, ds = w[swept], d[swept]
    r = _run(ws, ds, swept.size)
    assert np.all(r["flags"].cpu().numpy() & cq.FLAG_FP64_SWEEP)
    sol = oracle.solve(ws, ds, swept.size, n_threads=threads())
    same, near = check_minimax(ws, ds, swept.size, r, sol)
    check_pooled(ws, ds, swept.size, r["pooled_scales"], r["pooled_objective"], sol)
    flags = r["flags"].cpu().numpy()
    say(f"  bits equal {same}/{swept.size}, exact ties flagged {int(np.count_nonzero(flags & cq.FLAG_EXACT_TIE))}")


def _random_specs(count, seed):
    """Seeded quantizers: code ranges with qmin <= 0 <= qmax (one-sided ones included), group
    lengths from 1 to 256 and 1 to 9 environments."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        qmin, qmax = -int(rng.integers(0, 21)), int(rng.integers(0, 21))
        if qmin < qmax:
            out.append((qmin, qmax, int(rng.integers(1, 257)), int(rng.integers(1, 10))))
    return out


RANDOM_SPECS = _random_specs(10, 2026) + [(0, 7, 50, 3), (-8, 0, 90, 2)]  # and two one-sided ranges


@pytest.mark.parametrize("qmin,qmax,G,E", RANDOM_SPECS, ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in RANDOM_SPECS])
def test_seeded_random_quantizers_against_oracle(qmin, qmax, G, E):
    """Ten seeded quantizers (code range, group length, environment count) beyond the listed ones,
    and two one-sided code ranges, 24 groups each of the same structure: minimax and pooled against
    the oracle run with the same quantizer."""
    n = 24
    w, d = spec_groups(qmin, qmax, G, E, n, seed=7000 + 31 * G + qmax - qmin)
    r = _run(w, d, n, qmin=qmin, qmax=qmax)
    sol = oracle.solve(w, d, n, n_threads=threads(), qmin=qmin, qmax=qmax)
    same, near = check_minimax(w, d, n, r, sol, qmin=qmin, qmax=qmax)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol, qmin=qmin, qmax=qmax)
    say(f"quantizer [{qmin}, {qmax}], G={G}, E={E}: bits equal {same}/{n}, near ties {near}")


PACK_SPECS = [(2, 64, 70, 256), (8, 32, 33, 96), (4, 100, 17, 200), (2, 16, 130, 48), (8, 256, 5, 512),
              (4, 128, 65, 384), (8, 1, 9, 20)]


@pytest.mark.parametrize("bits,group,out,inp", PACK_SPECS, ids=[f"b{b}_g{g}_{o}x{i}" for b, g, o, i in PACK_SPECS])
def test_pack_other_field_widths_against_oracle(bits, group, out, inp):
    """GPTQ-v1 packing with 2-, 4- and 8-bit fields and other group lengths (ragged tiles in both
    directions) bit for bit against the oracle's packing; 4-bit fields in groups of 128 also equal
    the plain entry point's."""
    rng = np.random.default_rng(bits * 1000 + group + out + inp)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    codes = rng.integers(lo, hi + 1, (out, inp)).astype(np.int8)
    sbits = rng.integers(1, 0x7C00, (out, inp // group)).astype(np.uint16)
    qw, sc = cq.pack_gptq_v1(dev(codes), dev(sbits.view(np.int16)), out, inp, bits=bits, group=group)
    torch.cuda.synchronize()
    want_q, want_s = oracle.pack_gptq_v1(codes, sbits, out, inp, bits=bits, group=group)
    np.testing.assert_array_equal(qw.cpu().numpy(), want_q)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint16), want_s)
    back, _ = oracle.unpack_gptq_v1(qw.cpu().numpy(), sc.cpu().numpy().view(np.uint16), bits=bits)
    np.testing.assert_array_equal(back, codes)
    if bits == 4 and group == 128:
        q2 = torch.empty_like(qw)
        s2 = torch.empty_like(sc)
        cq.cq_pack_gptq_v1_spec(dev(codes), dev(sbits.view(np.int16)), out, inp, 4, 128, q2, s2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q2.cpu().numpy(), want_q)


def test_other_quantizer_solved_and_packed_end_to_end():
    """A 2-bit quantizer, [-2, 1] in groups of 32: a 48 x 256 matrix solved by the full grid, its
    codes and scales packed with 2-bit fields, and the packing unpacked again by the oracle."""
    rng = np.random.default_rng(77)
    out, inp, G = 48, 256, 32
    A = W.round_bf16(rng.normal(0, 0.02, (out, inp)).astype(np.float32))
    w = A.reshape(-1, G)
    d = rng.lognormal(0, 1, (inp // G, 2, G)).astype(np.float32)
    r = cq.quantize_groups(dev(w), dev(d), inp // G, method="exhaustive", qmin=-2, qmax=1)
    qw, sc = cq.pack_gptq_v1(r["codes"].reshape(out, inp), r["scales"].reshape(out, inp // G), out, inp,
                             bits=2, group=G)
    torch.cuda.synchronize()
    codes, sbits = oracle.unpack_gptq_v1(qw.cpu().numpy(), sc.cpu().numpy().view(np.uint16), bits=2)
    np.testing.assert_array_equal(codes, r["codes"].cpu().numpy().reshape(out, inp))
    np.testing.assert_array_equal(sbits.reshape(-1), bits_np(r["scales"]))
    sol = oracle.solve(w, d, inp // G, n_threads=threads(), qmin=-2, qmax=1)
    check_minimax(w, d, inp // G, r, sol, qmin=-2, qmax=1)


BASE_SPECS = [(-4, 3, 64, 4), (-2, 1, 32, 3), (-128, 127, 128, 4), (0, 15, 128, 2), (-8, 7, 256, 4),
              (-3, 5, 38, 1), (-8, 7, 100, 9)]


@pytest.mark.parametrize("qmin,qmax,G,E", BASE_SPECS, ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in BASE_SPECS])
def test_baselines_for_other_quantizers(qmin, qmax, G, E):
    """AbsMax for another quantizer (fp16(max|w| / qmax)): scales, codes and the binary64 objective
    bit for bit against the oracle, the same scales and codes without the objective; the pooled
    baseline equals the full grid's pooled policy."""
    n = 3 * (256 // E) + 5  # a ragged last workgroup
    w, d = spec_groups(qmin, qmax, G, E, n, seed=9000 + G + qmax)
    period = n - 2
    d = d[:period]
    ab = cq.baseline_scales(dev(w), dev(d), period, "absmax", qmin=qmin, qmax=qmax)
    ab0 = cq.baseline_scales(dev(w), dev(d), period, "absmax", objective=False, qmin=qmin, qmax=qmax)
    pl = cq.baseline_scales(dev(w), dev(d), period, "pooled", qmin=qmin, qmax=qmax)
    r = _run(w, d, period, qmin=qmin, qmax=qmax)
    bits = bits_np(ab["scales"])
    np.testing.assert_array_equal(bits, oracle.absmax_bits(w, qmax))
    np.testing.assert_array_equal(ab["codes"].cpu().numpy(), oracle.codes_for(w, bits, qmin, qmax))
    np.testing.assert_array_equal(ab["objective"].cpu().numpy(), oracle.objective(w, d, bits, period, threads(),
                                                                                  qmin, qmax))
    np.testing.assert_array_equal(bits_np(ab0["scales"]), bits)
    np.testing.assert_array_equal(ab0["codes"].cpu().numpy(), ab["codes"].cpu().numpy())
    np.testing.assert_array_equal(bits_np(pl["scales"]), bits_np(r["pooled_scales"]))
    np.testing.assert_array_equal(pl["objective"].cpu().numpy().view(np.uint64),
                                  r["pooled_objective"].cpu().numpy().view(np.uint64))
    np.testing.assert_array_equal(pl["codes"].cpu().numpy(), oracle.codes_for(w, bits_np(pl["scales"]), qmin, qmax))


@pytest.mark.parametrize("qmin,qmax,G,E", BASE_SPECS[:5], ids=[f"q{a}..{b}_G{g}_E{e}" for a, b, g, e in BASE_SPECS[:5]])
def test_proxy_for_other_quantizers(qmin, qmax, G, E):
    """The proxy for another quantizer (1/G for the pages' 1/128) for three policies in one call:
    per-group values, module means and macro against the oracle within the proxy tolerance; a
    ragged last workgroup and an empty module (NaN on both sides)."""
    n = 16 * 5 + 9
    w, d = spec_groups(qmin, qmax, G, E, n, seed=9500 + G + qmax)
    r = _run(w, d, n, qmin=qmin, qmax=qmax)
    rng = np.random.default_rng(G + E)
    bits = np.stack([bits_np(r["scales"]), bits_np(r["pooled_scales"]),
                     rng.integers(0x1400, 0x2400, n).astype(np.uint16)])
    off = np.array([0, 30, 30, 70, n], np.int64)
    mods = np.repeat(np.arange(4), np.diff(off))
    pg, mm, macro = cq.proxy_worst_env_wmse_multi(dev(w), dev(d), dev(bits.view(np.int16)), dev(off), qmin=qmin,
                                                  qmax=qmax)
    torch.cuda.synchronize()
    pg, mm, macro = pg.cpu().numpy(), mm.cpu().numpy(), macro.cpu().numpy()
    for k in range(3):
        rp, rm, rmac = oracle.proxy(w, d, bits[k], mods, 4, n, threads(), qmin, qmax)
        np.testing.assert_allclose(pg[k], rp, rtol=1e-6, atol=0)
        np.testing.assert_allclose(mm[k], rm, rtol=1e-6, atol=0, equal_nan=True)
        assert np.isnan(mm[k, 1]) and np.isnan(macro[k]) and np.isnan(rmac)
