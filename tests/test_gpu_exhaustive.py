"""GPU parity: the exhaustive searches (the full grid and the bounded sweep), the baselines, the
packer and the proxy against the oracle.

Every call goes through the C ABI (libcq.so).  Inputs are the seeded synthetic configs; the
oracle runs on the host on the same arrays (all groups where it takes seconds, seeded
samples otherwise).
"""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import bits_np, check_minimax, check_pooled, check_same_result, dev, say, threads

pytestmark = pytest.mark.gpu
BOTH = pytest.mark.parametrize("method", ["exhaustive", "bounded"])


def _run(w, d, d_period, method="exhaustive", pooled=True):
    r = cq.quantize_groups(dev(w), dev(d), d_period, method=method, pooled=pooled)
    torch.cuda.synchronize()
    return r


@BOTH
def test_config0_all_groups(method):
    say(f"config 0: 128 groups, E=4, {method} + pooled")
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    r = _run(w, d, p, method)
    sol = oracle.solve(w, d, p, n_threads=threads())
    same, near = check_minimax(w, d, p, r, sol)
    check_pooled(w, d, p, r["pooled_scales"], r["pooled_objective"], sol)
    flags = r["flags"].cpu().numpy()
    assert not np.any(flags & cq.FLAG_BAD_INPUT)
    say(f"  bits equal {same}/128, near ties {near}, flags {np.bincount(flags)}")


@BOTH
def test_pages_example_and_tiny_groups(method):
    w, d = W.pages_example()
    r = _run(w, d, 1, method)
    sol = oracle.solve(w, d)
    check_minimax(w, d, 1, r, sol)
    check_pooled(w, d, 1, r["pooled_scales"], r["pooled_objective"], sol)
    scale, obj, codes = cq.solve_breakpoint_exact([0.9, -0.4, 0.2, -1.1],
                                                  [[1.0, 0.8, 0.5, 1.2], [0.6, 1.4, 0.9, 0.7]],
                                                  method=method)
    assert scale == oracle.fp16_value(sol.mm_bits[0]) and obj == sol.mm_F1[0]
    assert codes == list(sol.codes[0, :4])


@BOTH
def test_constructed_ties_and_edge_groups(method):
    """All-zero (0x0001), symmetric pairs (c/2), single weights, a subnormal-scale group."""
    rng = np.random.default_rng(7)
    ws, ds = [], []
    ws.append(np.zeros(128, np.float32))
    for k in (5, 8, 10):
        c = 2.0 ** -k
        mult = np.array([1, 2, 3] + list(rng.integers(1, 4, 61)), np.float64)
        ws.append(rng.permutation(np.concatenate([mult * c, -mult * c])).astype(np.float32))
    for v in (0.75, -1.5, 2.0 ** -20):
        x = np.zeros(128, np.float32)
        x[17] = v
        ws.append(x)
    ws.append((rng.uniform(-1, 1, 128) * 1e-5).astype(np.float32))
    ws.append(W.round_bf16(rng.normal(0, 0.02, 128).astype(np.float32)))
    n = len(ws)
    w = np.stack(ws)
    d = rng.lognormal(0, 1, (n, 4, 128)).astype(np.float32)
    d[:, 1] = d[:, 0]
    d[-1, 2] = 0.0
    d[-1, 2, 5] = 128.0
    r = _run(w, d, n, method)
    sol = oracle.solve(w, d, n)
    check_minimax(w, d, n, r, sol)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol)
    bits = bits_np(r["scales"])
    assert bits[0] == 1
    for j, k in enumerate((5, 8, 10)):
        assert bits[1 + j] == int(np.float16(2.0 ** -(k + 1)).view(np.uint16))
    flags = r["flags"].cpu().numpy()
    assert np.all(flags[:4] & cq.FLAG_EXACT_TIE)


def test_top_pattern_ranges_sliced_and_unsliced():
    """Where the bounded sweep stops (the first scale >= 2 max|w|): past the grid (2 max|w| >
    65504, every pattern screened), in the last binade, in the subnormal range, and after a lone
    weight.  Twelve groups go through the sliced path; the same groups tiled to 1,200 go one
    workgroup each and must give identical results.  The full grid gives the same on the twelve."""
    rng = np.random.default_rng(23)
    ws = []
    big = rng.normal(0, 3000, 128)
    big[7] = 40000.0
    ws.append(big)
    mid = rng.normal(0, 2000, 128)
    mid[3] = -15000.0
    ws.append(mid)
    ws.append(rng.uniform(-1, 1, 128) * 1e-6)
    ws.append(rng.uniform(-1, 1, 128) * 3e-5)
    lone = np.zeros(128)
    lone[100] = 0.3
    ws.append(lone)
    for sd in (0.005, 0.02, 0.08, 0.5, 4.0, 100.0, 1000.0):
        ws.append(rng.normal(0, sd, 128))
    w = W.round_bf16(np.stack(ws).astype(np.float32))
    n = w.shape[0]
    d = rng.lognormal(0, 1, (n, 4, 128)).astype(np.float32)
    r = _run(w, d, n, "bounded")
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, r, sol)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol)
    check_same_result(r, _run(w, d, n, "exhaustive"), "full grid against the bounded sweep")
    reps = 100
    wt, dt = np.tile(w, (reps, 1)), np.tile(d, (reps, 1, 1))
    rt = _run(wt, dt, n * reps, "bounded")
    for key in ("scales", "objective", "flags", "pooled_scales", "pooled_objective", "codes"):
        a = r[key].cpu().numpy()
        b = rt[key].cpu().numpy().reshape((reps,) + a.shape)
        assert np.all(b == a[None]), key


def test_optimum_far_from_the_absmax_scale():
    """The screen starts at the chunk of max|w|/9 and skips chunks whose lower bound exceeds the
    best value seen; the candidate solver drops transitions below a bound from its probe there.
    Groups whose optimum lies far from there (8,010 patterns below to 683 above): a large weight
    whose diagonal is tiny (the optimum clips it, several binades below), diagonals that weigh
    the largest weight only (codes 1..7 of it all fit exactly; the small weights decide, above),
    one environment on a few small weights.  Exhaustive sliced (12 groups) and one workgroup each
    (tiled), and the candidate solver, against the oracle."""
    rng = np.random.default_rng(31)
    ws, ds = [], []
    for big, dbig in ((1.0, 1e-6), (0.5, 1e-4), (8.0, 1e-7), (0.25, 1e-3)):
        x = rng.normal(0, 0.01, 128)
        x[9] = big
        dd = rng.lognormal(0, 0.5, (4, 128))
        dd[:, 9] = dbig
        ws.append(x); ds.append(dd)
    for big in (0.75, 0.0625, 3.0, 0.4):
        x = rng.normal(0, 0.02, 128)
        x[50] = big
        dd = np.full((4, 128), 1e-6) * rng.lognormal(0, 0.3, (4, 128))
        dd[:, 50] = 1.0
        ws.append(x); ds.append(dd)
    for sd in (0.01, 0.03, 0.1, 1.0):
        x = rng.normal(0, sd, 128)
        dd = rng.lognormal(0, 1, (4, 128))
        dd[2] = 1e-5
        dd[2, :4] = 50.0
        ws.append(x); ds.append(dd)
    w = W.round_bf16(np.stack(ws).astype(np.float32))
    d = np.stack(ds).astype(np.float32)
    n = w.shape[0]
    say(f"optimum far from max|w|/7: {n} groups, sliced and tiled")
    r = _run(w, d, n, "bounded")
    check_same_result(r, _run(w, d, n, "exhaustive"), "full grid against the bounded sweep")
    sol = oracle.solve(w, d, n, n_threads=threads())
    check_minimax(w, d, n, r, sol)
    check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol)
    start = np.array([int(np.float16(np.abs(w[j]).max() / 9).view(np.uint16)) for j in range(n)])
    say(f"  winner minus start pattern: {bits_np(r['scales']).astype(np.int64) - start}")
    # the candidate solver's window (from its probe at max|w|/9) must keep these optima too
    c = cq.quantize_groups(dev(w), dev(d), n, method="candidate")
    torch.cuda.synchronize()
    check_minimax(w, d, n, c, sol)
    reps = 100
    rt = _run(np.tile(w, (reps, 1)), np.tile(d, (reps, 1, 1)), n * reps, "bounded")
    for key in ("scales", "objective", "flags", "pooled_scales", "pooled_objective", "codes"):
        a = r[key].cpu().numpy()
        b = rt[key].cpu().numpy().reshape((reps,) + a.shape)
        assert np.all(b == a[None]), key


def test_thirty_two_environments_every_method():
    """E = 32, the largest environment count: the full grid and the bounded sweep (minimax and
    pooled) and the candidate solver against the oracle on 16 groups with per-group diagonals."""
    rng = np.random.default_rng(31)
    n = 16
    w = W.round_bf16(rng.normal(0, 0.03, (n, 128)).astype(np.float32))
    w[::5, 7] *= 8.0
    d = rng.lognormal(0, 1.2, (n, 32, 128)).astype(np.float32)
    sol = oracle.solve(w, d, n, n_threads=threads())
    for method in ("exhaustive", "bounded"):
        r = _run(w, d, n, method)
        check_minimax(w, d, n, r, sol)
        check_pooled(w, d, n, r["pooled_scales"], r["pooled_objective"], sol)
    c = _run(w, d, n, method="candidate", pooled=False)
    check_minimax(w, d, n, c, sol)


def test_batch_sizes_around_the_slicing_switch():
    """Bounded sweep: 1,023 groups run sliced, 1,024 and 1,025 one workgroup each: every batch
    gives bit for bit what the same groups give inside one full-matrix run."""
    w, d, p = W.matrix_groups(*W.make_matrix(1, 0))
    full = _run(w, d, p, "bounded")
    for n in (1023, 1024, 1025):
        # keep whole d periods so that every group sees its own diagonal slice
        r = _run(w[:n], d, p, "bounded")
        for key in ("scales", "objective", "flags", "pooled_scales", "pooled_objective", "codes"):
            a = r[key].cpu().numpy()
            b = full[key].cpu().numpy()[:n]
            assert np.array_equal(a, b), (n, key)


@BOTH
def test_bad_inputs_are_flagged(method):
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (4, 128)).astype(np.float32)
    d = rng.lognormal(0, 1, (4, 2, 128)).astype(np.float32)
    w[1, 3] = np.nan
    d[2, 1, 7] = -1.0
    w[3, 0] = np.inf
    r = _run(w, d, 4, method)
    flags = r["flags"].cpu().numpy()
    assert list(flags & cq.FLAG_BAD_INPUT) == [0, 1, 1, 1]
    assert list(bits_np(r["scales"])[1:]) == [0, 0, 0]
    assert np.all(np.isnan(r["objective"].cpu().numpy()[1:]))
    sol = oracle.solve(w[:1], d[:1], 1)
    assert bits_np(r["scales"])[0] == sol.mm_bits[0]


@BOTH
def test_fp64_sweep_path_matches_oracle(method):
    """Groups outside the binary32 screen's guaranteed range (a diagonal entry of 1e-38, a
    weight 2^-60 next to ordinary ones) are decided by the full binary64 sweep."""
    rng = np.random.default_rng(11)
    w = W.round_bf16(rng.normal(0, 0.02, (3, 128)).astype(np.float32))
    d = rng.lognormal(0, 1, (3, 4, 128)).astype(np.float32)
    d[0, 1, 3] = 1e-38
    w[1, 9] = 2.0 ** -60
    r = _run(w, d, 3, method)
    sol = oracle.solve(w, d, 3)
    check_minimax(w, d, 3, r, sol)
    check_pooled(w, d, 3, r["pooled_scales"], r["pooled_objective"], sol)
    flags = r["flags"].cpu().numpy()
    assert flags[0] & cq.FLAG_FP64_SWEEP and flags[1] & cq.FLAG_FP64_SWEEP
    assert not flags[2] & cq.FLAG_FP64_SWEEP


@pytest.mark.parametrize("method", ["exhaustive", "bounded", "candidate"])
def test_empty_batch(method):
    w = torch.zeros((0, 128), dtype=torch.float32, device="cuda")
    d = torch.ones((1, 4, 128), dtype=torch.float32, device="cuda")
    r = cq.quantize_groups(w, d, 1, method=method)
    torch.cuda.synchronize()
    assert r["scales"].numel() == 0


@BOTH
def test_config1_full_size_sampled(method):
    """Config 1 at full size (the benchmark's launch configuration, one call per matrix); the
    oracle checks a seeded sample of 192 groups; properties checked on every group."""
    spec = W.config(1)
    gids = W.sample_groups(1, 192)
    m_idx, local = W.locate(1, gids)
    for m, mat in enumerate(spec.matrices):
        A, dm = W.make_matrix(1, m)
        w, d, p = W.matrix_groups(A, dm)
        say(f"config 1 {mat.name}: {w.shape[0]} groups")
        wt, dt = dev(w), dev(d)
        r = cq.quantize_groups(wt, dt, p, method=method, pooled=True)
        ab = cq.baseline_scales(wt, dt, p, "absmax")
        torch.cuda.synchronize()
        # properties on every group
        obj, abobj = r["objective"].cpu().numpy(), ab["objective"].cpu().numpy()
        assert np.all(obj <= abobj)
        assert not np.any(r["flags"].cpu().numpy() & cq.FLAG_BAD_INPUT)
        codes = r["codes"].cpu().numpy()
        assert codes.min() >= -8 and codes.max() <= 7
        # oracle on the sample
        sel = local[m_idx == m]
        ws, ds = w[sel], d[sel % p]
        sol = oracle.solve(ws, ds, ds.shape[0], n_threads=threads())
        sub = {k: (v[torch.from_numpy(sel).cuda()] if v is not None else None) for k, v in r.items()}
        check_minimax(ws, ds, ds.shape[0], sub, sol)
        check_pooled(ws, ds, ds.shape[0], sub["pooled_scales"], sub["pooled_objective"], sol)
        absub = bits_np(ab["scales"])[sel]
        np.testing.assert_array_equal(absub, oracle.absmax_bits(ws))


def test_absmax_matches_oracle():
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    w = w.copy()
    w[0] = 0.0
    w[1, 5] = 1e6
    w[2] = w[2] * np.float32(1e-7)
    ab = cq.baseline_scales(dev(w), dev(d), p, "absmax")
    torch.cuda.synchronize()
    bits = bits_np(ab["scales"])
    np.testing.assert_array_equal(bits, oracle.absmax_bits(w))
    np.testing.assert_array_equal(ab["codes"].cpu().numpy(), oracle.codes_for(w, bits))
    np.testing.assert_array_equal(ab["objective"].cpu().numpy(), oracle.objective(w, d, bits, p))


@pytest.mark.parametrize("E", [1, 3, 4, 8, 17, 32])
def test_absmax_objective_every_env_count(E):
    """The per-(group, environment) objective kernel at environment counts that fill a 256-thread
    workgroup unevenly, a group count that leaves the last workgroup ragged, and d shared with a
    period: scales, codes and the binary64 objective equal the oracle's bit for bit, and the
    scales and codes equal those of the call without the objective."""
    rng = np.random.default_rng(100 + E)
    gpb = 256 // E
    n = 3 * gpb + 5
    w = (rng.standard_normal((n, 128)) * np.exp(rng.uniform(-6, 2, (n, 1)))).astype(np.float32)
    w[0] = 0.0
    w[1, 7] = 3.0e4
    period = n - 2
    d = rng.gamma(0.7, 1.0, (period, E, 128)).astype(np.float32)
    say(f"AbsMax objective: E={E}, {n} groups, d period {period}")
    ab = cq.baseline_scales(dev(w), dev(d), period, "absmax")
    ab0 = cq.baseline_scales(dev(w), dev(d), period, "absmax", objective=False)
    torch.cuda.synchronize()
    bits = bits_np(ab["scales"])
    np.testing.assert_array_equal(bits, oracle.absmax_bits(w))
    np.testing.assert_array_equal(ab["codes"].cpu().numpy(), oracle.codes_for(w, bits))
    np.testing.assert_array_equal(ab["objective"].cpu().numpy(), oracle.objective(w, d, bits, period))
    np.testing.assert_array_equal(bits_np(ab0["scales"]), bits)
    np.testing.assert_array_equal(ab0["codes"].cpu().numpy(), ab["codes"].cpu().numpy())


@BOTH
def test_pooled_baseline_entry_matches_fused(method):
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    wt, dt = dev(w), dev(d)
    r = cq.quantize_groups(wt, dt, p, method=method, pooled=True)
    b = cq.baseline_scales(wt, dt, p, "pooled")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_np(b["scales"]), bits_np(r["pooled_scales"]))
    np.testing.assert_array_equal(b["objective"].cpu().numpy(), r["pooled_objective"].cpu().numpy())
    np.testing.assert_array_equal(b["codes"].cpu().numpy(), oracle.codes_for(w, bits_np(b["scales"])))


def test_pack_matches_oracle():
    for (k, m) in ((0, 0), (2, 149)):
        A, dm = W.make_matrix(k, m)
        out, inp = A.shape
        rng = np.random.default_rng(k)
        codes = rng.integers(-8, 8, (out, inp)).astype(np.int8)
        sb = rng.integers(1, 0x7C00, (out, inp // 128)).astype(np.uint16)
        qw, sc = cq.pack_gptq_v1(dev(codes), dev(sb.view(np.int16)), out, inp)
        torch.cuda.synchronize()
        rq, rs = oracle.pack_gptq_v1(codes, sb, out, inp)
        np.testing.assert_array_equal(qw.cpu().numpy(), rq)
        np.testing.assert_array_equal(bits_np(sc), rs)


def test_pack_multi_matches_oracle_per_matrix():
    """Several matrices in one launch, back to back: ragged row counts (a partial 64-row tile, one
    row), an empty matrix, and config 2's shapes; every block equals the oracle's packing of that
    matrix alone."""
    rng = np.random.default_rng(41)
    shapes = [(809, 4096), (0, 256), (64, 256), (803, 4096), (65, 128), (1, 384), (809, 4096)]
    codes = [rng.integers(-8, 8, (o, i)).astype(np.int8) for o, i in shapes]
    sbits = [rng.integers(1, 0x7C00, (o, i // 128)).astype(np.uint16) for o, i in shapes]
    flat_c = np.concatenate([c.ravel() for c in codes])
    flat_s = np.concatenate([b.ravel() for b in sbits])
    qw, sc = cq.pack_gptq_v1_multi(dev(flat_c), dev(flat_s.view(np.int16)), shapes)
    torch.cuda.synchronize()
    qw, sc = qw.cpu().numpy(), bits_np(sc)
    eq = es = 0
    for (o, i), c, b in zip(shapes, codes, sbits):
        rq, rs = oracle.pack_gptq_v1(c, b, o, i)
        np.testing.assert_array_equal(qw[eq:eq + o * i // 8].reshape(i // 8, o), rq)
        np.testing.assert_array_equal(sc[es:es + o * i // 128].reshape(i // 128, o), rs)
        eq += o * i // 8
        es += o * i // 128
    assert eq == qw.size and es == sc.size


def test_pack_multi_all_of_config2_equals_per_matrix_calls():
    """All 150 matrices of config 2 (3,883,008 groups) in one launch against 150 single-matrix calls."""
    spec = W.config(2)
    shapes = [(m.out, m.inp) for m in spec.matrices]
    n_el = sum(o * i for o, i in shapes)
    g = torch.Generator(device="cuda").manual_seed(5)
    codes = torch.randint(-8, 8, (n_el,), dtype=torch.int8, device="cuda", generator=g)
    sc16 = torch.randint(1, 0x7C00, (n_el // 128,), dtype=torch.int16, device="cuda", generator=g)
    qw, sc = cq.pack_gptq_v1_multi(codes, sc16, shapes)
    eq = es = ec = 0
    for o, i in shapes:
        q1, s1 = cq.pack_gptq_v1(codes[ec:ec + o * i].reshape(o, i), sc16[ec // 128:(ec + o * i) // 128].reshape(o, i // 128),
                                 o, i)
        assert torch.equal(qw[eq:eq + o * i // 8], q1.reshape(-1))
        assert torch.equal(sc[es:es + o * i // 128], s1.reshape(-1))
        eq += o * i // 8
        es += o * i // 128
        ec += o * i
    torch.cuda.synchronize()


def test_proxy_matches_oracle():
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    rng = np.random.default_rng(5)
    bits = rng.integers(0x1800, 0x2C00, w.shape[0]).astype(np.uint16)
    mods = np.repeat(np.arange(3), [40, 50, 38])
    off = np.array([0, 40, 90, 128], np.int64)
    pg, mm, macro = cq.proxy_worst_env_wmse(dev(w), dev(d), dev(bits.view(np.int16)), dev(off), p)
    torch.cuda.synchronize()
    rp, rm, rmac = oracle.proxy(w, d, bits, mods, 3, p)
    np.testing.assert_allclose(pg.cpu().numpy(), rp, rtol=1e-6, atol=0)
    np.testing.assert_allclose(mm.cpu().numpy(), rm, rtol=1e-6, atol=0)
    assert abs(macro.cpu().item() - rmac) <= 1e-6 * rmac


@pytest.mark.parametrize("E,n_pol", [(4, 3), (3, 6), (32, 1)])
def test_proxy_multi_matches_single_calls_and_oracle(E, n_pol):
    """Several policies in one call: each policy's per-group values, module means and macro equal
    those of a single-policy call bit for bit, and the oracle's within the proxy tolerance.  The
    group count is not a multiple of the 16 groups of a workgroup, and one module is empty."""
    rng = np.random.default_rng(200 + E)
    n = 16 * 9 + 7
    w = (rng.standard_normal((n, 128)) * 0.02).astype(np.float32)
    d = rng.gamma(0.7, 1.0, (n, E, 128)).astype(np.float32)
    bits = np.stack([rng.integers(0x1400, 0x2400, n) for _ in range(n_pol)]).astype(np.uint16)
    bits[0] = oracle.absmax_bits(w)
    off = np.array([0, 60, 60, 100, n], np.int64)
    mods = np.repeat(np.arange(4), np.diff(off))
    say(f"proxy multi: E={E}, {n_pol} policies, {n} groups")
    wt, dt, ot = dev(w), dev(d), dev(off)
    pg, mm, macro = cq.proxy_worst_env_wmse_multi(wt, dt, dev(bits.view(np.int16)), ot)
    torch.cuda.synchronize()
    pg, mm, macro = pg.cpu().numpy(), mm.cpu().numpy(), macro.cpu().numpy()
    for k in range(n_pol):
        p1, m1, mac1 = cq.proxy_worst_env_wmse(wt, dt, dev(bits[k].view(np.int16)), ot)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(pg[k], p1.cpu().numpy())
        np.testing.assert_array_equal(mm[k], m1.cpu().numpy())
        assert np.isnan(mm[k, 1])
        rp, rm, rmac = oracle.proxy(w, d, bits[k], mods, 4, n)
        np.testing.assert_allclose(pg[k], rp, rtol=1e-6, atol=0)
        # every module, the empty one included: NaN on both sides (no mean of no groups)
        assert np.isnan(rm[1])
        np.testing.assert_allclose(mm[k], rm, rtol=1e-6, atol=0, equal_nan=True)
        assert np.isnan(macro[k]) and np.isnan(mac1.cpu().item()) and np.isnan(rmac)


@BOTH
def test_repeatable(method):
    w, d, p = W.matrix_groups(*W.make_matrix(0, 0))
    a = _run(w, d, p, method)
    b = _run(w, d, p, method)
    for k in ("scales", "codes", "objective", "flags", "pooled_scales", "pooled_objective"):
        assert torch.equal(a[k], b[k]), k
