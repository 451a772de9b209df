"""Benchmark: exact minimax FP16 group-scale selection (W4, groups of 128) on one MI355X.

One step = the whole hot path over config 1 (the MLP block: gate and up 3584x1024, down
1024x3584; 86,016 groups, E = 4): for every matrix, the full-grid exhaustive search (all
31,743 scales for every weight; minimax and the pooled-WMSE policy from the same sums, codes
emitted), the candidate-set solver (which must agree with it), the AbsMax baseline, GPTQ-v1
packing of the minimax codes and scales, and the worst-environment weighted-MSE proxy of the
three policies.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` = groups per second of whole steps; `roofline` describes the
dominant kernel, the full-grid search, on the algorithmic count of every scale of every weight
(31,743 x 128 x (2E + 4) flop per group), with HIP events on its launch stream.  `bounded_path`
times the same step with the branch-and-bound search in place of the full grid (the same
outputs); `config2_pass` runs the candidate solver and one-launch packing over all 3,883,008
groups of config 2; `cpu_baseline` times the CPU oracle on a bounded sample of config 1.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "groups/s exact minimax FP16 scale search (G=128,E=4); % of FP32 VALU peak"
SCALES = 31743
PEAK_FP32_TFLOPS = 157.3  # 256 CU x 4 SIMD x 16 lanes x 2 (dual fp32) x 2 (fma) x 2.4 GHz
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def flops_per_pattern(E: int) -> int:
    """Algorithmic flops of one scale of one group's sweep: per weight one quotient multiply,
    a residual fma (2), a square (1) and E weighted fmas (2E)."""
    return 128 * (2 * E + 4)


def full_grid_flops(n_groups: int, E: int) -> float:
    """Algorithmic flops of the full-grid search of n_groups groups: every scale of every weight."""
    return float(n_groups) * SCALES * flops_per_pattern(E)


def sources_hash(files) -> str:
    """sha256 of the named kernel sources (in csrc/) with comments and blank space removed: a change
    of comments alone leaves the kernel, and the counters taken on it, as they were."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "post_weight_quantization_group_amd", "csrc")
    text = "".join(open(os.path.join(csrc, f)).read() for f in files)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


FULLGRID_SOURCES = ("fullgrid.hip", "device.h", "search_args.h")
BOUNDED_SOURCES = ("sweep.hip", "device.h", "search_args.h")
CANDIDATE_SOURCES = ("candidate.hip", "sweep.hip", "device.h", "search_args.h")


def profile_values(name: str, files) -> dict:
    """The `key: value` lines of a committed counter summary under profiles/, or {} when it is
    missing or was taken on kernel sources other than the current ones (its `sources_sha256`)."""
    import re
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    vals = dict(re.findall(r"^([a-z0-9_]+): (\S+)$", open(path).read(), re.M))
    if vals.get("sources_sha256") != sources_hash(files):
        return {}
    out = {}
    for k, v in vals.items():
        if k == "sources_sha256":
            continue
        try:
            out[k] = float(v) if "." in v or "e" in v else int(v)
        except ValueError:
            out[k] = v
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads() -> int:
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(cores, 256))


def oracle_rate(w, d, budget_s: float, threads: int):
    """(groups, wall seconds) of the oracle as it stands on a prefix of the groups (w, d), one
    diagonal slice per group, sized to about budget_s seconds on `threads` threads after a
    calibration on one group per thread."""
    import oracle
    t0 = time.perf_counter()
    oracle.solve(w[:threads], d[:threads], min(threads, w.shape[0]), n_threads=threads)
    t1 = time.perf_counter() - t0
    n = int(min(w.shape[0], max(threads, budget_s / max(t1, 1e-3) * threads)))
    t0 = time.perf_counter()
    oracle.solve(w[:n], d[:n], n, n_threads=threads)
    return n, time.perf_counter() - t0


def cpu_baseline(k: int, budget_s: float) -> dict:
    """The oracle as it stands (brute force over all 31,743 scales, minimax and pooled from one
    sweep) on the host's cores: a seeded sample of config k sized to about budget_s seconds with
    every core, then 128 groups on one thread."""
    import oracle
    import workloads as W
    threads = host_threads()
    gids = W.sample_groups(k, W.config(k).n_groups, salt=99)
    w, d, _ = W.gather_matrix_groups(k, gids[:max(4096, threads * 64)])
    n, dt = oracle_rate(w, d, budget_s, threads)
    t0 = time.perf_counter()
    oracle.solve(w[:128], d[:128], 128, n_threads=1)
    dt1 = time.perf_counter() - t0
    return {"value": n / dt, "unit": "groups/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} seeded groups of the same workload, brute force over all 31,743 scales "
                      f"(minimax and pooled), {dt:.1f} s wall on {threads} threads",
            "cpu_model": _cpu_model(), "single_thread_groups_per_s": 128 / dt1,
            "single_thread_sample": f"128 groups on one thread, {dt1:.1f} s"}


def _timed(fn, reps=1):
    """(result of the last call, average ms) of fn() on the current stream, after one warm-up."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        out = fn()
    b.record()
    torch.cuda.synchronize()
    return out, a.elapsed_time(b) / reps


def measure_aux() -> dict:
    """The rows beyond the solver: environment diagonals, the W4A16 consumer check and the held-out
    comparison, each on config 1 or config 2 at the pages' sizes; and the full grid on other
    quantizers (code ranges and group lengths)."""
    import torch
    import post_weight_quantization_group_amd as cq
    import workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res = {}
    # environment diagonals from calibration activations: config 1's gate/up (in 1,024) and down
    # (in 3,584) inputs, E = 4, 8,192 bf16 tokens per environment; HBM-bound (2 bytes per element)
    dg = {}
    for m in (0, 2):
        xb = torch.from_numpy(W.calibration_activations(1, m, 8192).view(np.int16)).to(dev)
        E_, T_, n_ = xb.shape
        _, ms = _timed(lambda: cq.environment_diagonals(xb), reps=5)
        nbytes = E_ * T_ * n_ * 2 + n_ * E_ * 4
        dg[f"in{n_}"] = {"E": E_, "tokens_per_env": T_, "ms": ms, "GB_per_s": nbytes / (ms / 1e3) / 1e9,
                         "hbm_frac": nbytes / (ms / 1e3) / 8e12}
        del xb
    res["config1_diagonals"] = dg
    # the W4A16 consumer check: config 1's gate matrix (3584 x 1024) quantized by the exhaustive
    # solver and packed, times M bf16 activation rows, on the matrix cores
    A, dmat = W.make_matrix(1, 0)
    w1, d1, p1 = W.matrix_groups(A, dmat)
    out1, in1 = A.shape
    r1 = cq.quantize_groups(torch.from_numpy(w1).to(dev), torch.from_numpy(d1).to(dev), p1)
    qw1, sc1 = cq.pack_gptq_v1(r1["codes"].reshape(out1, in1), r1["scales"].reshape(out1, in1 // 128), out1, in1)
    xs1 = torch.from_numpy(W.calibration_activations(1, 0, 8192)[0].view(np.int16)).to(dev)
    wq = {}
    for M in (16, 2048, 8192):
        xm = xs1[:M].contiguous()
        _, ms = _timed(lambda: cq.w4a16_matmul(xm, qw1, sc1), reps=10)
        fl = 2.0 * M * out1 * in1
        wq[f"M{M}"] = {"ms": ms, "TFLOP_per_s": fl / (ms / 1e3) / 1e12,
                       "bf16_mfma_frac": fl / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)}
    res["config1_w4a16"] = wq
    # held-out evaluation on config 2: 4,096 groups sampled across all 150 matrices, scales from
    # the calibration diagonals, the three policies' proxy on held-out diagonals, and minimax
    # against pooled with a 10,000-replicate module-stratified bootstrap
    wh, dh, deh, offh = W.heldout_sample(2, 4096)
    nh = wh.shape[0]
    idxh = W.bootstrap_indices(offh, 10000, seed=0)
    wt, dt, det = (torch.from_numpy(x).to(dev) for x in (wh, dh, deh))
    ot, it = torch.from_numpy(offh).to(dev), torch.from_numpy(idxh).to(dev)
    r = cq.quantize_groups(wt, dt, nh, method="exhaustive", pooled=True)
    ab = cq.baseline_scales(wt, dt, nh, "absmax", objective=False)
    sv = torch.stack((r["scales"], r["pooled_scales"], ab["scales"]))
    (pgh, mmh, mach), ms_p = _timed(lambda: cq.proxy_worst_env_wmse_multi(wt, det, sv, ot, nh))
    (cnt, eff, _, ci), ms_h = _timed(lambda: cq.heldout_compare(pgh[0].contiguous(), pgh[1].contiguous(), ot, it))
    macro = mach.cpu().numpy()
    res["config2_heldout"] = {"groups": nh, "modules": int(offh.size - 1), "E": 4, "replicates": 10000,
                              "proxy_macro_minimax_pooled_absmax": [float(x) for x in macro],
                              "minimax_wins_ties_losses_vs_pooled": [int(x) for x in cnt.cpu().numpy()],
                              "effect_pooled_minus_minimax": float(eff.cpu().item()),
                              "effect_ci95": [float(x) for x in ci.cpu().numpy()],
                              "proxy_ms": ms_p, "compare_ms": ms_h}
    # other quantizers (README, "Use the solver": a code range and a group of any length): the
    # full grid on 28,672 seeded groups each, E = 4, every scale of every weight; flops count
    # 31,743 x G x (2E + 4) per group as for the pages' quantizer; the candidate solver beside it
    # where it takes the quantizer
    rng = np.random.default_rng(2024)
    sq = {}
    for qmin, qmax, G in ((-4, 3, 64), (-2, 1, 32), (0, 15, 128), (-128, 127, 256)):
        n, E = 28672, 4
        ws = W.round_bf16((rng.normal(0, 0.02, (n, G)) * np.where(rng.random((n, G)) < 0.01, 8.0, 1.0))
                          .astype(np.float32))
        ds = rng.lognormal(0, 1, (n // 8, E, G)).astype(np.float32)
        wt, dt = torch.from_numpy(ws).to(dev), torch.from_numpy(ds).to(dev)
        r, ms = _timed(lambda: cq.quantize_groups(wt, dt, n // 8, method="exhaustive", qmin=qmin, qmax=qmax), reps=3)
        fl = float(n) * SCALES * G * (2 * E + 4)
        sq[f"q{qmin}..{qmax}_G{G}"] = {"groups": n, "E": E, "ms": ms, "groups_per_s": n / (ms / 1e3),
                                       "TFLOP_per_s": fl / (ms / 1e3) / 1e12,
                                       "frac_fp32_peak": fl / (ms / 1e3) / (PEAK_FP32_TFLOPS * 1e12),
                                       "fp64_sweep_groups": int(torch.count_nonzero(r["flags"] & cq.FLAG_FP64_SWEEP).item()),
                                       "near_tie_groups": int(torch.count_nonzero(r["flags"] & cq.FLAG_NEAR_TIE).item())}
        if G <= 128 and qmin >= -8 and qmax <= 8:
            # the candidate solver on the same groups (its tied groups decided by the full grid)
            rc, msc = _timed(lambda: cq.quantize_groups(wt, dt, n // 8, method="candidate", qmin=qmin, qmax=qmax),
                             reps=3)
            e = sq[f"q{qmin}..{qmax}_G{G}"]
            e["candidate_ms"] = msc
            e["candidate_groups_per_s"] = n / (msc / 1e3)
            e["candidate_fallback_groups"] = int(torch.count_nonzero(rc["flags"] & cq.FLAG_FALLBACK).item())
            e["candidate_vs_full_grid_scale_mismatches"] = int(torch.count_nonzero(rc["scales"] != r["scales"]).item())
    res["spec_quantizers_full_grid"] = sq
    return res


def issue_ceiling() -> dict:
    """The vector units' fp32 fma ceiling as measured: the library's issue probe (eight independent
    fma chains per thread, 2,048 workgroups of 256 threads) in both encodings, each launch timed by
    HIP events, and the shader clock the chip held during it (shader cycles over wall-clock ticks)."""
    import torch
    import post_weight_quantization_group_amd as cq
    blocks, iters = 256 * 8, 200000
    res = {"what": "fp32 fma issue probe (cq_probe_valu_fma): 2,048 workgroups x 256 threads x 8 independent "
                   "chains x 200,000 fmas; v_fma_f32 (three-operand encoding, vector operands), v_fmac_f32 "
                   "(accumulate encoding, the form of the full grid's environment sums) and v_fma_f32 with a "
                   "scalar operand"}
    for mode, name in ((0, "v_fma_f32"), (1, "v_fmac_f32"), (2, "v_fma_f32_scalar_operands")):
        cq.probe_valu_fma(1000, blocks, mode)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = cq.probe_valu_fma(iters, blocks, mode)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        clk = r["clocks"].cpu().numpy().astype(np.float64)
        ghz = clk[:, 0].sum() / clk[:, 1].sum() * r["wall_clock_hz"] / 1e9
        wave_instr = float(blocks) * 4 * 8 * iters
        tflops = wave_instr * 64 * 2 / (ms / 1e3) / 1e12
        res[name] = {"ms": ms, "fp32_TFLOP_per_s": tflops, "frac_of_published_peak": tflops / PEAK_FP32_TFLOPS,
                     "clock_ghz": ghz, "issue_per_cu_clock": wave_instr / (256 * (ms / 1e3) * ghz * 1e9)}
    return res


def config2_pass(dev) -> dict:
    """Config 2 at full size: the candidate solver on every one of the 3,883,008 groups (one call
    per matrix, each with its own diagonals) into codes and scales laid out matrix after matrix,
    then GPTQ-v1 packing of all 150 matrices in one launch.  Returns the timings (HIP events on the
    launch stream) and the fallback count."""
    import torch

    import post_weight_quantization_group_amd as cq
    import workloads as W
    spec = W.config(2)
    mats = []
    for m, mat in enumerate(spec.matrices):
        w, d, p = W.matrix_groups(*W.make_matrix(2, m))
        mats.append((torch.from_numpy(w).to(dev), torch.from_numpy(d).to(dev), p, mat))
    n_all = sum(t[0].shape[0] for t in mats)
    codes = torch.empty((n_all, 128), dtype=torch.int8, device=dev)
    scales = torch.empty(n_all, dtype=torch.int16, device=dev)
    obj = torch.empty(n_all, dtype=torch.float64, device=dev)
    flags = torch.empty(n_all, dtype=torch.uint8, device=dev)
    nmax = max(t[0].shape[0] for t in mats)
    ws = torch.empty(cq.cq_workspace_size(cq.CANDIDATE, 4, nmax), dtype=torch.uint8, device=dev)
    shapes = [(t[3].out, t[3].inp) for t in mats]
    qweight = torch.empty(n_all * 16, dtype=torch.int32, device=dev)
    qscales = torch.empty(n_all, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    def solve():
        g0 = 0
        for w, d, p, _ in mats:
            n = w.shape[0]
            cq.cq_quantize_groups(w, d, p, 4, n, cq.CANDIDATE, scales[g0:g0 + n], codes[g0:g0 + n],
                                  obj[g0:g0 + n], flags[g0:g0 + n], None, None, ws)
            g0 += n

    def pack():
        cq.cq_pack_gptq_v1_multi(codes, scales, len(shapes), [o for o, _ in shapes], [i for _, i in shapes],
                                 qweight, qscales)
    solve()
    pack()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    reps = 3
    t_solve = t_pack = 0.0
    for _ in range(reps):
        ev[0].record(stream)
        solve()
        ev[1].record(stream)
        pack()
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_solve += ev[0].elapsed_time(ev[1]) / reps
        t_pack += ev[1].elapsed_time(ev[2]) / reps
    fb = int(torch.count_nonzero(flags & cq.FLAG_FALLBACK).item())
    pack_bytes = n_all * (128 + 2 + 64 + 2)
    return {"groups": n_all, "E": 4, "candidate_ms": t_solve, "candidate_groups_per_s": n_all / t_solve * 1e3,
            "candidate_fallback_groups": fb, "pack_ms": t_pack, "pack_launches": 1,
            "pack_GB_per_s": pack_bytes / (t_pack / 1e3) / 1e9, "pack_hbm_frac": pack_bytes / (t_pack / 1e3) / 8e12,
            "pack_bytes": pack_bytes}


def measure_all_configs(oracle_budget_s=None) -> dict:
    """Throughput of every kernel on the five synthetic configs (reported beside the headline).

    config 0/1/4: full grid (minimax + pooled from the same sums), bounded search, candidate,
    AbsMax, pack, proxies; config 2: the full-size candidate and packing pass plus the seeded
    10,000-group sample through the full grid and the bounded search; config 3: every search on all
    262,144 groups.  Fractions of the FP32 peak count every scale of every weight (full grid).
    With oracle_budget_s, the oracle is timed beside each config on the host's cores, on a prefix
    of that config's seeded oracle sample (all of config 0; config 2's 10,000-group sample; seeded
    samples of the others) sized to about that many seconds.
    """
    import torch

    import post_weight_quantization_group_amd as cq
    import workloads as W
    dev = torch.device("cuda:0")
    res = {}
    peak = PEAK_FP32_TFLOPS * 1e12

    def searches(wt, dt, p, n, E, pooled, tot):
        r, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="exhaustive", pooled=pooled))
        tot["full_ms"] += ms
        b, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="bounded", pooled=pooled))
        tot["bounded_ms"] += ms
        c, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="candidate"))
        tot["candidate_ms"] += ms
        tot["fallback"] += int(torch.count_nonzero(c["flags"] & cq.FLAG_FALLBACK).item())
        tot["fp64_sweep"] += int(torch.count_nonzero(r["flags"] & cq.FLAG_FP64_SWEEP).item())
        tot["mismatch"] += int(torch.count_nonzero(r["scales"] != c["scales"]).item())
        tot["mismatch"] += int(torch.count_nonzero(r["scales"] != b["scales"]).item())
        tot["groups"] += n
        tot["flops"] += full_grid_flops(n, E)
        return r

    def summary(tot, E):
        return {"groups": tot["groups"], "E": E,
                "full_grid_groups_per_s": tot["groups"] / tot["full_ms"] * 1e3,
                "full_grid_frac_fp32_peak": tot["flops"] / (tot["full_ms"] / 1e3) / peak,
                "bounded_groups_per_s": tot["groups"] / tot["bounded_ms"] * 1e3,
                "candidate_groups_per_s": tot["groups"] / tot["candidate_ms"] * 1e3,
                "candidate_fallback_groups": tot["fallback"], "full_grid_fp64_sweep_groups": tot["fp64_sweep"],
                "scale_mismatches_between_methods": tot["mismatch"]}

    def new_tot():
        return {"full_ms": 0.0, "bounded_ms": 0.0, "candidate_ms": 0.0, "absmax_ms": 0.0, "pack_ms": 0.0,
                "proxy_ms": 0.0, "groups": 0, "fallback": 0, "fp64_sweep": 0, "mismatch": 0, "flops": 0.0}

    def matrix_pass(k):
        spec = W.config(k)
        E = spec.E
        tot = new_tot()
        module_means = {"minimax": [], "pooled": [], "absmax": []}
        for m, mat in enumerate(spec.matrices):
            w, d, p = W.matrix_groups(*W.make_matrix(k, m))
            n = w.shape[0]
            wt, dt = torch.from_numpy(w).to(dev), torch.from_numpy(d).to(dev)
            r = searches(wt, dt, p, n, E, True, tot)
            ab, ms = _timed(lambda: cq.baseline_scales(wt, dt, p, "absmax", objective=False))
            tot["absmax_ms"] += ms
            codes = r["codes"].reshape(mat.out, mat.inp)
            sc = r["scales"].reshape(mat.out, mat.inp // 128)
            _, ms = _timed(lambda: cq.pack_gptq_v1(codes, sc, mat.out, mat.inp))
            tot["pack_ms"] += ms
            off = torch.tensor([0, n], dtype=torch.int64, device=dev)
            sv = torch.stack((r["scales"], r["pooled_scales"], ab["scales"]))
            (_, mm, _), ms = _timed(lambda: cq.proxy_worst_env_wmse_multi(wt, dt, sv, off, p, per_group=False))
            tot["proxy_ms"] += ms
            for j, name in enumerate(("minimax", "pooled", "absmax")):
                module_means[name].append(float(mm.cpu()[j, 0]))
        out = summary(tot, E)
        out.update({"absmax_groups_per_s": tot["groups"] / tot["absmax_ms"] * 1e3, "pack_ms": tot["pack_ms"],
                    "proxy_ms": tot["proxy_ms"],
                    "proxy_module_macro": {k2: float(np.mean(v)) for k2, v in module_means.items()}})
        return out

    threads = host_threads()

    def oracle_beside(w, d, what):
        n, dt = oracle_rate(w, d, oracle_budget_s, threads)
        return {"groups": n, "wall_s": dt, "groups_per_s": n / dt, "threads": threads,
                "sample": f"the first {n} of {what}, brute force over all 31,743 scales (minimax and pooled)"}

    for k in (0, 1, 4):
        res[f"config{k}"] = matrix_pass(k)
        if oracle_budget_s:
            count = {0: 128, 1: 8192, 4: 16384}[k]
            gids = W.sample_groups(k, count, salt=99)
            wo, do, _ = W.gather_matrix_groups(k, gids)
            res[f"config{k}"]["oracle"] = oracle_beside(wo, do, f"{gids.size} seeded groups")
    res.update(measure_aux())
    res["config2"] = config2_pass(dev)
    gids = W.sample_groups(2, 10000)
    ws_, ds_, _ = W.gather_matrix_groups(2, gids)
    tot = new_tot()
    searches(torch.from_numpy(ws_).to(dev), torch.from_numpy(ds_).to(dev), ws_.shape[0], ws_.shape[0], 4, True, tot)
    res["config2"]["sample"] = summary(tot, 4)
    if oracle_budget_s:
        res["config2"]["sample"]["oracle"] = oracle_beside(ws_, ds_, "the seeded 10,000-group sample")
    w3, d3, _, _ = W.make_groups(3)
    tot = new_tot()
    searches(torch.from_numpy(w3).to(dev), torch.from_numpy(d3).to(dev), w3.shape[0], w3.shape[0], 8, True, tot)
    res["config3"] = summary(tot, 8)
    if oracle_budget_s:
        gids = W.sample_groups(3, 65536, salt=99)
        res["config3"]["oracle"] = oracle_beside(w3[gids], d3[gids], "65,536 seeded groups")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-config2", action="store_true", help="skip the full-size config 2 candidate and packing pass")
    ap.add_argument("--no-bounded", action="store_true", help="skip the step with the bounded search")
    ap.add_argument("--aux-only", action="store_true",
                    help="only measure the diagonals, W4A16 and held-out rows (one JSON line, no step)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also measure every kernel on the five synthetic configs (adds 'per_config')")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a plain copy kernel of known "
                         "size, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): every group is independent, "
              "so several GPUs would each run this same benchmark on their own share.", file=sys.stderr)
        sys.exit(2)

    if args.aux_only:
        print(json.dumps({"aux": measure_aux()}), flush=True)
        return

    import torch

    import post_weight_quantization_group_amd as cq
    import workloads as W

    k = 1
    spec = W.config(k)
    E = spec.E
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    mats = []
    for m, mat in enumerate(spec.matrices):
        A, dm = W.make_matrix(k, m)
        w, d, p = W.matrix_groups(A, dm)
        n = w.shape[0]
        t = {
            "name": mat.name, "out": mat.out, "inp": mat.inp, "n": n, "p": p,
            "w": torch.from_numpy(w).to(dev), "d": torch.from_numpy(d).to(dev),
            "sc3": torch.empty((3, n), dtype=torch.int16, device=dev),
            "codes": torch.empty((n, 128), dtype=torch.int8, device=dev),
            "obj": torch.empty(n, dtype=torch.float64, device=dev),
            "flags": torch.empty(n, dtype=torch.uint8, device=dev),
            "pobj": torch.empty(n, dtype=torch.float64, device=dev),
            "cscales": torch.empty(n, dtype=torch.int16, device=dev),
            "ccodes": torch.empty((n, 128), dtype=torch.int8, device=dev),
            "cobj": torch.empty(n, dtype=torch.float64, device=dev),
            "cflags": torch.empty(n, dtype=torch.uint8, device=dev),
            "acodes": torch.empty((n, 128), dtype=torch.int8, device=dev),
            "aobj": torch.empty(n, dtype=torch.float64, device=dev),
            "qweight": torch.empty((mat.inp // 8, mat.out), dtype=torch.int32, device=dev),
            "qscales": torch.empty((mat.inp // 128, mat.out), dtype=torch.int16, device=dev),
            "ws": torch.empty(cq.cq_workspace_size(cq.EXHAUSTIVE, E, n), dtype=torch.uint8, device=dev),
            "cws": torch.empty(cq.cq_workspace_size(cq.CANDIDATE, E, n), dtype=torch.uint8, device=dev),
            "off": torch.tensor([0, n], dtype=torch.int64, device=dev),
            "mm": torch.empty((3, 1), dtype=torch.float64, device=dev),
            "macro": torch.empty((3, 1), dtype=torch.float64, device=dev),
            "pg": torch.empty((3, n), dtype=torch.float64, device=dev),
        }
        t["scales"], t["pscales"], t["ascales"] = t["sc3"][0], t["sc3"][1], t["sc3"][2]
        mats.append(t)
    n_total = sum(t["n"] for t in mats)
    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step(method, ev):
        """The whole path over config 1 with `method` deciding minimax and pooled; launches of the
        search and of the candidate solver bracketed by HIP events on the launch stream."""
        for t in mats:
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3)) if ev is not None else (None,) * 3
            if a is not None:
                a.record(stream)
            cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], method, t["scales"], t["codes"],
                                  t["obj"], t["flags"], t["pscales"], t["pobj"], t["ws"])
            if b is not None:
                b.record(stream)
            cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], cq.CANDIDATE, t["cscales"],
                                  t["ccodes"], t["cobj"], t["cflags"], None, None, t["cws"])
            if c is not None:
                c.record(stream)
                ev.append((a, b, c, t))
            cq.cq_baseline_scales(t["w"], t["d"], t["p"], E, t["n"], cq.ABSMAX, t["ascales"], t["acodes"],
                                  t["aobj"])
            cq.cq_pack_gptq_v1(t["codes"], t["scales"], t["out"], t["inp"], t["qweight"], t["qscales"])
            # minimax, pooled and AbsMax scales are the rows of sc3: one proxy pass for all three
            cq.cq_proxy_worst_env_wmse_multi(t["w"], t["d"], t["p"], E, t["n"], 3, t["sc3"], t["off"], 1, t["mm"],
                                             t["macro"], t["pg"])

    def timed_steps(method, steps, warmup):
        for _ in range(warmup):
            step(method, None)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev = []
        wall0 = time.perf_counter()
        t0.record(stream)
        for _ in range(steps):
            step(method, ev)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = t0.elapsed_time(t1) / steps
        search_ms = float(np.mean([a.elapsed_time(b) for a, b, _, _ in ev]))
        cand_ms = float(np.mean([b.elapsed_time(c) for _, b, c, _ in ev]))
        return ms_step, search_ms, cand_ms, wall

    ms_step, full_ms, cand_ms, wall = timed_steps(cq.EXHAUSTIVE, args.steps, args.warmup)
    value = n_total / (ms_step / 1e3)
    flags = torch.cat([t["flags"] for t in mats])
    cflags = torch.cat([t["cflags"] for t in mats])
    mism = sum(int(torch.count_nonzero(t["scales"] != t["cscales"]).item()) for t in mats)
    groups_per_launch = float(np.mean([t["n"] for t in mats]))
    flops_per_launch = full_grid_flops(groups_per_launch, E)
    achieved = flops_per_launch / (full_ms / 1e3) / 1e12
    fg = profile_values("fullgrid_config1_counters.md", FULLGRID_SOURCES)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "groups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "config 1: " + spec.description, "groups": n_total, "E": E,
                   "matrices": [f"{t['name']} {t['out']}x{t['inp']}" for t in mats],
                   "step": "per matrix: full-grid exhaustive search (minimax and pooled, codes), candidate-set "
                           "solver, AbsMax, GPTQ-v1 packing, proxy of the three policies"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_TFLOPS, "traffic": fg.get("traffic_bytes_per_launch"),
                     "kernel": "full-grid exhaustive search (cq_quantize_groups, CQ_EXHAUSTIVE: "
                               "full_screen_kernel<4> plus two short launches)",
                     "launch_ms": full_ms, "groups_per_launch": groups_per_launch,
                     "flops_per_launch": flops_per_launch,
                     "flops_per_group": SCALES * flops_per_pattern(E),
                     "counting": "31,743 scales x 128 weights x (2E + 4) flop per group: a quotient multiply, "
                                 "a residual fma (2), a square and E weighted fmas (2E); 'executed' gives the fp32 "
                                 "work the counters show executed (terms whose code is proven constant over a "
                                 "chunk skip the quotient)"},
        "full_grid_groups_per_s": groups_per_launch / (full_ms / 1e3),
        "candidate_launch_ms": cand_ms,
        "candidate_vs_full_grid_scale_mismatches": mism,
        "flag_counts": {"near_tie": int(torch.count_nonzero(flags & 2).item()),
                        "exact_tie": int(torch.count_nonzero(flags & 4).item()),
                        "fp64_sweep": int(torch.count_nonzero(flags & 16).item()),
                        "candidate_fallback": int(torch.count_nonzero(cflags & 8).item())},
        "wall_s": wall,
    }
    if fg:
        line["roofline"]["counters"] = {k2: v for k2, v in fg.items() if k2 != "traffic_bytes_per_launch"}
        if "fp32_flop_executed_per_launch" in fg:
            # the fp32 work the kernel executes (counters), over the same launch time: runs of weights
            # whose code is proven constant over a chunk take it from the row, without the quotient
            ex = fg["fp32_flop_executed_per_launch"] / (full_ms / 1e3) / 1e12
            line["roofline"]["executed"] = {"fp32_flop_per_launch": fg["fp32_flop_executed_per_launch"],
                                             "of_algorithmic": fg["fp32_flop_executed_per_launch"] / flops_per_launch,
                                             "achieved": ex, "frac": ex / PEAK_FP32_TFLOPS}
    ceil = issue_ceiling()
    ceil["full_grid_frac_of_measured"] = achieved / ceil["v_fmac_f32"]["fp32_TFLOP_per_s"]
    line["roofline"]["measured_ceiling"] = ceil
    if not args.no_bounded:
        ms_b, bnd_ms, cand_b, wall_b = timed_steps(cq.BOUNDED, args.steps, args.warmup)
        line["bounded_path"] = {
            "what": "the same step with the branch-and-bound search (CQ_BOUNDED) in place of the full grid: "
                    "the same outputs",
            "groups_per_s": n_total / (ms_b / 1e3), "ms_per_step": ms_b,
            "bounded_launch_ms": bnd_ms, "candidate_launch_ms": cand_b,
            "counters": profile_values("bounded_candidate_config1_counters.md", CANDIDATE_SOURCES) or None}
    if not args.no_config2:
        line["config2_pass"] = config2_pass(dev)
    if args.all_configs:
        line["per_config"] = measure_all_configs(None if args.no_cpu_baseline else args.cpu_budget / 2)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(k, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
