"""Benchmark: exact minimax FP16 group-scale selection (W4, groups of 128) on one MI355X.

One step = the whole hot path over one batch: for every matrix of the workload, the
exhaustive minimax sweep (the pooled-WMSE policy decided in the same sweep, codes emitted),
the candidate-set solver, the AbsMax baseline, GPTQ-v1 packing of the minimax codes and
scales, and the worst-environment weighted-MSE proxy for the three policies.  Inputs are
resident in HBM before timing starts.

Prints one JSON line.  `value` = groups per second of whole steps; `roofline` describes the
headline kernel (the binary32 exhaustive sweep) measured with HIP events on its own stream;
`cpu_baseline` times the CPU oracle on a bounded sample of the same groups.
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


def screened_patterns(w: np.ndarray) -> np.ndarray:
    """Scale patterns the exhaustive sweep evaluates per group: 1 up to the first binary16 scale
    >= 2 max|w| (every one when 2 max|w| > 65504).  From there on every code is 0 and the
    objective is the same value at every pattern, so the lowest of them stands for all."""
    grid = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    t = 2.0 * np.abs(w.astype(np.float64)).max(axis=1)
    return np.minimum(np.searchsorted(grid, t, side="left") + 1, SCALES)


def active_terms(w: np.ndarray) -> float:
    """Terms (scale, weight) over the screened patterns whose code is neither 0 nor held at the
    clip end.  Weight i has code 0 at scale s when s >= 2|w_i|, and its code is held at 7 (w > 0)
    or -8 (w < 0) for every scale below w/6.5 (w > 0) or up to |w|/7.5 (w < 0).  Both kinds of
    term have a closed form at every scale (d w^2, and a quadratic in s with fixed coefficients),
    so the sweep sums them once per chunk of scales; the active ones each take a quotient, a
    rounding, a residual, a square and E weighted sums."""
    grid = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    a = np.abs(w.astype(np.float64))
    top = screened_patterns(w)[:, None]
    nonzero = np.minimum(np.searchsorted(grid, 2.0 * a, side="left"), top)
    held = np.where(w > 0, np.searchsorted(grid, a / 6.5, side="left"),
                    np.searchsorted(grid, a / 7.5, side="right"))
    held = np.minimum(np.where(w == 0, 0, held), top)
    return float((nonzero - held).sum())


def necessary_terms(w: np.ndarray, d: np.ndarray, opt_m: np.ndarray, opt_p: np.ndarray, chunk: int = 128):
    """Active terms (see active_terms) of the chunks of `chunk` consecutive patterns that the
    binary32 screen cannot skip, per group, and the number of those chunks.  The screen skips a
    chunk when a lower bound on the objective over it exceeds 1.001 times the best value screened
    so far, for minimax and for pooled; the bound is the code-0 prefix sum (weights with clip key
    <= s_lo/15) plus, for weights clipped throughout (clip key > s_hi), d (|w| - |q| s_hi)^2 when
    positive.  The best value screened is never below the optimum, so every chunk whose bound is
    at most 1.0009 times the optimum (binary64 here, a margin for the screen's binary32) is
    screened: the count is a lower bound on the work done.  w [n, 128], d [n, E, 128], opt_m the
    minimax optimum and opt_p the pooled optimum times E (a sum over environments)."""
    grid = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    top = screened_patterns(w)
    w64, d64 = w.astype(np.float64), d.astype(np.float64)
    a = np.abs(w64)
    nonzero = np.minimum(np.searchsorted(grid, 2.0 * a, side="left"), top[:, None])
    held = np.where(w64 > 0, np.searchsorted(grid, a / 6.5, side="left"), np.searchsorted(grid, a / 7.5, side="right"))
    held = np.minimum(np.where(w64 == 0, 0, held), top[:, None])
    key = np.where(w64 > 0, w64 / 6.5, a / 7.5)
    qa = np.where(w64 > 0, 7.0, 8.0)
    terms = np.zeros(w.shape[0])
    chunks = np.zeros(w.shape[0])
    for j in range(w.shape[0]):
        nch = (int(top[j]) - 1) // chunk + 1
        c0 = np.arange(nch) * chunk                        # first pattern index (0-based) of each chunk
        c1 = np.minimum(c0 + chunk, int(top[j]))           # one past the last
        lo, hi = grid[c0], grid[c1 - 1]
        zmask = key[j][None, :] <= lo[:, None] / 15.0      # [nch, 128]
        cmask = key[j][None, :] > hi[:, None]
        t = np.maximum(0.0, a[j][None, :] - qa[j][None, :] * hi[:, None]) * cmask
        zt = np.where(zmask, a[j][None, :] ** 2, 0.0)
        lb = np.einsum("ce,ke->kc", d64[j], t * t + zt)   # [nch, E]
        need = lb.max(axis=1) <= 1.0009 * opt_m[j]
        if opt_p is not None:
            need |= lb.sum(axis=1) <= 1.0009 * opt_p[j]
        ov = np.minimum(nonzero[j][None, :], c1[:, None]) - np.maximum(held[j][None, :], c0[:, None])
        terms[j] = np.clip(ov, 0, None)[need].sum()
        chunks[j] = need.sum()
    return terms, chunks


def sampled_sweep_flops(w: np.ndarray, d: np.ndarray, d_period: int, r: dict, E: int, pooled: bool,
                        n_sample: int = 512, seed: int = 2024) -> float:
    """The sweep's work over all groups of w (2E + 4 flops per unskippable active term, see
    necessary_terms), from a seeded sample of its groups and the optima in r (quantize_groups)."""
    rng = np.random.default_rng(seed)
    n = w.shape[0]
    idx = np.sort(rng.choice(n, size=min(n_sample, n), replace=False))
    om = r["objective"].cpu().numpy()[idx]
    op = r["pooled_objective"].cpu().numpy()[idx] * E if pooled else None
    terms, _ = necessary_terms(w[idx], d[idx % d_period], om, op, chunk=128)
    return float(terms.mean()) * n * (2 * E + 4)


def sweep_flops(w: np.ndarray, E: int) -> float:
    """Algorithmic flops of the exhaustive sweep over the groups w [n, 128]: 2E + 4 per active
    term (a quotient multiply, a residual fma, a square and E weighted fmas)."""
    return active_terms(w) * (2 * E + 4)


def full_grid_flops(n_groups: int, E: int) -> float:
    """The same count for a plain sweep of every weight at every one of the 31,743 scales."""
    return float(n_groups) * SCALES * flops_per_pattern(E)


def sweep_traffic(config: int):
    """HBM bytes per sweep launch from the committed counter summary (FETCH_SIZE and WRITE_SIZE
    passes, each scaled by a 256 MiB device copy), or None when that summary is missing, covers
    another workload, or was taken on sweep sources other than the current ones."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "sweep_f32_config1_hbm_counters.md")
    if config != 1 or not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    h = re.search(r"^sweep_sources_sha256: ([0-9a-f]{64})$", text, re.M)
    if not t or not h:
        return None
    return int(t.group(1)) if sweep_sources_hash() == h.group(1) else None


def sweep_sources_hash() -> str:
    """sha256 of the sweep's sources (sweep.hip, device.h, launch.h) with comments and blank
    space removed: a change of comments alone leaves the kernel, and its counters, as they were."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "post_weight_quantization_group_amd", "csrc")
    text = "".join(open(os.path.join(csrc, f)).read() for f in ("sweep.hip", "device.h", "launch.h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


def cpu_baseline(k: int, budget_s: float) -> dict:
    import oracle
    import workloads as W
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(cores, 256))
    gids = W.sample_groups(k, W.config(k).n_groups, salt=99)
    w, d, _ = W.gather_matrix_groups(k, gids)
    # calibrate on one group per thread, then size the sample to the time budget
    t0 = time.perf_counter()
    oracle.solve(w[:threads], d[:threads], threads, n_threads=threads)
    t1 = time.perf_counter() - t0
    n = int(min(w.shape[0], max(threads, budget_s / max(t1, 1e-3) * threads)))
    t0 = time.perf_counter()
    oracle.solve(w[:n], d[:n], n, n_threads=threads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "groups/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} seeded groups of the same workload, brute force over all 31,743 scales "
                      f"(minimax and pooled), {dt:.1f} s wall"}


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
    comparison, each on config 1 or config 2 at the pages' sizes."""
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
    return res


def measure_all_configs() -> dict:
    """Throughput of every kernel on the five synthetic configs (reported beside the headline).

    config 0/1/4: exhaustive (minimax + pooled in one sweep), candidate, AbsMax, pack, proxies;
    config 2: candidate, pack and proxy on all 150 matrices, exhaustive on the seeded
    10,000-group sample; config 3: exhaustive and candidate on all 262,144 groups.
    """
    import torch

    import post_weight_quantization_group_amd as cq
    import workloads as W
    dev = torch.device("cuda:0")
    res = {}

    def matrix_pass(k, mats_idx=None):
        spec = W.config(k)
        E = spec.E
        idx = range(len(spec.matrices)) if mats_idx is None else mats_idx
        tot = {"exhaustive_ms": 0.0, "candidate_ms": 0.0, "absmax_ms": 0.0, "pack_ms": 0.0, "proxy_ms": 0.0,
               "groups": 0, "fallback": 0, "fp64_sweep": 0, "mismatch": 0, "flops": 0.0}
        module_means = {"minimax": [], "pooled": [], "absmax": []}
        for m in idx:
            mat = spec.matrices[m]
            w, d, p = W.matrix_groups(*W.make_matrix(k, m))
            n = w.shape[0]
            wt, dt = torch.from_numpy(w).to(dev), torch.from_numpy(d).to(dev)
            r, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="exhaustive", pooled=True))
            tot["exhaustive_ms"] += ms
            tot["flops"] += sampled_sweep_flops(w, d, p, r, E, True)
            c, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="candidate"))
            tot["candidate_ms"] += ms
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
            f = c["flags"].cpu().numpy()
            tot["fallback"] += int(np.count_nonzero(f & cq.FLAG_FALLBACK))
            tot["fp64_sweep"] += int(np.count_nonzero(r["flags"].cpu().numpy() & cq.FLAG_FP64_SWEEP))
            tot["mismatch"] += int(torch.count_nonzero(r["scales"] != c["scales"]).item())
            tot["groups"] += n
        out = {"groups": tot["groups"], "E": E,
               "exhaustive_groups_per_s": tot["groups"] / tot["exhaustive_ms"] * 1e3,
               "exhaustive_frac_fp32_peak": tot["flops"] / (tot["exhaustive_ms"] / 1e3) / (PEAK_FP32_TFLOPS * 1e12),
               "candidate_groups_per_s": tot["groups"] / tot["candidate_ms"] * 1e3,
               "candidate_hbm_frac": tot["groups"] * 642 / (tot["candidate_ms"] / 1e3) / 8e12,
               "absmax_groups_per_s": tot["groups"] / tot["absmax_ms"] * 1e3,
               "pack_ms": tot["pack_ms"], "pack_hbm_frac": tot["groups"] * 196 / (tot["pack_ms"] / 1e3) / 8e12,
               "proxy_ms": tot["proxy_ms"],
               "candidate_fallback_groups": tot["fallback"], "exhaustive_fp64_sweep_groups": tot["fp64_sweep"],
               "candidate_vs_exhaustive_scale_mismatches": tot["mismatch"],
               "proxy_module_macro": {k2: float(np.mean(v)) for k2, v in module_means.items()}}
        return out

    res["config0"] = matrix_pass(0)
    res["config1"] = matrix_pass(1)
    res["config4"] = matrix_pass(4)
    res.update(measure_aux())
    # config 2: candidate + pack + proxy on every matrix, exhaustive on the 10,000-group sample
    spec = W.config(2)
    cand_ms = pack_ms = proxy_ms = 0.0
    fb = n_all = 0
    means = []
    for m, mat in enumerate(spec.matrices):
        w, d, p = W.matrix_groups(*W.make_matrix(2, m))
        n = w.shape[0]
        wt, dt = torch.from_numpy(w).to(dev), torch.from_numpy(d).to(dev)
        c, ms = _timed(lambda: cq.quantize_groups(wt, dt, p, method="candidate"))
        cand_ms += ms
        codes = c["codes"].reshape(mat.out, mat.inp)
        sc = c["scales"].reshape(mat.out, mat.inp // 128)
        _, ms = _timed(lambda: cq.pack_gptq_v1(codes, sc, mat.out, mat.inp))
        pack_ms += ms
        off = torch.tensor([0, n], dtype=torch.int64, device=dev)
        (_, mm, _), ms = _timed(lambda: cq.proxy_worst_env_wmse(wt, dt, c["scales"], off, p, per_group=False))
        proxy_ms += ms
        means.append(float(mm.cpu()[0]))
        fb += int(np.count_nonzero(c["flags"].cpu().numpy() & cq.FLAG_FALLBACK))
        n_all += n
    gids = W.sample_groups(2, 10000)
    ws_, ds_, _ = W.gather_matrix_groups(2, gids)
    wt, dt = torch.from_numpy(ws_).to(dev), torch.from_numpy(ds_).to(dev)
    r, ms_x = _timed(lambda: cq.quantize_groups(wt, dt, ws_.shape[0], method="exhaustive"))
    c, ms_c = _timed(lambda: cq.quantize_groups(wt, dt, ws_.shape[0], method="candidate"))
    res["config2"] = {"groups": n_all, "E": 4, "candidate_groups_per_s": n_all / cand_ms * 1e3,
                      "candidate_hbm_frac": n_all * 642 / (cand_ms / 1e3) / 8e12,
                      "candidate_ms": cand_ms, "candidate_fallback_groups": fb,
                      "pack_ms": pack_ms, "pack_hbm_frac": n_all * 196 / (pack_ms / 1e3) / 8e12,
                      "proxy_ms": proxy_ms, "proxy_module_macro_minimax": float(np.mean(means)),
                      "sample_groups": int(ws_.shape[0]),
                      "sample_exhaustive_groups_per_s": ws_.shape[0] / ms_x * 1e3,
                      "sample_exhaustive_frac_fp32_peak":
                          sampled_sweep_flops(ws_, ds_, ws_.shape[0], r, 4, False) / (ms_x / 1e3)
                          / (PEAK_FP32_TFLOPS * 1e12),
                      "sample_candidate_vs_exhaustive_scale_mismatches":
                          int(torch.count_nonzero(r["scales"] != c["scales"]).item())}
    # config 3: per-group diagonals
    w3, d3, cat3, _ = W.make_groups(3)
    n3 = w3.shape[0]
    wt, dt = torch.from_numpy(w3).to(dev), torch.from_numpy(d3).to(dev)
    r, ms_x = _timed(lambda: cq.quantize_groups(wt, dt, n3, method="exhaustive", pooled=False))
    flops3 = sampled_sweep_flops(w3, d3, n3, r, 8, False)
    del d3
    c, ms_c = _timed(lambda: cq.quantize_groups(wt, dt, n3, method="candidate"))
    fl = c["flags"].cpu().numpy()
    res["config3"] = {"groups": n3, "E": 8, "exhaustive_groups_per_s": n3 / ms_x * 1e3,
                      "exhaustive_frac_fp32_peak": flops3 / (ms_x / 1e3) / (PEAK_FP32_TFLOPS * 1e12),
                      "candidate_groups_per_s": n3 / ms_c * 1e3,
                      "candidate_fallback_groups": int(np.count_nonzero(fl & cq.FLAG_FALLBACK)),
                      "exhaustive_fp64_sweep_groups": int(np.count_nonzero(r["flags"].cpu().numpy() & cq.FLAG_FP64_SWEEP)),
                      "candidate_vs_exhaustive_scale_mismatches":
                          int(torch.count_nonzero(r["scales"] != c["scales"]).item())}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-candidate", action="store_true")
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

    spec = W.config(args.config)
    if spec.per_group:
        raise SystemExit("the benchmark workload is a matrix config")
    E = spec.E
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    mats = []
    for m, mat in enumerate(spec.matrices):
        A, dm = W.make_matrix(args.config, m)
        w, d, p = W.matrix_groups(A, dm)
        n = w.shape[0]
        t = {
            "name": mat.name, "out": mat.out, "inp": mat.inp, "n": n, "p": p,
            "w_np": w, "d_np": d, "patterns": float(screened_patterns(w).mean()),
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
    use_candidate = not args.no_candidate
    if use_candidate:
        try:
            t = mats[0]
            cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], cq.CANDIDATE, t["cscales"], t["ccodes"],
                                  t["cobj"], t["cflags"], None, None, t["cws"])
        except cq.CQError:
            use_candidate = False
    torch.cuda.synchronize()

    sweep_ev = []

    def step(record):
        for t in mats:
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], cq.EXHAUSTIVE, t["scales"], t["codes"],
                                  t["obj"], t["flags"], t["pscales"], t["pobj"], t["ws"])
            if record:
                b.record(stream)
                sweep_ev.append((a, b, t))
            if use_candidate:
                cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], cq.CANDIDATE, t["cscales"],
                                      t["ccodes"], t["cobj"], t["cflags"], None, None, t["cws"])
            cq.cq_baseline_scales(t["w"], t["d"], t["p"], E, t["n"], cq.ABSMAX, t["ascales"], t["acodes"],
                                  t["aobj"])
            cq.cq_pack_gptq_v1(t["codes"], t["scales"], t["out"], t["inp"], t["qweight"], t["qscales"])
            # minimax, pooled and AbsMax scales are the rows of sc3: one proxy pass for all three
            cq.cq_proxy_worst_env_wmse_multi(t["w"], t["d"], t["p"], E, t["n"], 3, t["sc3"], t["off"], 1, t["mm"],
                                             t["macro"], t["pg"])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step(True)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    value = n_total / (ms_step / 1e3)

    # headline kernel: the exhaustive sweep call, per launch (one launch per matrix).  Its work:
    # the active terms of the chunks no exact screen with its lower bound can skip, per group from
    # a seeded sample of 1,024 groups per matrix (against the optima the sweep returned), times
    # 2E + 4 flops; chunks of 128 patterns as in the kernel.
    rng = np.random.default_rng(2024)
    nec_chunks, all_terms = [], []
    for t in mats:
        idx = np.sort(rng.choice(t["n"], size=min(1024, t["n"]), replace=False))
        om = t["obj"].cpu().numpy()[idx]
        op = t["pobj"].cpu().numpy()[idx] * E
        terms, chunks = necessary_terms(t["w_np"][idx], t["d_np"][idx % t["p"]], om, op, chunk=128)
        t["flops"] = float(terms.mean()) * t["n"] * (2 * E + 4)
        nec_chunks.append(float(chunks.mean()))
        all_terms.append(active_terms(t["w_np"][idx]) / idx.size)
    durs = [a.elapsed_time(b) for a, b, _ in sweep_ev]
    avg_ms = float(np.mean(durs))
    avg_groups = float(np.mean([t["n"] for _, _, t in sweep_ev]))
    avg_flops = float(np.mean([t["flops"] for _, _, t in sweep_ev]))
    achieved = avg_flops / (avg_ms / 1e3) / 1e12
    patterns = float(np.mean([t["patterns"] for t in mats]))
    flags = torch.cat([t["flags"] for t in mats]).cpu().numpy()

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
        "config": {"workload": f"config {args.config}: " + spec.description, "groups": n_total, "E": E,
                   "matrices": [f"{t['name']} {t['out']}x{t['inp']}" for t in mats],
                   "candidate_solver_in_step": use_candidate},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_TFLOPS, "traffic": sweep_traffic(args.config),
                     "kernel": "binary32 exhaustive sweep (cq_quantize_groups, CQ_EXHAUSTIVE)",
                     "launch_ms": avg_ms, "groups_per_launch": avg_groups,
                     "flops_per_launch": avg_flops, "flops_per_active_term": 2 * E + 4,
                     "patterns_per_group": patterns,
                     "chunks_per_group": float(np.mean([(t["patterns"] - 1) // 128 + 1 for t in mats])),
                     "unskippable_chunks_per_group": float(np.mean(nec_chunks)),
                     "active_terms_per_group_unskippable": avg_flops / avg_groups / (2 * E + 4),
                     "active_terms_per_group_all_chunks": float(np.mean(all_terms))},
        "sweep_groups_per_s": avg_groups / (avg_ms / 1e3),
        "sweep_full_grid_equivalent_tflops": full_grid_flops(avg_groups, E) / (avg_ms / 1e3) / 1e12,
        "flag_counts": {"near_tie": int(np.count_nonzero(flags & 2)), "exact_tie": int(np.count_nonzero(flags & 4)),
                        "fp64_sweep": int(np.count_nonzero(flags & 16))},
        "wall_s": wall,
    }
    if args.all_configs:
        line["per_config"] = measure_all_configs()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
