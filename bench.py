"""Benchmark: exact minimax FP16 group-scale selection (W4, groups of 128) on one MI355X.

One step = the whole hot path over one batch: for every matrix of the workload, the
exhaustive minimax sweep (the pooled-WMSE policy decided in the same sweep, codes emitted),
the candidate-set solver, the AbsMax baseline, GPTQ-v1 packing of the minimax codes and
scales, and the worst-environment weighted-MSE proxy for the three policies.  Inputs are
resident in HBM before timing starts.

Prints one JSON line.  `value` = groups per second of whole steps; `roofline` describes the
dominant kernel (the binary32 sweep) measured with HIP events on its own stream;
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


def flops_per_group(E: int) -> int:
    """Algorithmic flops of one group's sweep: per scale and weight one quotient multiply,
    a residual fma (2), a square (1) and E weighted fmas (2E)."""
    return SCALES * 128 * (2 * E + 4)


def cpu_baseline(k: int, budget_s: float) -> dict:
    import oracle
    import workloads as W
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(cores, 256))
    gids = W.sample_groups(k, 86016, salt=99)
    w, d, _ = W.gather_matrix_groups(k, gids[: max(threads, 1) * 64])
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-candidate", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a plain copy kernel of known "
                         "size, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): every group is independent, "
              "so several GPUs would each run this same benchmark on their own share.", file=sys.stderr)
        sys.exit(2)

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
            "w": torch.from_numpy(w).to(dev), "d": torch.from_numpy(d).to(dev),
            "scales": torch.empty(n, dtype=torch.int16, device=dev),
            "codes": torch.empty((n, 128), dtype=torch.int8, device=dev),
            "obj": torch.empty(n, dtype=torch.float64, device=dev),
            "flags": torch.empty(n, dtype=torch.uint8, device=dev),
            "pscales": torch.empty(n, dtype=torch.int16, device=dev),
            "pobj": torch.empty(n, dtype=torch.float64, device=dev),
            "cscales": torch.empty(n, dtype=torch.int16, device=dev),
            "ccodes": torch.empty((n, 128), dtype=torch.int8, device=dev),
            "cobj": torch.empty(n, dtype=torch.float64, device=dev),
            "cflags": torch.empty(n, dtype=torch.uint8, device=dev),
            "ascales": torch.empty(n, dtype=torch.int16, device=dev),
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
                sweep_ev.append((a, b, t["n"]))
            if use_candidate:
                cq.cq_quantize_groups(t["w"], t["d"], t["p"], E, t["n"], cq.CANDIDATE, t["cscales"],
                                      t["ccodes"], t["cobj"], t["cflags"], None, None, t["cws"])
            cq.cq_baseline_scales(t["w"], t["d"], t["p"], E, t["n"], cq.ABSMAX, t["ascales"], t["acodes"],
                                  t["aobj"])
            cq.cq_pack_gptq_v1(t["codes"], t["scales"], t["out"], t["inp"], t["qweight"], t["qscales"])
            for j, sc in enumerate((t["scales"], t["pscales"], t["ascales"])):
                cq.cq_proxy_worst_env_wmse(t["w"], t["d"], t["p"], E, t["n"], sc, t["off"], 1, t["mm"][j],
                                           t["macro"][j], t["pg"][j])

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

    # dominant kernel: the exhaustive sweep call, per launch (one launch per matrix)
    durs = [a.elapsed_time(b) for a, b, _ in sweep_ev]
    groups = [n for _, _, n in sweep_ev]
    avg_ms = float(np.mean(durs))
    avg_groups = float(np.mean(groups))
    achieved = flops_per_group(E) * avg_groups / (avg_ms / 1e3) / 1e12
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
                     "frac": achieved / PEAK_FP32_TFLOPS, "traffic": None,
                     "kernel": "binary32 exhaustive sweep (cq_quantize_groups, CQ_EXHAUSTIVE)",
                     "launch_ms": avg_ms, "groups_per_launch": avg_groups,
                     "flops_per_group": flops_per_group(E)},
        "sweep_groups_per_s": avg_groups / (avg_ms / 1e3),
        "flag_counts": {"near_tie": int(np.count_nonzero(flags & 2)), "exact_tie": int(np.count_nonzero(flags & 4)),
                        "fp64_sweep": int(np.count_nonzero(flags & 16))},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
