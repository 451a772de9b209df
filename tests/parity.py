"""Comparison helpers for GPU-versus-oracle parity (the criteria the tests apply)."""
import os
import sys

import numpy as np
import torch

import oracle

GAP = 1e-9      # scale bits must match when the oracle's runner-up gap exceeds this (relative)
OBJ_TOL = 1e-9  # otherwise the GPU objective must be within this of the oracle minimum (relative)
PROXY_TOL = 1e-6


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return (t.detach().cpu().numpy().astype(np.int64) & 0xFFFF).astype(np.uint16)


def dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_policy(name, w, d, d_period, gpu_bits, gpu_obj, best_bits, F1, gap, objective_fn):
    """Criterion (i) plus: the GPU's binary64 objective equals the oracle's objective at the GPU's
    own scale, bit for bit (both sum in the same fixed order)."""
    gpu_bits = np.asarray(gpu_bits)
    sure = gap > GAP
    bad = np.nonzero(sure & (gpu_bits != best_bits))[0]
    assert bad.size == 0, f"{name}: bits differ on {bad.size} groups with gap > 1e-9, e.g. {bad[:5]}, " \
                          f"gpu {[hex(x) for x in gpu_bits[bad[:5]]]} oracle {[hex(x) for x in best_bits[bad[:5]]]}"
    close = ~sure
    if close.any():
        rel = np.where(F1[close] == 0, np.abs(gpu_obj[close]),
                       np.abs(gpu_obj[close] - F1[close]) / np.where(F1[close] == 0, 1, F1[close]))
        assert np.all(rel <= OBJ_TOL), f"{name}: near-tie objective off by {rel.max()}"
    at_gpu = objective_fn(gpu_bits)
    mism = np.nonzero(at_gpu != gpu_obj)[0]
    assert mism.size == 0, f"{name}: objective at the chosen scale differs on {mism[:5]}"
    return int(np.count_nonzero(gpu_bits == best_bits)), int(close.sum())


def check_minimax(w, d, d_period, r, sol, codes=True):
    """GPU result dict `r` against an oracle Solution `sol` for the same groups."""
    bits = bits_np(r["scales"])
    obj = r["objective"].cpu().numpy()
    same, near = check_policy("minimax", w, d, d_period, bits, obj, sol.mm_bits, sol.mm_F1, sol.mm_gap,
                              lambda b: oracle.objective(w, d, b, d_period, threads()))
    if codes and r.get("codes") is not None:
        want = oracle.codes_for(w, bits)
        got = r["codes"].cpu().numpy()
        diff = np.nonzero(np.any(got != want, axis=1))[0]
        assert diff.size == 0, f"codes differ on groups {diff[:5]}"
    return same, near


def check_pooled(w, d, d_period, pbits_t, pobj_t, sol):
    bits = bits_np(pbits_t)
    obj = pobj_t.cpu().numpy()

    def pooled_at(b):
        Fe = oracle.env_errors(w, d, b, d_period, threads())
        P = Fe[:, 0].copy()
        for e in range(1, Fe.shape[1]):
            P = P + Fe[:, e]
        return P / Fe.shape[1]
    return check_policy("pooled", w, d, d_period, bits, obj, sol.pl_bits, sol.pl_P1, sol.pl_gap, pooled_at)
