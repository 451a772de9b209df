"""Comparison helpers for GPU-versus-oracle parity (the criteria the tests apply)."""
import os
import sys

import numpy as np
import torch

import oracle
import workloads as W

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


def check_minimax(w, d, d_period, r, sol, codes=True, qmin=-8, qmax=7):
    """GPU result dict `r` against an oracle Solution `sol` for the same groups."""
    bits = bits_np(r["scales"])
    obj = r["objective"].cpu().numpy()
    same, near = check_policy("minimax", w, d, d_period, bits, obj, sol.mm_bits, sol.mm_F1, sol.mm_gap,
                              lambda b: oracle.objective(w, d, b, d_period, threads(), qmin, qmax))
    if codes and r.get("codes") is not None:
        want = oracle.codes_for(w, bits, qmin, qmax)
        got = r["codes"].cpu().numpy()
        diff = np.nonzero(np.any(got != want, axis=1))[0]
        assert diff.size == 0, f"codes differ on groups {diff[:5]}"
    return same, near


def pooled_at(w, d, d_period, b, qmin=-8, qmax=7):
    """The oracle's pooled objective (environment sums added in order, then / E) at given bits."""
    Fe = oracle.env_errors(w, d, b, d_period, threads(), qmin, qmax)
    P = Fe[:, 0].copy()
    for e in range(1, Fe.shape[1]):
        P = P + Fe[:, e]
    return P / Fe.shape[1]


def check_pooled(w, d, d_period, pbits_t, pobj_t, sol, qmin=-8, qmax=7):
    bits = bits_np(pbits_t)
    obj = pobj_t.cpu().numpy()
    return check_policy("pooled", w, d, d_period, bits, obj, sol.pl_bits, sol.pl_P1, sol.pl_gap,
                        lambda b: pooled_at(w, d, d_period, b, qmin, qmax))


def check_same_result(a, b, label, keys=("scales", "codes", "objective", "pooled_scales", "pooled_objective")):
    """Two GPU result dicts of the same groups (two methods, or two launch shapes) agree bit for bit
    on every output they both carry (floating outputs compared as bit patterns, so NaN equals NaN)."""
    for k in keys:
        if a.get(k) is None or b.get(k) is None:
            continue
        x, y = a[k].cpu().numpy(), b[k].cpu().numpy()
        x, y = x.reshape(x.shape[0], -1).view(np.uint8), y.reshape(y.shape[0], -1).view(np.uint8)
        bad = np.nonzero(np.any((x != y).reshape(x.shape[0], -1), axis=1))[0]
        assert bad.size == 0, f"{label}: {k} differs on {bad.size} groups, e.g. {bad[:5]}"


def spec_groups(qmin, qmax, G, E, n, seed):
    """Seeded groups of G weights (bf16-valued normal weights with 2% outliers x8, a few tiny and
    all-zero groups, constructed exact ties) and per-group lognormal diagonals."""
    rng = np.random.default_rng(seed)
    w = W.round_bf16((rng.normal(0, 0.02, (n, G)) * np.where(rng.random((n, G)) < 0.02, 8.0, 1.0))
                     .astype(np.float32))
    w[1] = 0.0
    w[2] = (rng.uniform(-1, 1, G) * 1e-5).astype(np.float32)
    # symmetric +-c n pairs: zero error at s = c and c/2 (and, for wide ranges, smaller powers)
    c = 2.0 ** -7
    m = rng.integers(1, min(qmax, 3) + 1, G // 2) if qmax >= 1 else np.ones(G // 2)
    pair = np.zeros(G, np.float32)
    pair[: 2 * (G // 2)] = np.concatenate([m * c, -m * c]).astype(np.float32)
    w[3] = pair
    d = rng.lognormal(0, 1, (n, E, G)).astype(np.float32)
    if E > 1:
        d[3, 1] = d[3, 0]
    return w, d
