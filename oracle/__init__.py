"""CPU oracle for exact minimax FP16 group-scale selection -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``post_weight_quantization_group_amd``) and neither imports the other.

The brute force itself is plain C (``cq_oracle.c``, built with gcc); this
module marshals numpy arrays into it and adds the two steps that are plain
array reshuffles or means:

* GPTQ-v1 packing (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card,
  "Quantization configuration": GPTQ v1, 4 bits, group 128, symmetric; 2- and
  8-bit codes and other group lengths packed the same way, field by field);
* the module-macro worst-environment weighted-MSE proxy (same card,
  "Held-out reconstruction proxy"; CliffQuant README, "Held-out
  reconstruction proxy");
* the held-out comparison of two policies on that proxy: per-group wins, ties
  and losses, the macro effect and the interval of a bootstrap that resamples
  groups within modules, paired across the two policies (CliffQuant README, "Held-out reconstruction proxy").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GROUP = 128                       # the group length the pages use
QMIN, QMAX = -8, 7                # the code range the pages use (signed 4-bit)
MAX_GROUP = 1024                  # longest group the oracle takes
FIRST_BITS, LAST_BITS = 0x0001, 0x7BFF
N_SCALES = LAST_BITS - FIRST_BITS + 1  # 31,743

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cq_oracle.c")
# CQ_ORACLE_LIB names another build of cq_oracle.c to load instead; the mutation test uses it
# to run the pins against copies with a planted mistake.
_LIB = os.environ.get("CQ_ORACLE_LIB") or os.path.join(_HERE, "libcq_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE arithmetic: no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64, I32, U32 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        lib.oracle_fp16_value.restype = ctypes.c_double
        lib.oracle_fp16_value.argtypes = [U32]
        lib.oracle_solve.restype = I32
        lib.oracle_solve.argtypes = [P, P, I64, I32, I64, I32, I32, I32, P, P, P, P, P, P, P, P, I32]
        lib.oracle_codes.restype = None
        lib.oracle_codes.argtypes = [P, I64, U32, I32, I32, P]
        lib.oracle_env_errors.restype = I32
        lib.oracle_env_errors.argtypes = [P, P, I64, I32, I64, I32, I32, I32, P, P, I32]
        lib.oracle_curve.restype = I32
        lib.oracle_curve.argtypes = [P, P, I32, I32, I32, I32, P, P]
        lib.oracle_fp16_round.restype = U32
        lib.oracle_fp16_round.argtypes = [ctypes.c_float]
        lib.oracle_absmax.restype = None
        lib.oracle_absmax.argtypes = [P, I64, I32, I32, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _spec(qmin: int, qmax: int):
    qmin, qmax = int(qmin), int(qmax)
    if not (-128 <= qmin <= 0 <= qmax <= 127 and qmin < qmax):
        raise ValueError("code range must satisfy -128 <= qmin <= 0 <= qmax <= 127, qmin < qmax")
    return qmin, qmax


def _groups(w, d, d_period):
    w = np.ascontiguousarray(w, dtype=np.float32)
    d = np.ascontiguousarray(d, dtype=np.float32)
    if w.ndim != 2 or not 1 <= w.shape[1] <= MAX_GROUP:
        raise ValueError("w must be [n_groups, G] with 1 <= G <= 1024")
    G = w.shape[1]
    if d.ndim != 3 or d.shape[2] != G:
        raise ValueError("d must be [n_d, E, G]")
    if d_period is None:
        d_period = d.shape[0]
    if not (1 <= d_period <= d.shape[0]):
        raise ValueError("bad d_period")
    E = d.shape[1]
    if not (1 <= E <= 32):
        raise ValueError("E must be in 1..32")
    return w, d, int(d_period), E, G


def fp16_value(bits: int) -> float:
    """Exact value of a positive binary16 bit pattern."""
    return _load().oracle_fp16_value(int(bits))


def fp16_round(x: float) -> int:
    """Binary16 bit pattern nearest to a non-negative float32 (ties to even; 0x7C00 = overflow)."""
    return int(_load().oracle_fp16_round(float(np.float32(x))))


def codes_at(w, bits: int, qmin: int = QMIN, qmax: int = QMAX) -> np.ndarray:
    """q_i = clip(round-half-even(fl32(w_i / s)), qmin, qmax) for every weight, at one scale."""
    qmin, qmax = _spec(qmin, qmax)
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    out = np.empty(w.size, dtype=np.int8)
    _load().oracle_codes(_ptr(w), w.size, int(bits), qmin, qmax, _ptr(out))
    return out


class Solution:
    """Brute-force result per group (see ``solve``)."""

    def __init__(self, n, G=GROUP):
        self.mm_bits = np.zeros(n, np.uint16)
        self.mm_F1 = np.zeros(n, np.float64)
        self.mm_F2 = np.zeros(n, np.float64)
        self.pl_bits = np.zeros(n, np.uint16)
        self.pl_P1 = np.zeros(n, np.float64)
        self.pl_P2 = np.zeros(n, np.float64)
        self.codes = np.zeros((n, G), np.int8)
        self.ok = np.zeros(n, np.uint8)

    @staticmethod
    def _gap(f1, f2):
        f1, f2 = np.asarray(f1, np.float64), np.asarray(f2, np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            g = (f2 - f1) / f1
        return np.where(f1 == 0.0, np.where(f2 == 0.0, 0.0, np.inf), g)

    @property
    def mm_gap(self):
        """(F2 - F1) / F1; 0 for an exact zero tie, +inf when only the winner is zero."""
        return self._gap(self.mm_F1, self.mm_F2)

    @property
    def pl_gap(self):
        return self._gap(self.pl_P1, self.pl_P2)


def solve(w, d, d_period=None, n_threads: int = 0, qmin: int = QMIN, qmax: int = QMAX) -> Solution:
    """Exhaustive minimax and pooled-WMSE scale selection over all 31,743 FP16 scales.

    CliffQuant README, "What CliffQuant changes": the objective, the code rule,
    the admissible set and the lower-bit-pattern tie rule; the pooled policy
    averages the environments first (README opening question; proxy table).
    The quantizer is the README's "Use the solver" specification: codes in
    [qmin, qmax], groups of G = w.shape[1] weights (the pages run [-8, 7], G = 128).
    """
    w, d, d_period, E, G = _groups(w, d, d_period)
    qmin, qmax = _spec(qmin, qmax)
    n = w.shape[0]
    r = Solution(n, G)
    rc = _load().oracle_solve(_ptr(w), _ptr(d), d_period, E, n, G, qmin, qmax,
                              _ptr(r.mm_bits), _ptr(r.mm_F1), _ptr(r.mm_F2),
                              _ptr(r.pl_bits), _ptr(r.pl_P1), _ptr(r.pl_P2),
                              _ptr(r.codes), _ptr(r.ok), int(n_threads))
    if rc != 0:
        raise ValueError("the oracle rejected the quantizer specification")
    return r


def env_errors(w, d, bits, d_period=None, n_threads: int = 0, qmin: int = QMIN, qmax: int = QMAX) -> np.ndarray:
    """[n_groups, E] per-environment weighted squared error at the given scales."""
    w, d, d_period, E, G = _groups(w, d, d_period)
    qmin, qmax = _spec(qmin, qmax)
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if bits.shape != (w.shape[0],):
        raise ValueError("one scale per group")
    out = np.empty((w.shape[0], E), np.float64)
    rc = _load().oracle_env_errors(_ptr(w), _ptr(d), d_period, E, w.shape[0], G, qmin, qmax, _ptr(bits),
                                   _ptr(out), int(n_threads))
    if rc != 0:
        raise ValueError("the oracle rejected the quantizer specification")
    return out


def objective(w, d, bits, d_period=None, n_threads: int = 0, qmin: int = QMIN, qmax: int = QMAX) -> np.ndarray:
    """Worst-environment objective max_e F_e at the given scales."""
    return env_errors(w, d, bits, d_period, n_threads, qmin, qmax).max(axis=1)


def curve(w_group, d_group, qmin: int = QMIN, qmax: int = QMAX):
    """(F[31743], P[31743]) over b = 1..0x7BFF for one group (w [G], d [E, G])."""
    qmin, qmax = _spec(qmin, qmax)
    w = np.ascontiguousarray(w_group, dtype=np.float32).ravel()
    G = w.size
    d = np.ascontiguousarray(d_group, dtype=np.float32).reshape(-1, G)
    E = d.shape[0]
    F = np.empty(N_SCALES, np.float64)
    P = np.empty(N_SCALES, np.float64)
    if _load().oracle_curve(_ptr(w), _ptr(d), E, G, qmin, qmax, _ptr(F), _ptr(P)) != 0:
        raise ValueError("the oracle rejected the quantizer specification")
    return F, P


def absmax_bits(w, qmax: int = QMAX) -> np.ndarray:
    """AbsMax policy: fp16(fl32(max|w| / qmax)), 0 -> 0x0001, overflow -> 0x7BFF (qmax = 7 on the pages)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or not 1 <= int(qmax) <= 127:
        raise ValueError("w must be [n_groups, G] and 1 <= qmax <= 127")
    out = np.empty(w.shape[0], np.uint16)
    _load().oracle_absmax(_ptr(w), w.shape[0], w.shape[1], int(qmax), _ptr(out))
    return out


def codes_for(w, bits, qmin: int = QMIN, qmax: int = QMAX) -> np.ndarray:
    """[n_groups, G] codes of each group at its own scale."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape[0] == 0:
        return np.zeros((0, w.shape[1] if w.ndim == 2 else GROUP), np.int8)
    return np.stack([codes_at(w[g], int(bits[g]), qmin, qmax) for g in range(w.shape[0])])


# ---------------------------------------------------------------- GPTQ-v1 packing
def pack_gptq_v1(codes, grp_scale_bits, out: int, inp: int, bits: int = 4, group: int = GROUP):
    """GPTQ-v1 symmetric packing of one matrix, `bits` in {2, 4, 8} (the pages use 4).

    codes          -- [out, in] int8 in [-2^(bits-1), 2^(bits-1) - 1] (group g = row*(in/group) + in_chunk);
    grp_scale_bits -- [out, in/group] binary16 bit patterns.
    Returns (qweight [in*bits/32, out] int32, scales [in/group, out] uint16): field j
    (bits j*bits .. j*bits + bits - 1, low field first) of qweight[r, o] holds
    codes[o, (32/bits)*r + j] + 2^(bits-1).
    """
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    per = 32 // bits
    c = np.asarray(codes, dtype=np.int64).reshape(out, inp)
    if inp % group or inp % per:
        raise ValueError("in must be a multiple of the group length and of 32/bits")
    u = (c + (1 << (bits - 1))).reshape(out, inp // per, per)
    word = np.zeros((out, inp // per), dtype=np.uint64)
    for j in range(per):
        word |= (u[:, :, j].astype(np.uint64) << np.uint64(bits * j))
    qweight = word.T.astype(np.uint32).view(np.int32)
    scales = np.asarray(grp_scale_bits, dtype=np.uint16).reshape(out, inp // group).T
    return np.ascontiguousarray(qweight), np.ascontiguousarray(scales)


def unpack_gptq_v1(qweight, scales, bits: int = 4):
    """Inverse of ``pack_gptq_v1``: (codes [out, in] int8, grp_scale_bits [out, in/group])."""
    per = 32 // bits
    q = np.asarray(qweight).view(np.uint32).astype(np.int64)
    rows, out = q.shape
    mask = (1 << bits) - 1
    fld = np.stack([(q >> (bits * j)) & mask for j in range(per)], axis=1)  # [rows, per, out]
    codes = (fld.reshape(rows * per, out).T - (1 << (bits - 1))).astype(np.int8)
    return codes, np.ascontiguousarray(np.asarray(scales, np.uint16).T)


# ---------------------------------------------------------------- proxy
def proxy(w, d_eval, bits, module_of_group, n_modules: int, d_period=None, n_threads: int = 0,
          qmin: int = QMIN, qmax: int = QMAX):
    """Module-macro worst-environment weighted MSE.

    Per group p_g = max_e (1/G) sum_i d_eval[e][i] (w_i - s_g q_i)^2; then the
    mean of p_g over each module's groups (in group order); then the mean over
    modules (in module order).  A module with no groups has no mean: NaN, and
    the macro over modules is then NaN too (the reading the held-out comparison
    takes for an empty module as well).  Returns (per_group, module_mean, macro).
    """
    F = env_errors(w, d_eval, bits, d_period, n_threads, qmin, qmax)
    G = np.asarray(w).shape[1]
    per_group = (F / float(G)).max(axis=1)
    mod = np.asarray(module_of_group, dtype=np.int64)
    module_mean = np.zeros(n_modules, np.float64)
    for m in range(n_modules):
        vals = per_group[mod == m]
        acc = 0.0
        for v in vals:
            acc = acc + float(v)
        module_mean[m] = acc / len(vals) if len(vals) else float("nan")
    acc = 0.0
    for v in module_mean:
        acc = acc + float(v)
    return per_group, module_mean, acc / n_modules


# ---------------------------------------------------------------- held-out comparison
def _seq_sum_rows(x: np.ndarray) -> np.ndarray:
    """Left-to-right binary64 sum of each row (numpy's cumsum adds in order; sum() would not)."""
    if x.shape[-1] == 0:
        return np.zeros(x.shape[:-1])
    return np.cumsum(x, axis=-1)[..., -1]


def heldout_compare(pa, pb, module_offsets, boot_idx, alpha: float = 0.05):
    """Policy A against policy B on per-group proxy values (CliffQuant README, "Held-out
    reconstruction proxy": CliffQuant's wins, ties and losses against Pooled-WMSE by group, and the
    bootstrap of the effect, resampling within modules and paired across policies, with its 95%
    interval).

    Readings where the pages are silent:
    * a win of A is p_A < p_B, a tie p_A == p_B, a loss p_A > p_B (exact comparisons);
    * the effect is the mean over modules of each module's mean of (p_B - p_A), summed in order
      (the paired form of macro_B - macro_A);
    * replicate r resamples each module's groups with replacement, the same draw for both
      policies: position j of module m takes group boot_idx[r, j] (drawn in m's range), and the
      replicate effect is the effect formula on those groups;
    * the interval is the linear-interpolation percentile at 100 alpha/2 and 100 (1 - alpha/2) of
      the replicates sorted ascending: position q (B - 1), value v[lo] + (v[lo+1] - v[lo]) t.
    A module whose range is empty, or a replicate with a draw outside its module, gives NaN.

    Returns (counts [wins, ties, losses], effect, replicates sorted ascending, (lo, hi))."""
    pa = np.asarray(pa, dtype=np.float64)
    pb = np.asarray(pb, dtype=np.float64)
    off = np.asarray(module_offsets, dtype=np.int64)
    idx = np.asarray(boot_idx, dtype=np.int64)
    counts = np.array([np.count_nonzero(pa < pb), np.count_nonzero(pa == pb), np.count_nonzero(pa > pb)],
                      dtype=np.int64)
    diff = pb - pa
    M = off.size - 1
    B = idx.shape[0]
    # rows: the point estimate (identity draw) then the replicates
    means = np.empty((B + 1, M))
    for m in range(M):
        lo, hi = int(off[m]), int(off[m + 1])
        if hi <= lo:
            means[:, m] = np.nan
            continue
        pos = np.arange(lo, hi)
        draw = np.vstack([pos[None, :], idx[:, lo:hi]])
        ok = np.all((draw >= lo) & (draw < hi), axis=1)
        vals = diff[np.clip(draw, lo, hi - 1)]
        means[:, m] = np.where(ok, _seq_sum_rows(vals) / float(hi - lo), np.nan)
    effects = _seq_sum_rows(means) / float(M)
    effect = float(effects[0])
    reps = np.sort(effects[1:])  # NaN sorts last

    def pct(q):
        if B == 0 or np.isnan(reps[-1]):
            return float("nan")
        pos = q * (B - 1)
        lo = int(np.floor(pos))
        t = pos - lo
        if lo + 1 >= B:
            return float(reps[B - 1])
        return float(reps[lo] + (reps[lo + 1] - reps[lo]) * t)

    return counts, effect, reps, (pct(alpha / 2.0), pct(1.0 - alpha / 2.0))


# ---------------------------------------------------------------- environment diagonals
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (the top half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def environment_diagonals(x_bits) -> np.ndarray:
    """Separately normalized environment diagonals from calibration activations (CliffQuant
    README, "What CliffQuant changes": each channel's sensitivity weighted by its activations, per
    calibration environment, each environment normalized on its own).

    Reading where the pages are silent: for environment e with tokens t = 1..T,
    d_{e,i} = (1/T) sum_t x_{t,i}^2, then divided by its mean over the channels i, in binary64,
    and rounded once to binary32.  x_bits: bfloat16 bit patterns [E, T, in].  Returns d
    [in/128, E, 128] float32, the layout the solver takes with d_period = in/128.  An
    environment whose activations are all zero gives NaN."""
    x = bf16_to_f64(x_bits)
    E, T, n = x.shape
    m = (x * x).sum(axis=1) / float(T)                 # [E, in]
    with np.errstate(invalid="ignore", divide="ignore"):
        d = m / m.mean(axis=1, keepdims=True)
    return np.ascontiguousarray(d.astype(np.float32).reshape(E, n // GROUP, GROUP).transpose(1, 0, 2))


# ---------------------------------------------------------------- W4A16 consumer check
def w4a16_matmul(x_bits, qweight, scales):
    """y = x W^T with W dequantized from the GPTQ-v1 tensors (model card, "Quantization
    configuration": GPTQ v1, 4 bits, group 128, symmetric; the W4A16 checkpoint keeps 16-bit
    activations): W[o][k] = s[k/128][o] (u - 8) with u the nibble of qweight.  x_bits: bfloat16 bit
    patterns [M, in]; qweight int32 [in/8, out]; scales binary16 bit patterns [in/128, out].
    Returns y [M, out] in binary64 (the exact dequantized product up to binary64 rounding) and the
    bound sum_k |x_k| |W[o][k]| per output, [M, out], for error bounds."""
    codes, sbits = unpack_gptq_v1(qweight, scales)           # [out, in], [out, in/128]
    svals = np.asarray(sbits, np.uint16).view(np.float16).astype(np.float64)
    Wd = codes.astype(np.float64) * np.repeat(svals, GROUP, axis=1)
    x = bf16_to_f64(x_bits)
    return x @ Wd.T, np.abs(x) @ np.abs(Wd).T
