"""Seeded synthetic inputs for W4/G128 group-scale selection.

This module is shared by the CPU oracle's tests and by the GPU library's
tests and benchmark.  It draws random numbers and lays them out; it holds
none of the scale-selection arithmetic.

What the inputs stand in for (CliffQuant repository README, "Experiment 001";
Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Calibration and
evaluation data"): real weight matrices quantized in groups of 128 consecutive
input channels, and per-environment activation-weighted diagonals, each
environment normalised on its own.  Neither the checkpoint nor the corpora are
available, so weights and diagonals are drawn from fixed distributions.

Layout handed to both sides:

* ``w``  -- ``[n_groups, 128]`` float32; group ``g`` of a matrix ``[out, in]``
  is row ``g // (in/128)``, input channels ``128*(g % (in/128))`` onward.
* ``d``  -- ``[n_d, E, 128]`` float32; group ``g`` uses slice ``g % d_period``.
  A matrix has ``d_period = in/128`` (groups inherit the diagonal slice of
  their input channels); per-group diagonals have ``d_period = n_groups``.

Every stream is ``numpy.random.Generator(PCG64(SeedSequence(1000 + k,
spawn_key=(unit, stream))))`` for config ``k``, so any matrix (or any chunk
of per-group config 3) can be produced alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128

# stream ids inside one unit (matrix or chunk)
_S_WEIGHT, _S_OUTLIER, _S_DBASE, _S_DPERT, _S_PERM, _S_STD, _S_DEVAL, _S_BOOT, _S_ACT = range(9)


def _rng(k: int, unit: int, stream: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(1000 + k, spawn_key=(unit, stream))))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@dataclass(frozen=True)
class Matrix:
    name: str
    out: int
    inp: int

    @property
    def n_groups(self) -> int:
        return self.out * self.inp // GROUP

    @property
    def d_period(self) -> int:
        return self.inp // GROUP


@dataclass(frozen=True)
class ConfigSpec:
    k: int
    E: int
    description: str
    matrices: tuple = field(default_factory=tuple)  # empty => per-group diagonals
    n_groups_per_group_mode: int = 0
    chunk: int = 4096  # per-group mode: groups per independently seeded chunk

    @property
    def per_group(self) -> bool:
        return not self.matrices

    @property
    def n_groups(self) -> int:
        if self.per_group:
            return self.n_groups_per_group_mode
        return sum(m.n_groups for m in self.matrices)

    def matrix_offsets(self) -> np.ndarray:
        return np.cumsum([0] + [m.n_groups for m in self.matrices]).astype(np.int64)


def config(k: int) -> ConfigSpec:
    if k == 0:
        return ConfigSpec(0, 4, "one matrix 64x256, 128 groups, E=4",
                          (Matrix("w", 64, 256),))
    if k == 1:
        return ConfigSpec(1, 4, "MLP block gate/up 3584x1024, down 1024x3584; 86,016 groups, E=4",
                          (Matrix("gate", 3584, 1024), Matrix("up", 3584, 1024),
                           Matrix("down", 1024, 3584)))
    if k == 2:
        mats = tuple(Matrix(f"m{j:03d}", 809, 4096) for j in range(149)) + (Matrix("m149", 803, 4096),)
        return ConfigSpec(2, 4, "150 matrices, 3,883,008 groups, E=4", mats)
    if k == 3:
        return ConfigSpec(3, 8, "edge and tie stress: 262,144 groups, per-group diagonals, E=8",
                          (), n_groups_per_group_mode=262144)
    if k == 4:
        return ConfigSpec(4, 16, "8 matrices 4096x4096, 1,048,576 groups, E=16",
                          tuple(Matrix(f"m{j}", 4096, 4096) for j in range(8)))
    raise ValueError(f"unknown config {k}")


# ---------------------------------------------------------------- diagonals
def _normalise_rows(d: np.ndarray) -> np.ndarray:
    """Scale each environment row (last axis) to mean 1, in float64, then cast to float32."""
    d = np.asarray(d, dtype=np.float64)
    return (d / d.mean(axis=-1, keepdims=True)).astype(np.float32)


def _diag_lognormal_pert(rng_base, rng_pert, E: int, n: int) -> np.ndarray:
    """base_i ~ LogNormal(0,1) per channel times pert_{e,i} ~ LogNormal(0,0.5); mean 1 per env."""
    base = rng_base.lognormal(0.0, 1.0, size=n)
    pert = rng_pert.lognormal(0.0, 0.5, size=(E, n))
    return _normalise_rows(base[None, :] * pert)


def _diag_permuted(rng_base, rng_perm, E: int, n: int) -> np.ndarray:
    """base_i ~ LogNormal(0,1.5); per env a random 10% of channels permuted among themselves."""
    base = rng_base.lognormal(0.0, 1.5, size=n)
    m = int(round(0.1 * n))
    out = np.empty((E, n), dtype=np.float64)
    for e in range(E):
        idx = rng_perm.choice(n, size=m, replace=False)
        row = base.copy()
        row[idx] = base[idx[rng_perm.permutation(m)]]
        out[e] = row
    return _normalise_rows(out)


# ---------------------------------------------------------------- matrices
def make_matrix(k: int, m: int):
    """Return (W [out, in] float32, dmat [E, in] float32) for matrix ``m`` of config ``k``."""
    spec = config(k)
    if spec.per_group:
        raise ValueError("config 3 has per-group diagonals; use make_groups")
    mat = spec.matrices[m]
    rw, ro = _rng(k, m, _S_WEIGHT), _rng(k, m, _S_OUTLIER)
    rb, rp = _rng(k, m, _S_DBASE), _rng(k, m, _S_DPERT)
    shape = (mat.out, mat.inp)
    if k in (0, 1):
        W = rw.normal(0.0, 0.02, size=shape)
        W = np.where(ro.random(shape) < 0.01, W * 8.0, W)
        dmat = _diag_lognormal_pert(rb, rp, spec.E, mat.inp)
    elif k == 2:
        std = _rng(k, m, _S_STD).uniform(0.01, 0.05)
        W = rw.normal(0.0, std, size=shape)
        W = np.where(ro.random(shape) < 0.005, W * 10.0, W)
        dmat = _diag_lognormal_pert(rb, rp, spec.E, mat.inp)
    elif k == 4:
        W = rw.normal(0.0, 0.03, size=shape)
        dmat = _diag_permuted(rb, _rng(k, m, _S_PERM), spec.E, mat.inp)
    else:
        raise ValueError(k)
    return round_bf16(W.astype(np.float32)), dmat


def matrix_groups(W: np.ndarray, dmat: np.ndarray):
    """Lay a matrix out as (w [n_groups,128], d [in/128, E, 128], d_period)."""
    out, inp = W.shape
    E = dmat.shape[0]
    w = np.ascontiguousarray(W.reshape(out * inp // GROUP, GROUP), dtype=np.float32)
    d = np.ascontiguousarray(dmat.reshape(E, inp // GROUP, GROUP).transpose(1, 0, 2), dtype=np.float32)
    return w, d, inp // GROUP


# ---------------------------------------------------------------- config 3
CAT_STUDENT_T, CAT_TINY, CAT_ZERO, CAT_PAIR_TIE, CAT_ONE_CHANNEL = range(5)
_CAT_COUNTS = (104858, 52429, 26214, 26214, 52429)


def config3_categories() -> np.ndarray:
    """Category of each of the 262,144 config-3 groups (seeded permutation)."""
    cats = np.repeat(np.arange(5, dtype=np.int8), _CAT_COUNTS)
    return cats[_rng(3, 1 << 20, _S_PERM).permutation(cats.size)]


def pair_tie_unit(c_exp: int) -> float:
    """The c = 2**-c_exp of a symmetric-pair tie group."""
    return float(2.0 ** -c_exp)


def _config3_chunk(chunk: int, cats: np.ndarray):
    spec = config(3)
    E = spec.E
    lo = chunk * spec.chunk
    n = min(spec.chunk, spec.n_groups - lo)
    cat = cats[lo:lo + n]
    rw, ro = _rng(3, chunk, _S_WEIGHT), _rng(3, chunk, _S_OUTLIER)
    rb, rp, rq = _rng(3, chunk, _S_DBASE), _rng(3, chunk, _S_DPERT), _rng(3, chunk, _S_PERM)
    # every group gets config-0 style diagonals over its own 128 channels
    base = rb.lognormal(0.0, 1.0, size=(n, 1, GROUP))
    pert = rp.lognormal(0.0, 0.5, size=(n, E, GROUP))
    d = base * pert
    # weights of every category are drawn for every group, then selected
    t = rw.standard_t(3.0, size=(n, GROUP)) * 0.02
    tiny = rw.uniform(-1.0, 1.0, size=(n, GROUP)) * 1e-5
    gauss = rw.normal(0.0, 0.02, size=(n, GROUP))
    c_exp = rq.integers(5, 11, size=n)            # c = 2^-k, k in 5..10
    mult = rq.integers(1, 4, size=(n, GROUP // 2))  # n_j in {1,2,3}
    mult[:, :3] = (1, 2, 3)                         # every multiple present
    pair_order = np.argsort(rq.random((n, GROUP)), axis=1)
    one_env = rq.integers(0, E, size=n)
    one_chan = rq.integers(0, GROUP, size=n)

    w = np.zeros((n, GROUP), dtype=np.float32)
    sel = cat == CAT_STUDENT_T
    w[sel] = t[sel].astype(np.float32)
    sel = cat == CAT_TINY
    w[sel] = tiny[sel].astype(np.float32)
    sel = cat == CAT_ONE_CHANNEL
    w[sel] = round_bf16(gauss[sel].astype(np.float32))
    for j in np.nonzero(cat == CAT_PAIR_TIE)[0]:
        c = pair_tie_unit(int(c_exp[j]))
        vals = np.concatenate([mult[j] * c, -mult[j] * c])
        w[j] = vals[pair_order[j]].astype(np.float32)
        d[j, 1::2] = d[j, 0::2]                     # environments duplicated in pairs
    d = _normalise_rows(d)
    for j in np.nonzero(cat == CAT_ONE_CHANNEL)[0]:
        d[j, one_env[j]] = 0.0
        d[j, one_env[j], one_chan[j]] = 128.0
    return w, d, c_exp


def make_groups(k: int, idx=None):
    """Per-group config (3): return (w [n,128], d [n,E,128], categories [n], c_exp [n]).

    ``idx`` selects groups (sorted or not); ``None`` means all of them.
    """
    spec = config(k)
    if not spec.per_group:
        raise ValueError("make_groups is for per-group configs")
    cats = config3_categories()
    idx = np.arange(spec.n_groups) if idx is None else np.asarray(idx, dtype=np.int64)
    w = np.empty((idx.size, GROUP), dtype=np.float32)
    d = np.empty((idx.size, spec.E, GROUP), dtype=np.float32)
    ce = np.zeros(idx.size, dtype=np.int64)
    chunks = idx // spec.chunk
    for ch in np.unique(chunks):
        cw, cd, cc = _config3_chunk(int(ch), cats)
        sel = np.nonzero(chunks == ch)[0]
        off = idx[sel] - ch * spec.chunk
        w[sel], d[sel], ce[sel] = cw[off], cd[off], cc[off]
    return w, d, cats[idx], ce


# ---------------------------------------------------------------- samples
def sample_groups(k: int, count: int, salt: int = 0) -> np.ndarray:
    """Seeded uniform sample of global group ids without replacement, sorted."""
    n = config(k).n_groups
    rng = _rng(k, (1 << 21) + salt, _S_PERM)
    return np.sort(rng.choice(n, size=min(count, n), replace=False)).astype(np.int64)


def locate(k: int, gids: np.ndarray):
    """Map global group ids of a matrix config to (matrix index, local group id)."""
    off = config(k).matrix_offsets()
    m = np.searchsorted(off, gids, side="right") - 1
    return m, gids - off[m]


def gather_matrix_groups(k: int, gids: np.ndarray):
    """Return (w [n,128], d [n,E,128], matrix index [n]) for global group ids of a matrix config.

    The diagonal slice each group uses is expanded per group (``d_period = n``).
    """
    spec = config(k)
    gids = np.asarray(gids, dtype=np.int64)
    m_idx, local = locate(k, gids)
    w = np.empty((gids.size, GROUP), dtype=np.float32)
    d = np.empty((gids.size, spec.E, GROUP), dtype=np.float32)
    for m in np.unique(m_idx):
        W, dmat = make_matrix(k, int(m))
        wg, dg, period = matrix_groups(W, dmat)
        sel = np.nonzero(m_idx == m)[0]
        w[sel] = wg[local[sel]]
        d[sel] = dg[local[sel] % period]
    return w, d, m_idx


# ---------------------------------------------------------------- held-out evaluation
def heldout_matrix_diagonals(k: int, m: int) -> np.ndarray:
    """Held-out diagonals [E, in] of matrix ``m`` (configs 0-2): the same per-channel base as the
    calibration diagonals of make_matrix, times a fresh per-environment perturbation.  The stand-in
    for diagonals estimated from held-out text windows disjoint from the calibration windows
    (model card, "Calibration and evaluation data"): the same channels matter, the sampling noise
    differs."""
    spec = config(k)
    if k not in (0, 1, 2):
        raise ValueError("held-out diagonals are drawn for configs 0-2")
    mat = spec.matrices[m]
    return _diag_lognormal_pert(_rng(k, m, _S_DBASE), _rng(k, m, _S_DEVAL), spec.E, mat.inp)


def heldout_sample(k: int, count: int, salt: int = 7):
    """A seeded sample of ``count`` groups across all matrices of config ``k`` (sorted, so each
    matrix's groups are contiguous) with calibration and held-out diagonals expanded per group.
    Returns (w [n,128], d [n,E,128], d_eval [n,E,128], module_offsets [n_modules+1] int64) where
    the modules are the matrices that have at least one sampled group."""
    spec = config(k)
    gids = sample_groups(k, count, salt)
    m_idx, local = locate(k, gids)
    w = np.empty((gids.size, GROUP), dtype=np.float32)
    d = np.empty((gids.size, spec.E, GROUP), dtype=np.float32)
    de = np.empty((gids.size, spec.E, GROUP), dtype=np.float32)
    for m in np.unique(m_idx):
        W, dmat = make_matrix(k, int(m))
        wg, dg, period = matrix_groups(W, dmat)
        _, dge, _ = matrix_groups(W, heldout_matrix_diagonals(k, int(m)))
        sel = np.nonzero(m_idx == m)[0]
        w[sel] = wg[local[sel]]
        d[sel] = dg[local[sel] % period]
        de[sel] = dge[local[sel] % period]
    starts = np.searchsorted(m_idx, np.unique(m_idx), side="left")
    off = np.concatenate([starts, [gids.size]]).astype(np.int64)
    return w, d, de, off


def bootstrap_indices(module_offsets, n_boot: int, seed: int = 0) -> np.ndarray:
    """Resampling draws for a module-stratified bootstrap: int32 [n_boot, n_groups] where entry
    [r, j] for j in module m's range [off[m], off[m+1]) is uniform on that range (with
    replacement).  Only random numbers: the resampling arithmetic lives with the callers."""
    off = np.asarray(module_offsets, dtype=np.int64)
    n = int(off[-1])
    rng = _rng(0, (1 << 22) + seed, _S_BOOT)
    idx = np.empty((n_boot, n), dtype=np.int32)
    for m in range(off.size - 1):
        lo, hi = int(off[m]), int(off[m + 1])
        if hi > lo:
            idx[:, lo:hi] = rng.integers(lo, hi, size=(n_boot, hi - lo), dtype=np.int64)
    return idx


# ---------------------------------------------------------------- calibration activations
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round binary32 values to bfloat16 bit patterns (nearest, ties to even)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def calibration_activations(k: int, m: int, T: int) -> np.ndarray:
    """bfloat16 bit patterns [E, T, in] of calibration activations for matrix ``m`` of config
    ``k`` (configs 0-2): token t of environment e has x_i ~ N(0, base_i pert_{e,i}) with the
    per-channel base and per-environment perturbation of make_matrix's diagonals, so that the
    diagonals estimated from them follow the same structure (model card, "Calibration and
    evaluation data": four environments of 256-token windows; the model runs in 16 bits)."""
    spec = config(k)
    if k not in (0, 1, 2):
        raise ValueError("calibration activations are drawn for configs 0-2")
    inp = spec.matrices[m].inp
    base = _rng(k, m, _S_DBASE).lognormal(0.0, 1.0, size=inp)
    pert = _rng(k, m, _S_DPERT).lognormal(0.0, 0.5, size=(spec.E, inp))
    std = np.sqrt(base[None, :] * pert).astype(np.float32)           # [E, in]
    z = _rng(k, m, _S_ACT).standard_normal(size=(spec.E, T, inp), dtype=np.float32)
    return f32_to_bf16_bits(z * std[:, None, :])


# ---------------------------------------------------------------- the pages' example
def pages_example():
    """The four-weight, two-environment solver input printed in the CliffQuant README
    ("Use the solver").  Python floats there; our boundary is float32, so values are
    rounded to float32.  Zero-padded to one 128-weight group (zeros add nothing to any
    environment's error at any scale)."""
    w = np.zeros((1, GROUP), dtype=np.float32)
    w[0, :4] = np.array([0.9, -0.4, 0.2, -1.1], dtype=np.float32)
    d = np.zeros((1, 2, GROUP), dtype=np.float32)
    d[0, 0, :4] = np.array([1.0, 0.8, 0.5, 1.2], dtype=np.float32)
    d[0, 1, :4] = np.array([0.6, 1.4, 0.9, 0.7], dtype=np.float32)
    return w, d
