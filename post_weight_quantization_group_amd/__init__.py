"""Exact minimax FP16 group scales for W4/G128 quantization on MI355X (gfx950).

A thin ctypes binding over ``libcq.so`` (C ABI in ``include/cq.h``).  The
functions named ``cq_*`` mirror the C entry points one to one and only
marshal arguments: torch tensors already on the GPU are passed by pointer on
the current stream, and a non-OK status raises ``CQError``.  The helpers
without the prefix allocate outputs and a workspace with torch and call the
``cq_*`` functions.  Every step of the computation runs in the HIP kernels;
there is no CPU path, and importing this package on a machine without the
built library raises.

The method (CliffQuant repository README, "What CliffQuant changes"): per
group of 128 weights, the positive finite binary16 scale minimising the worst
environment's diagonal-weighted squared error, codes round-half-even then
clipped to [-8, 7], exact ties to the lower bit pattern; the result is stored
in the GPTQ-v1 layout (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card,
"Quantization configuration").
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CQError", "GROUP", "MAX_GROUP", "EXHAUSTIVE", "CANDIDATE", "BOUNDED", "ABSMAX", "POOLED_WMSE",
    "FLAG_BAD_INPUT", "FLAG_NEAR_TIE", "FLAG_EXACT_TIE", "FLAG_FALLBACK", "FLAG_FP64_SWEEP",
    "library_path", "load", "cq_abi_version", "cq_status_string", "cq_workspace_size",
    "cq_quantize_groups", "cq_quantize_groups_spec", "cq_quantize_groups_noalloc", "cq_baseline_scales",
    "cq_baseline_scales_spec", "cq_proxy_worst_env_wmse_multi_spec",
    "cq_pack_gptq_v1", "cq_pack_gptq_v1_spec",
    "cq_pack_gptq_v1_multi", "pack_gptq_v1_multi", "cq_proxy_workspace_size",
    "cq_proxy_worst_env_wmse", "cq_proxy_worst_env_wmse_multi", "quantize_groups", "baseline_scales",
    "pack_gptq_v1", "proxy_worst_env_wmse", "proxy_worst_env_wmse_multi", "solve_breakpoint_exact",
    "cq_heldout_workspace_size", "cq_heldout_compare", "heldout_compare", "cq_diagonals_workspace_size",
    "cq_environment_diagonals", "environment_diagonals", "cq_w4a16_matmul", "w4a16_matmul", "EXPORTED_SYMBOLS",
    "cq_probe_valu_fma", "probe_valu_fma",
]

GROUP = 128
MAX_GROUP = 256
EXHAUSTIVE, CANDIDATE, BOUNDED = 0, 1, 2
ABSMAX, POOLED_WMSE = 0, 1
FLAG_BAD_INPUT, FLAG_NEAR_TIE, FLAG_EXACT_TIE, FLAG_FALLBACK, FLAG_FP64_SWEEP = 1, 2, 4, 8, 16
_METHODS = {"exhaustive": EXHAUSTIVE, "candidate": CANDIDATE, "bounded": BOUNDED}
EXPORTED_SYMBOLS = ("cq_abi_version", "cq_status_string", "cq_workspace_size", "cq_quantize_groups",
                    "cq_quantize_groups_spec", "cq_quantize_groups_noalloc",
                    "cq_baseline_scales", "cq_baseline_scales_spec", "cq_pack_gptq_v1", "cq_pack_gptq_v1_spec",
                    "cq_pack_gptq_v1_multi", "cq_proxy_worst_env_wmse_multi_spec",
                    "cq_proxy_workspace_size",
                    "cq_proxy_worst_env_wmse", "cq_proxy_worst_env_wmse_multi", "cq_heldout_workspace_size",
                    "cq_heldout_compare", "cq_diagonals_workspace_size", "cq_environment_diagonals",
                    "cq_w4a16_matmul", "cq_probe_valu_fma")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class CQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {cq_status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.environ.get("CQ_LIBRARY", os.path.join(_HERE, "libcq.so"))


def load():
    """Load libcq.so (raises when it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m post_weight_quantization_group_amd.build`")
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.cq_abi_version.restype = I32
        lib.cq_abi_version.argtypes = []
        lib.cq_status_string.restype = ctypes.c_char_p
        lib.cq_status_string.argtypes = [I32]
        lib.cq_workspace_size.restype = SZ
        lib.cq_workspace_size.argtypes = [I32, I32, I64]
        lib.cq_quantize_groups.restype = I32
        lib.cq_quantize_groups.argtypes = [P, P, I64, I32, I64, I32, P, P, P, P, P, P, P, SZ, P]
        lib.cq_quantize_groups_noalloc.restype = I32
        lib.cq_quantize_groups_noalloc.argtypes = [P, P, I64, I32, I64, I32, P, P, P, P, P, P, P]
        lib.cq_quantize_groups_spec.restype = I32
        lib.cq_quantize_groups_spec.argtypes = [P, P, I32, I32, I32, I64, I32, I64, I32, P, P, P, P, P, P, P, SZ, P]
        lib.cq_baseline_scales.restype = I32
        lib.cq_baseline_scales.argtypes = [P, P, I64, I32, I64, I32, P, P, P, P, SZ, P]
        lib.cq_pack_gptq_v1.restype = I32
        lib.cq_pack_gptq_v1.argtypes = [P, P, I64, I64, P, P, P]
        lib.cq_pack_gptq_v1_spec.restype = I32
        lib.cq_baseline_scales_spec.restype = I32
        lib.cq_baseline_scales_spec.argtypes = [P, P, I32, I32, I32, I64, I32, I64, I32, P, P, P, P, SZ, P]
        lib.cq_proxy_worst_env_wmse_multi_spec.restype = I32
        lib.cq_proxy_worst_env_wmse_multi_spec.argtypes = [P, P, I32, I32, I32, I64, I32, I64, I32, P, P, I32, P, P,
                                                           P, P, SZ, P]
        lib.cq_pack_gptq_v1_spec.argtypes = [P, P, I64, I64, I32, I32, P, P, P]
        lib.cq_pack_gptq_v1_multi.restype = I32
        lib.cq_pack_gptq_v1_multi.argtypes = [P, P, I32, P, P, P, P, P]
        lib.cq_proxy_workspace_size.restype = SZ
        lib.cq_proxy_workspace_size.argtypes = [I64]
        lib.cq_proxy_worst_env_wmse.restype = I32
        lib.cq_proxy_worst_env_wmse.argtypes = [P, P, I64, I32, I64, P, P, I32, P, P, P, P, SZ, P]
        lib.cq_proxy_worst_env_wmse_multi.restype = I32
        lib.cq_proxy_worst_env_wmse_multi.argtypes = [P, P, I64, I32, I64, I32, P, P, I32, P, P, P, P, SZ, P]
        lib.cq_w4a16_matmul.restype = I32
        lib.cq_w4a16_matmul.argtypes = [P, P, P, I64, I64, I64, P, P]
        lib.cq_diagonals_workspace_size.restype = SZ
        lib.cq_diagonals_workspace_size.argtypes = [I32, I64, I64]
        lib.cq_environment_diagonals.restype = I32
        lib.cq_environment_diagonals.argtypes = [P, I32, I64, I64, P, P, SZ, P]
        lib.cq_heldout_workspace_size.restype = SZ
        lib.cq_heldout_workspace_size.argtypes = [I32, I32]
        lib.cq_heldout_compare.restype = I32
        lib.cq_heldout_compare.argtypes = [P, P, I64, P, I32, P, I32, ctypes.c_double, P, P, P, P, P, SZ, P]
        lib.cq_probe_valu_fma.restype = I32
        lib.cq_probe_valu_fma.argtypes = [I32, I32, I32, P, P, ctypes.POINTER(ctypes.c_double), P]
        _lib = lib
    return _lib


# ---------------------------------------------------------------- marshalling
def _p(t):
    """Device pointer of a CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("arrays passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("arrays passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise CQError(status, where)


# ---------------------------------------------------------------- C entry points
def cq_abi_version() -> int:
    return load().cq_abi_version()


def cq_status_string(status: int) -> str:
    return load().cq_status_string(status).decode()


def cq_workspace_size(method: int, E: int, n_groups: int) -> int:
    return load().cq_workspace_size(method, E, n_groups)


def cq_proxy_workspace_size(n_groups: int) -> int:
    return load().cq_proxy_workspace_size(n_groups)


def cq_quantize_groups(w, d, d_period, E, n_groups, method, scales, codes=None, objective=None, flags=None,
                       pooled_scales=None, pooled_objective=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_quantize_groups(_p(w), _p(d), d_period, E, n_groups, method, _p(scales), _p(codes),
                                     _p(objective), _p(flags), _p(pooled_scales), _p(pooled_objective),
                                     _p(workspace), ws_bytes, _stream(stream)), "cq_quantize_groups")


def cq_quantize_groups_noalloc(w, d, d_period, E, n_groups, method, scales, codes=None, objective=None, flags=None,
                               pooled_scales=None, pooled_objective=None, stream=None):
    _check(load().cq_quantize_groups_noalloc(_p(w), _p(d), d_period, E, n_groups, method, _p(scales), _p(codes),
                                             _p(objective), _p(flags), _p(pooled_scales), _p(pooled_objective),
                                             _stream(stream)), "cq_quantize_groups_noalloc")


def cq_quantize_groups_spec(w, d, group_len, qmin, qmax, d_period, E, n_groups, method, scales, codes=None,
                            objective=None, flags=None, pooled_scales=None, pooled_objective=None, workspace=None,
                            stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_quantize_groups_spec(_p(w), _p(d), group_len, qmin, qmax, d_period, E, n_groups, method,
                                          _p(scales), _p(codes), _p(objective), _p(flags), _p(pooled_scales),
                                          _p(pooled_objective), _p(workspace), ws_bytes, _stream(stream)),
           "cq_quantize_groups_spec")


def cq_baseline_scales(w, d, d_period, E, n_groups, which, scales, codes=None, objective=None, workspace=None,
                       stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_baseline_scales(_p(w), _p(d), d_period, E, n_groups, which, _p(scales), _p(codes),
                                     _p(objective), _p(workspace), ws_bytes, _stream(stream)),
           "cq_baseline_scales")


def cq_pack_gptq_v1(codes, grp_scales, out, inp, qweight, scales, stream=None):
    _check(load().cq_pack_gptq_v1(_p(codes), _p(grp_scales), out, inp, _p(qweight), _p(scales),
                                  _stream(stream)), "cq_pack_gptq_v1")


def cq_baseline_scales_spec(w, d, group_len, qmin, qmax, d_period, E, n_groups, which, scales, codes=None,
                            objective=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_baseline_scales_spec(_p(w), _p(d), group_len, qmin, qmax, d_period, E, n_groups, which,
                                          _p(scales), _p(codes), _p(objective), _p(workspace), ws_bytes,
                                          _stream(stream)), "cq_baseline_scales_spec")


def cq_proxy_worst_env_wmse_multi_spec(w, d_eval, group_len, qmin, qmax, d_period, E, n_groups, n_policies, scales,
                                       module_offsets, n_modules, module_mean, macro, per_group=None,
                                       workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_proxy_worst_env_wmse_multi_spec(_p(w), _p(d_eval), group_len, qmin, qmax, d_period, E,
                                                     n_groups, n_policies, _p(scales), _p(module_offsets),
                                                     n_modules, _p(module_mean), _p(macro), _p(per_group),
                                                     _p(workspace), ws_bytes, _stream(stream)),
           "cq_proxy_worst_env_wmse_multi_spec")


def cq_pack_gptq_v1_spec(codes, grp_scales, out, inp, bits, group_len, qweight, scales, stream=None):
    _check(load().cq_pack_gptq_v1_spec(_p(codes), _p(grp_scales), out, inp, bits, group_len, _p(qweight),
                                       _p(scales), _stream(stream)), "cq_pack_gptq_v1_spec")


def cq_pack_gptq_v1_multi(codes, grp_scales, n_mats, outs, ins, qweight, scales, stream=None):
    """outs, ins: host sequences of n_mats shapes (marshalled to int64 host arrays)."""
    o = (ctypes.c_int64 * max(1, n_mats))(*[int(x) for x in outs])
    i = (ctypes.c_int64 * max(1, n_mats))(*[int(x) for x in ins])
    _check(load().cq_pack_gptq_v1_multi(_p(codes), _p(grp_scales), n_mats, ctypes.cast(o, ctypes.c_void_p),
                                        ctypes.cast(i, ctypes.c_void_p), _p(qweight), _p(scales), _stream(stream)),
           "cq_pack_gptq_v1_multi")


def cq_proxy_worst_env_wmse(w, d_eval, d_period, E, n_groups, scales, module_offsets, n_modules, module_mean,
                            macro, per_group=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_proxy_worst_env_wmse(_p(w), _p(d_eval), d_period, E, n_groups, _p(scales),
                                          _p(module_offsets), n_modules, _p(module_mean), _p(macro),
                                          _p(per_group), _p(workspace), ws_bytes, _stream(stream)),
           "cq_proxy_worst_env_wmse")


def cq_proxy_worst_env_wmse_multi(w, d_eval, d_period, E, n_groups, n_policies, scales, module_offsets, n_modules,
                                  module_mean, macro, per_group=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_proxy_worst_env_wmse_multi(_p(w), _p(d_eval), d_period, E, n_groups, n_policies, _p(scales),
                                                _p(module_offsets), n_modules, _p(module_mean), _p(macro),
                                                _p(per_group), _p(workspace), ws_bytes, _stream(stream)),
           "cq_proxy_worst_env_wmse_multi")


def cq_w4a16_matmul(x, qweight, scales, M, out, inp, y, stream=None):
    _check(load().cq_w4a16_matmul(_p(x), _p(qweight), _p(scales), M, out, inp, _p(y), _stream(stream)),
           "cq_w4a16_matmul")


def w4a16_matmul(x, qweight, scales, stream=None):
    """y [M, out] float32 = x [M, in] (bfloat16, or int16 bit patterns) times the dequantized
    GPTQ-v1 tensors (qweight int32 [in/8, out], scales int16 binary16 bits [in/128, out])."""
    M, inp = x.shape
    out = qweight.shape[1]
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    y = torch.empty((M, out), dtype=torch.float32, device=x.device)
    cq_w4a16_matmul(xb, qweight, scales, M, out, inp, y, stream)
    return y


def cq_probe_valu_fma(iters, blocks, mode, out, clocks, stream=None) -> float:
    """Runs the fp32 fma issue probe; returns the wall clock's rate in Hz."""
    hz = ctypes.c_double(0.0)
    _check(load().cq_probe_valu_fma(iters, blocks, mode, _p(out), _p(clocks), ctypes.byref(hz), _stream(stream)),
           "cq_probe_valu_fma")
    return hz.value


def probe_valu_fma(iters: int, blocks: int, mode: int = 1, device="cuda", stream=None) -> dict:
    """The issue probe on `blocks` workgroups (mode 0: v_fma_f32, 1: v_fmac_f32, 2: v_fma_f32
    with a scalar operand): the sums,
    per-workgroup (shader cycles, wall ticks) and the wall clock's rate.  The caller times the
    launch."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    clocks = torch.empty((blocks, 2), dtype=torch.int64, device=device)
    hz = cq_probe_valu_fma(iters, blocks, mode, out, clocks, stream)
    return {"out": out, "clocks": clocks, "wall_clock_hz": hz}


def cq_diagonals_workspace_size(E: int, T: int, inp: int) -> int:
    return load().cq_diagonals_workspace_size(E, T, inp)


def cq_environment_diagonals(x, E, T, inp, d, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_environment_diagonals(_p(x), E, T, inp, _p(d), _p(workspace), ws_bytes, _stream(stream)),
           "cq_environment_diagonals")


def cq_heldout_workspace_size(n_boot: int, n_modules: int) -> int:
    return load().cq_heldout_workspace_size(n_boot, n_modules)


def cq_heldout_compare(pa, pb, n_groups, module_offsets, n_modules, boot_idx, n_boot, alpha, counts, effect, boot,
                       ci, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().cq_heldout_compare(_p(pa), _p(pb), n_groups, _p(module_offsets), n_modules, _p(boot_idx), n_boot,
                                     float(alpha), _p(counts), _p(effect), _p(boot), _p(ci), _p(workspace), ws_bytes,
                                     _stream(stream)), "cq_heldout_compare")


# ---------------------------------------------------------------- helpers
def _workspace(nbytes: int, device):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _shape_check(w, d):
    if w.dim() != 2 or w.shape[1] != GROUP or w.dtype != torch.float32:
        raise ValueError("w must be float32 [n_groups, 128]")
    if d.dim() != 3 or d.shape[2] != GROUP or d.dtype != torch.float32:
        raise ValueError("d must be float32 [n_d, E, 128]")


def _spec_shape(w, d, qmin, qmax):
    """(G, spec): G from w; spec is True unless the quantizer is the pages' (G = 128, [-8, 7])."""
    G = w.shape[1] if w.dim() == 2 else -1
    spec = (G, int(qmin), int(qmax)) != (GROUP, -8, 7)
    if spec:
        if w.dim() != 2 or not 1 <= G <= MAX_GROUP or w.dtype != torch.float32:
            raise ValueError("w must be float32 [n_groups, G] with 1 <= G <= 256")
        if d.dim() != 3 or d.shape[2] != G or d.dtype != torch.float32:
            raise ValueError("d must be float32 [n_d, E, G]")
    else:
        _shape_check(w, d)
    return G, spec


def quantize_groups(w, d, d_period=None, method="exhaustive", codes=True, pooled=False, workspace=None,
                    stream=None, qmin=-8, qmax=7):
    """Minimax scales (and codes, objective, flags; optionally the pooled policy) for every group.

    w is float32 [n_groups, G] and d float32 [n_d, E, G]; G = 128 with codes in [qmin, qmax] =
    [-8, 7] is the pages' quantizer, any other G <= 256 or range goes through
    cq_quantize_groups_spec (method "exhaustive", or "candidate" for G <= 128 and
    -8 <= qmin, qmax <= 8).  method: "exhaustive" (every scale), "bounded" (branch and bound) or
    "candidate"; all give the same result.
    Returns a dict of device tensors: scales (uint16 bit patterns held in int16
    storage -> use ``.view(torch.uint16)`` or ``& 0xFFFF``), codes, objective,
    flags and, with ``pooled=True``, pooled_scales and pooled_objective.
    """
    G, spec = _spec_shape(w, d, qmin, qmax)
    n, E = w.shape[0], d.shape[1]
    d_period = d.shape[0] if d_period is None else int(d_period)
    m = _METHODS[method] if isinstance(method, str) else int(method)
    dev = w.device
    out = {
        "scales": torch.empty(n, dtype=torch.int16, device=dev),
        "codes": torch.empty((n, G), dtype=torch.int8, device=dev) if codes else None,
        "objective": torch.empty(n, dtype=torch.float64, device=dev),
        "flags": torch.empty(n, dtype=torch.uint8, device=dev),
    }
    if pooled:
        out["pooled_scales"] = torch.empty(n, dtype=torch.int16, device=dev)
        out["pooled_objective"] = torch.empty(n, dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = _workspace(cq_workspace_size(m, E, n), dev)
    if spec:
        cq_quantize_groups_spec(w, d, G, qmin, qmax, d_period, E, n, m, out["scales"], out["codes"], out["objective"],
                                out["flags"], out.get("pooled_scales"), out.get("pooled_objective"), workspace, stream)
    else:
        cq_quantize_groups(w, d, d_period, E, n, m, out["scales"], out["codes"], out["objective"], out["flags"],
                           out.get("pooled_scales"), out.get("pooled_objective"), workspace, stream)
    return out


def baseline_scales(w, d, d_period=None, which="absmax", codes=True, objective=True, workspace=None,
                    stream=None, qmin=-8, qmax=7):
    """AbsMax or pooled-WMSE scales: dict with scales, codes, objective.  Another group length
    (w [n_groups, G], d [n_d, E, G]) or code range goes through cq_baseline_scales_spec."""
    G, spec = _spec_shape(w, d, qmin, qmax)
    n, E = w.shape[0], d.shape[1]
    d_period = d.shape[0] if d_period is None else int(d_period)
    k = {"absmax": ABSMAX, "pooled": POOLED_WMSE}[which] if isinstance(which, str) else int(which)
    dev = w.device
    out = {
        "scales": torch.empty(n, dtype=torch.int16, device=dev),
        "codes": torch.empty((n, G), dtype=torch.int8, device=dev) if codes else None,
        "objective": torch.empty(n, dtype=torch.float64, device=dev) if objective else None,
    }
    if k == POOLED_WMSE and workspace is None:
        workspace = _workspace(cq_workspace_size(EXHAUSTIVE, E, n), dev)
    if spec:
        cq_baseline_scales_spec(w, d, G, qmin, qmax, d_period, E, n, k, out["scales"], out["codes"],
                                out["objective"], workspace, stream)
    else:
        cq_baseline_scales(w, d, d_period, E, n, k, out["scales"], out["codes"], out["objective"], workspace,
                           stream)
    return out


def pack_gptq_v1(codes, grp_scales, out: int, inp: int, stream=None, bits: int = 4, group: int = GROUP):
    """GPTQ-v1 (qweight int32 [in*bits/32, out], scales int16-stored fp16 bits [in/group, out]);
    4-bit fields and groups of 128 by default, else bits in {2, 4, 8} and any group length."""
    qweight = torch.empty((inp * bits // 32, out), dtype=torch.int32, device=codes.device)
    scales = torch.empty((inp // group, out), dtype=torch.int16, device=codes.device)
    if bits == 4 and group == GROUP:
        cq_pack_gptq_v1(codes, grp_scales, out, inp, qweight, scales, stream)
    else:
        cq_pack_gptq_v1_spec(codes, grp_scales, out, inp, bits, group, qweight, scales, stream)
    return qweight, scales


def pack_gptq_v1_multi(codes, grp_scales, shapes, stream=None):
    """GPTQ-v1 packing of several matrices in one launch.  codes int8 and grp_scales int16 (binary16
    bits) hold the matrices back to back (flat, or any contiguous tensor); shapes is a list of
    (out, in).  Returns (qweight, scales) as flat int32 and int16 tensors holding each matrix's
    [in/8, out] and [in/128, out] blocks back to back."""
    n_el = sum(int(o) * int(i) for o, i in shapes)
    qweight = torch.empty(n_el // 8, dtype=torch.int32, device=codes.device)
    scales = torch.empty(n_el // GROUP, dtype=torch.int16, device=codes.device)
    cq_pack_gptq_v1_multi(codes, grp_scales, len(shapes), [o for o, _ in shapes], [i for _, i in shapes], qweight,
                          scales, stream)
    return qweight, scales


def proxy_worst_env_wmse(w, d_eval, scales, module_offsets, d_period=None, per_group=True, stream=None):
    """(per_group or None, module_mean [n_modules], macro [1]) as float64 device tensors."""
    _shape_check(w, d_eval)
    n, E = w.shape[0], d_eval.shape[1]
    d_period = d_eval.shape[0] if d_period is None else int(d_period)
    n_modules = module_offsets.numel() - 1
    dev = w.device
    mm = torch.empty(n_modules, dtype=torch.float64, device=dev)
    macro = torch.empty(1, dtype=torch.float64, device=dev)
    pg = torch.empty(n, dtype=torch.float64, device=dev) if per_group else None
    ws = None if per_group else _workspace(cq_proxy_workspace_size(n), dev)
    cq_proxy_worst_env_wmse(w, d_eval, d_period, E, n, scales, module_offsets, n_modules, mm, macro, pg, ws,
                            stream)
    return pg, mm, macro


def proxy_worst_env_wmse_multi(w, d_eval, scales, module_offsets, d_period=None, per_group=True, stream=None,
                               qmin=-8, qmax=7):
    """The proxy for several policies at once: scales [P, n_groups] int16 on the device.
    Returns (per_group [P, n] or None, module_mean [P, n_modules], macro [P]) as float64 device tensors.
    Another group length or code range goes through cq_proxy_worst_env_wmse_multi_spec."""
    G, spec = _spec_shape(w, d_eval, qmin, qmax)
    n, E = w.shape[0], d_eval.shape[1]
    if scales.dim() != 2 or scales.shape[1] != n:
        raise ValueError("scales must be [n_policies, n_groups]")
    n_pol = scales.shape[0]
    d_period = d_eval.shape[0] if d_period is None else int(d_period)
    n_modules = module_offsets.numel() - 1
    dev = w.device
    mm = torch.empty((n_pol, n_modules), dtype=torch.float64, device=dev)
    macro = torch.empty(n_pol, dtype=torch.float64, device=dev)
    pg = torch.empty((n_pol, n), dtype=torch.float64, device=dev) if per_group else None
    ws = None if per_group else _workspace(cq_proxy_workspace_size(n * n_pol), dev)
    if spec:
        cq_proxy_worst_env_wmse_multi_spec(w, d_eval, G, qmin, qmax, d_period, E, n, n_pol, scales, module_offsets,
                                           n_modules, mm, macro, pg, ws, stream)
    else:
        cq_proxy_worst_env_wmse_multi(w, d_eval, d_period, E, n, n_pol, scales, module_offsets, n_modules, mm,
                                      macro, pg, ws, stream)
    return pg, mm, macro


def environment_diagonals(x, stream=None):
    """Diagonals [in/128, E, 128] float32 from bfloat16 activations x [E, T, in] (a torch.bfloat16
    or int16 device tensor holding the bit patterns)."""
    if x.dim() != 3:
        raise ValueError("x must be [E, T, in]")
    E, T, inp = x.shape
    xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    d = torch.empty((inp // GROUP, E, GROUP), dtype=torch.float32, device=x.device)
    ws = _workspace(cq_diagonals_workspace_size(E, T, inp), x.device)
    cq_environment_diagonals(xb, E, T, inp, d, ws, stream)
    return d


def heldout_compare(pa, pb, module_offsets, boot_idx, alpha=0.05, stream=None):
    """Policy A against policy B on per-group proxy values (float64 [n] device tensors), with the
    bootstrap draws boot_idx (int32 [n_boot, n] device tensor).  Returns (counts int64 [3] =
    wins/ties/losses of A, effect [1], replicates [n_boot] sorted, ci [2]) as device tensors."""
    n = pa.numel()
    n_modules = module_offsets.numel() - 1
    n_boot = boot_idx.shape[0] if boot_idx is not None else 0
    dev = pa.device
    counts = torch.empty(3, dtype=torch.int64, device=dev)
    effect = torch.empty(1, dtype=torch.float64, device=dev)
    boot = torch.empty(max(n_boot, 1), dtype=torch.float64, device=dev)
    ci = torch.empty(2, dtype=torch.float64, device=dev)
    ws = _workspace(cq_heldout_workspace_size(n_boot, n_modules), dev)
    cq_heldout_compare(pa, pb, n, module_offsets, n_modules, boot_idx if n_boot > 0 else None, n_boot, alpha, counts,
                       effect, boot, ci, ws, stream)
    return counts, effect, boot[:n_boot], ci


def solve_breakpoint_exact(weights, environment_diagonals, qmin: int = -8, qmax: int = 7, method=None,
                           device="cuda"):
    """One group, in the shape of the pages' solver call (CliffQuant README, "Use the solver": the
    weights, the environment diagonals and a quantizer specification with qmin and qmax).

    ``weights`` has at most 256 entries, ``environment_diagonals`` is [E][len(weights)].  For
    the pages' range [-8, 7] a group shorter than 128 is zero-padded to 128 (a zero weight adds
    nothing at any scale) and any method serves it (default "candidate"); other ranges run the
    group at its own length, by default through the candidate solver where it takes the
    quantizer (at most 128 weights, -8 <= qmin, qmax <= 8) and the exhaustive method elsewhere.
    Returns (scale as float, objective, codes list).
    """
    n = len(weights)
    if not 1 <= n <= MAX_GROUP:
        raise ValueError("1..256 weights")
    E = len(environment_diagonals)
    L = GROUP if (qmin, qmax) == (-8, 7) and n <= GROUP else n
    if method is None:
        method = "candidate" if L <= GROUP and qmin >= -8 and qmax <= 8 else "exhaustive"
    w = torch.zeros((1, L), dtype=torch.float32)
    w[0, :n] = torch.tensor(weights, dtype=torch.float32)
    d = torch.zeros((1, E, L), dtype=torch.float32)
    d[0, :, :n] = torch.tensor(environment_diagonals, dtype=torch.float32)
    r = quantize_groups(w.to(device), d.to(device), method=method, qmin=qmin, qmax=qmax)
    torch.cuda.current_stream().synchronize()
    bits = int(r["scales"].cpu().view(torch.uint16)[0]) if hasattr(torch, "uint16") else \
        int(r["scales"].cpu()[0]) & 0xFFFF
    scale = float(torch.tensor([bits], dtype=torch.int16).view(torch.float16)[0])
    return scale, float(r["objective"].cpu()[0]), r["codes"].cpu()[0, :n].tolist()
