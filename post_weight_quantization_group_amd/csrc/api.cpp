// C ABI of the scale-selection library: argument checks, workspace carving,
// and kernel launches on the caller's stream.  Declared in include/cq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "cq.h"
#include "launch.h"

namespace {

constexpr size_t ALIGN = 256;
inline size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int32_t hip_status(hipError_t e) { return e == hipSuccess ? CQ_OK : CQ_EHIP; }

// Full-grid workspace: [counter | pad][int32 queue of n_groups]
size_t full_ws(int64_t n) { return ALIGN + round_up((size_t)n * 4u); }
// Bounded-sweep workspace: [counter | pad][int32 queue of n_groups][slice parts]
size_t sweep_ws(int64_t n) { return full_ws(n) + round_up(sizeof(cqk::SlicePart) * cqk::SLICE_PARTS); }
// Candidate workspace: [tie counter | pad][int32 tie list][sweep workspace]
size_t cand_ws(int64_t n) { return ALIGN + round_up((size_t)n * 4u) + sweep_ws(n); }

bool groups_ok(const float* w, const float* d, int64_t d_period, int32_t E, int64_t n_groups, size_t align = 16) {
    if (n_groups < 0 || E < 1 || E > CQ_MAX_ENVS) return false;
    if (n_groups == 0) return true;
    if (!w || !d || d_period < 1) return false;
    return aligned(w, align) && aligned(d, align);
}

bool spec_ok(int32_t G, int32_t qmin, int32_t qmax) {
    return G >= 1 && G <= CQ_MAX_GROUP && qmin >= -128 && qmin <= 0 && qmax >= 0 && qmax <= 127 && qmin < qmax;
}

// Quantizers the candidate solver takes besides the pages' own: at most 8 codes on each side of
// zero (8 transition slots per weight) and groups of at most 128 weights.
bool cand_spec_ok(int32_t G, int32_t qmin, int32_t qmax) { return G <= CQ_GROUP && qmin >= -8 && qmax <= 8; }

int32_t run_fullgrid(const float* w, const float* d, int32_t G, int32_t qmin, int32_t qmax, int64_t d_period, int32_t E,
                     int64_t n_groups, uint16_t* scales, int8_t* codes, double* objective, uint8_t* flags,
                     uint16_t* pooled_scales, double* pooled_objective, int want_minimax, uint8_t* ws,
                     hipStream_t st) {
    cqk::FullArgs a{};
    a.w = w; a.d = d; a.d_period = d_period; a.G = G; a.qmin = qmin; a.qmax = qmax;
    a.ratio = cqk::fullgrid_ratio(G, qmin, qmax, E);
    a.scales = scales; a.codes = codes; a.objective = objective; a.flags = flags;
    a.pscales = pooled_scales; a.pobjective = pooled_objective;
    a.want_minimax = want_minimax;
    a.want_pooled = (pooled_scales || pooled_objective) ? 1 : 0;
    a.fb_count = (int32_t*)ws;
    a.fb_list = (int32_t*)(ws + ALIGN);
    a.parts = (cqk::SlicePart*)(ws + full_ws(n_groups));  // the workspace is sweep_ws(n_groups) bytes
    return hip_status(cqk::launch_fullgrid(a, E, n_groups, st));
}

}  // namespace

extern "C" {

int32_t cq_abi_version(void) { return CQ_ABI_VERSION; }

const char* cq_status_string(int32_t s) {
    switch (s) {
        case CQ_OK: return "ok";
        case CQ_EINVAL: return "invalid argument";
        case CQ_EWORKSPACE: return "workspace missing, misaligned or too small";
        case CQ_EHIP: return "HIP launch failed";
        case CQ_EUNSUPPORTED: return "not supported by this entry point";
        case CQ_ELIMIT: return "more groups than the fixed scratch of the no-allocation entry point holds";
        default: return "unknown status";
    }
}

size_t cq_workspace_size(int32_t method, int32_t E, int64_t n_groups) {
    if (E < 1 || E > CQ_MAX_ENVS || n_groups < 0) return 0;
    // the full grid needs less than the bounded sweep; one size serves both, and the pooled
    // baseline (a bounded sweep) accepts the CQ_EXHAUSTIVE size too
    if (method == CQ_EXHAUSTIVE || method == CQ_BOUNDED) return sweep_ws(n_groups);
    if (method == CQ_CANDIDATE) return cand_ws(n_groups);
    return 0;
}

int32_t cq_quantize_groups(const float* w, const float* d, int64_t d_period, int32_t E, int64_t n_groups,
                           int32_t method, uint16_t* scales, int8_t* codes, double* objective, uint8_t* flags,
                           uint16_t* pooled_scales, double* pooled_objective, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!groups_ok(w, d, d_period, E, n_groups)) return CQ_EINVAL;
    if (method != CQ_EXHAUSTIVE && method != CQ_CANDIDATE && method != CQ_BOUNDED) return CQ_EINVAL;
    if (n_groups > 0 && !scales) return CQ_EINVAL;
    if (n_groups > INT32_MAX) return CQ_EINVAL;
    if (method == CQ_CANDIDATE && (pooled_scales || pooled_objective)) return CQ_EUNSUPPORTED;
    if (n_groups == 0) return CQ_OK;
    const size_t need = cq_workspace_size(method, E, n_groups);
    if (!workspace || workspace_bytes < need || !aligned(workspace, ALIGN)) return CQ_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    if (method == CQ_EXHAUSTIVE)
        return run_fullgrid(w, d, CQ_GROUP, -8, 7, d_period, E, n_groups, scales, codes, objective, flags,
                            pooled_scales, pooled_objective, 1, ws, st);
    if (method == CQ_BOUNDED) {
        cqk::SweepArgs a{};
        a.w = w; a.d = d; a.d_period = d_period;
        a.scales = scales; a.codes = codes; a.objective = objective; a.flags = flags;
        a.pscales = pooled_scales; a.pobjective = pooled_objective;
        a.fb_count = (int32_t*)ws;
        a.fb_list = (int32_t*)(ws + ALIGN);
        a.parts = (cqk::SlicePart*)(ws + ALIGN + round_up((size_t)n_groups * 4u));
        a.want_minimax = 1;
        a.want_pooled = (pooled_scales || pooled_objective) ? 1 : 0;
        return hip_status(cqk::launch_sweep(a, E, n_groups, st));
    }
    cqk::CandArgs c{};
    c.w = w; c.d = d; c.d_period = d_period; c.n_groups = n_groups;
    c.G = CQ_GROUP; c.qmin = -8; c.qmax = 7; c.start_ratio = 1.0f / 9.0f;
    c.scales = scales; c.codes = codes; c.objective = objective; c.flags = flags;
    c.tie_count = (int32_t*)ws;
    c.tie_list = (int32_t*)(ws + ALIGN);
    // groups whose direct candidates tied are decided by the exhaustive sweep, whose binary64
    // queue counter is cleared together with the tie counter
    uint8_t* sws = ws + ALIGN + round_up((size_t)n_groups * 4u);
    c.zero_also = (int32_t*)sws;
    hipError_t e = cqk::launch_candidate(c, E, st);
    if (e != hipSuccess) return CQ_EHIP;
    cqk::SweepArgs a{};
    a.w = w; a.d = d; a.d_period = d_period;
    a.list = c.tie_list; a.list_count = c.tie_count;
    a.scales = scales; a.codes = codes; a.objective = objective; a.flags = flags;
    a.fb_count = (int32_t*)sws;
    a.fb_list = (int32_t*)(sws + ALIGN);
    a.parts = (cqk::SlicePart*)(sws + ALIGN + round_up((size_t)n_groups * 4u));
    a.want_minimax = 1;
    a.want_pooled = 0;
    a.mark_fallback = 1;
    a.fb_zeroed = 1;
    return hip_status(cqk::launch_sweep(a, E, n_groups, st));
}

int32_t cq_quantize_groups_spec(const float* w, const float* d, int32_t group_len, int32_t qmin, int32_t qmax,
                                int64_t d_period, int32_t E, int64_t n_groups, int32_t method, uint16_t* scales,
                                int8_t* codes, double* objective, uint8_t* flags, uint16_t* pooled_scales,
                                double* pooled_objective, void* workspace, size_t workspace_bytes, void* stream) {
    if (!spec_ok(group_len, qmin, qmax)) return CQ_EINVAL;
    if (method != CQ_EXHAUSTIVE && method != CQ_CANDIDATE && method != CQ_BOUNDED) return CQ_EINVAL;
    if (group_len == CQ_GROUP && qmin == -8 && qmax == 7)
        return cq_quantize_groups(w, d, d_period, E, n_groups, method, scales, codes, objective, flags, pooled_scales,
                                  pooled_objective, workspace, workspace_bytes, stream);
    const bool cand = method == CQ_CANDIDATE && cand_spec_ok(group_len, qmin, qmax);
    if (method != CQ_EXHAUSTIVE && !cand) return CQ_EUNSUPPORTED;
    if (!groups_ok(w, d, d_period, E, n_groups, 4)) return CQ_EINVAL;
    if (n_groups > 0 && !scales) return CQ_EINVAL;
    if (n_groups > INT32_MAX) return CQ_EINVAL;
    if (cand && (pooled_scales || pooled_objective)) return CQ_EUNSUPPORTED;
    if (n_groups == 0) return CQ_OK;
    if (!workspace || workspace_bytes < cq_workspace_size(method, E, n_groups) || !aligned(workspace, ALIGN))
        return CQ_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    if (!cand)
        return run_fullgrid(w, d, group_len, qmin, qmax, d_period, E, n_groups, scales, codes, objective, flags,
                            pooled_scales, pooled_objective, 1, ws, st);
    // the candidate solver; the groups whose direct candidates tied are decided by the full grid
    // (list mode), which takes every quantizer
    cqk::CandArgs c{};
    c.w = w; c.d = d; c.d_period = d_period; c.n_groups = n_groups;
    c.G = group_len; c.qmin = qmin; c.qmax = qmax;
    c.start_ratio = 1.0f / (float)((-qmin > qmax ? -qmin : qmax) + 1);
    c.scales = scales; c.codes = codes; c.objective = objective; c.flags = flags;
    c.tie_count = (int32_t*)ws;
    c.tie_list = (int32_t*)(ws + ALIGN);
    uint8_t* fws = ws + ALIGN + round_up((size_t)n_groups * 4u);  // sweep_ws(n_groups) bytes
    hipError_t e = cqk::launch_candidate(c, E, st);
    if (e != hipSuccess) return CQ_EHIP;
    cqk::FullArgs a{};
    a.w = w; a.d = d; a.d_period = d_period; a.G = group_len; a.qmin = qmin; a.qmax = qmax;
    a.ratio = cqk::fullgrid_ratio(group_len, qmin, qmax, E);
    a.scales = scales; a.codes = codes; a.objective = objective; a.flags = flags;
    a.want_minimax = 1;
    a.want_pooled = 0;
    a.fb_count = (int32_t*)fws;
    a.fb_list = (int32_t*)(fws + ALIGN);
    a.parts = (cqk::SlicePart*)(fws + full_ws(n_groups));
    a.list = c.tie_list;
    a.list_count = c.tie_count;
    a.flag_or = CQ_FLAG_FALLBACK;
    return hip_status(cqk::launch_fullgrid(a, E, n_groups, st));
}

int32_t cq_baseline_scales(const float* w, const float* d, int64_t d_period, int32_t E, int64_t n_groups,
                           int32_t which, uint16_t* scales, int8_t* codes, double* objective, void* workspace,
                           size_t workspace_bytes, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (n_groups < 0 || n_groups > INT32_MAX) return CQ_EINVAL;
    if (which == CQ_ABSMAX) {
        if (n_groups == 0) return CQ_OK;
        if (!w || !scales || !aligned(w, 16) || (codes && !aligned(codes, 16))) return CQ_EINVAL;
        if (objective && !groups_ok(w, d, d_period, E, n_groups)) return CQ_EINVAL;
        return hip_status(cqk::launch_absmax(w, d, d_period, E, n_groups, scales, codes, objective, st));
    }
    if (which != CQ_POOLED_WMSE) return CQ_EINVAL;
    if (!groups_ok(w, d, d_period, E, n_groups)) return CQ_EINVAL;
    if (n_groups == 0) return CQ_OK;
    if (!scales) return CQ_EINVAL;
    const size_t need = cq_workspace_size(CQ_BOUNDED, E, n_groups);
    if (!workspace || workspace_bytes < need || !aligned(workspace, ALIGN)) return CQ_EWORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    cqk::SweepArgs a{};
    a.w = w; a.d = d; a.d_period = d_period;
    a.codes = codes; a.pscales = scales; a.pobjective = objective;
    a.fb_count = (int32_t*)ws;
    a.fb_list = (int32_t*)(ws + ALIGN);
    a.parts = (cqk::SlicePart*)(ws + ALIGN + round_up((size_t)n_groups * 4u));
    a.want_minimax = 0;
    a.want_pooled = 1;
    return hip_status(cqk::launch_sweep(a, E, n_groups, st));
}

int32_t cq_baseline_scales_spec(const float* w, const float* d, int32_t group_len, int32_t qmin, int32_t qmax,
                                int64_t d_period, int32_t E, int64_t n_groups, int32_t which, uint16_t* scales,
                                int8_t* codes, double* objective, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!spec_ok(group_len, qmin, qmax)) return CQ_EINVAL;
    if (group_len == CQ_GROUP && qmin == -8 && qmax == 7)
        return cq_baseline_scales(w, d, d_period, E, n_groups, which, scales, codes, objective, workspace,
                                  workspace_bytes, stream);
    hipStream_t st = (hipStream_t)stream;
    if (n_groups < 0 || n_groups > INT32_MAX) return CQ_EINVAL;
    if (which == CQ_ABSMAX) {
        if (qmax < 1) return CQ_EINVAL;  // the largest magnitude maps to the largest positive code
        if (n_groups == 0) return CQ_OK;
        if (!w || !scales || !aligned(w, 4)) return CQ_EINVAL;
        if (objective && !groups_ok(w, d, d_period, E, n_groups, 4)) return CQ_EINVAL;
        return hip_status(cqk::launch_absmax_spec(w, d, d_period, group_len, qmin, qmax, E, n_groups, scales, codes,
                                                  objective, st));
    }
    if (which != CQ_POOLED_WMSE) return CQ_EINVAL;
    if (!groups_ok(w, d, d_period, E, n_groups, 4)) return CQ_EINVAL;
    if (n_groups == 0) return CQ_OK;
    if (!scales) return CQ_EINVAL;
    if (!workspace || workspace_bytes < cq_workspace_size(CQ_EXHAUSTIVE, E, n_groups) || !aligned(workspace, ALIGN))
        return CQ_EWORKSPACE;
    // the full grid's pooled policy alone; its codes are those of the pooled scale
    return run_fullgrid(w, d, group_len, qmin, qmax, d_period, E, n_groups, nullptr, codes, nullptr, nullptr, scales,
                        objective, 0, (uint8_t*)workspace, st);
}

int32_t cq_pack_gptq_v1(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                        int32_t* qweight, uint16_t* scales, void* stream) {
    if (out < 0 || in < 0 || in % CQ_GROUP != 0) return CQ_EINVAL;
    if (out == 0 || in == 0) return CQ_OK;
    if (!codes || !grp_scales || !qweight || !scales) return CQ_EINVAL;
    if (!aligned(codes, 16) || !aligned(grp_scales, 2) || !aligned(qweight, 4) || !aligned(scales, 2))
        return CQ_EINVAL;
    if (in / CQ_GROUP > 65535 || (out + 63) / 64 > INT32_MAX) return CQ_EINVAL;
    return hip_status(cqk::launch_pack(codes, grp_scales, out, in, qweight, scales, (hipStream_t)stream));
}

int32_t cq_pack_gptq_v1_spec(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in, int32_t bits,
                             int32_t group_len, int32_t* qweight, uint16_t* scales, void* stream) {
    if (bits != 2 && bits != 4 && bits != 8) return CQ_EINVAL;
    if (group_len < 1 || group_len > CQ_MAX_GROUP) return CQ_EINVAL;
    if (out < 0 || in < 0 || in % group_len != 0 || in % (32 / bits) != 0) return CQ_EINVAL;
    if (out == 0 || in == 0) return CQ_OK;
    if (!codes || !grp_scales || !qweight || !scales) return CQ_EINVAL;
    if (!aligned(codes, 4) || !aligned(grp_scales, 2) || !aligned(qweight, 4) || !aligned(scales, 2))
        return CQ_EINVAL;
    if ((in + 127) / 128 > 65535 || (out + 63) / 64 > INT32_MAX || (in / group_len) > INT64_MAX / (out + 1) ||
        ((in / group_len) * out + 255) / 256 > INT32_MAX)
        return CQ_EINVAL;
    return hip_status(cqk::launch_pack_spec(codes, grp_scales, out, in, bits, group_len, qweight, scales,
                                            (hipStream_t)stream));
}

int32_t cq_pack_gptq_v1_multi(const int8_t* codes, const uint16_t* grp_scales, int32_t n_mats, const int64_t* outs,
                              const int64_t* ins, int32_t* qweight, uint16_t* scales, void* stream) {
    if (n_mats < 0 || n_mats > CQ_MAX_PACK_MATRICES) return CQ_EINVAL;
    if (n_mats == 0) return CQ_OK;
    if (!outs || !ins) return CQ_EINVAL;
    cqk::PackShapes m{};
    m.n = n_mats;
    int64_t elems = 0, tiles = 0;
    for (int32_t k = 0; k < n_mats; ++k) {
        const int64_t o = outs[k], i = ins[k];
        if (o < 0 || i < 0 || i % CQ_GROUP != 0 || o > INT32_MAX || i > INT32_MAX) return CQ_EINVAL;
        if (i / CQ_GROUP > 65535) return CQ_EINVAL;
        m.out[k] = (int32_t)o;
        m.in[k] = (int32_t)i;
        elems += o * i;
        tiles += (o + 63) / 64 * (i / CQ_GROUP);
        if (elems > ((int64_t)1 << 46)) return CQ_EINVAL;
    }
    if (tiles == 0) return CQ_OK;
    if (!codes || !grp_scales || !qweight || !scales) return CQ_EINVAL;
    if (!aligned(codes, 16) || !aligned(grp_scales, 2) || !aligned(qweight, 4) || !aligned(scales, 2))
        return CQ_EINVAL;
    return hip_status(cqk::launch_pack_multi(codes, grp_scales, m, qweight, scales, (hipStream_t)stream));
}

size_t cq_proxy_workspace_size(int64_t n_groups) {
    return n_groups < 0 ? 0 : round_up((size_t)n_groups * 8u);
}

int32_t cq_proxy_worst_env_wmse_multi(const float* w, const float* d_eval, int64_t d_period, int32_t E,
                                      int64_t n_groups, int32_t n_policies, const uint16_t* scales,
                                      const int64_t* module_offsets, int32_t n_modules, double* module_mean,
                                      double* macro, double* per_group, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (!groups_ok(w, d_eval, d_period, E, n_groups)) return CQ_EINVAL;
    if (n_policies < 1 || n_policies > CQ_MAX_POLICIES) return CQ_EINVAL;
    if (n_modules < 1 || !module_offsets || !module_mean || !macro) return CQ_EINVAL;
    if (n_groups > 0 && !scales) return CQ_EINVAL;
    if ((n_groups + 15) / 16 > INT32_MAX || n_groups > INT64_MAX / 8 / n_policies) return CQ_EINVAL;
    if (!per_group) {
        if (!workspace || workspace_bytes < cq_proxy_workspace_size(n_groups * n_policies) ||
            !aligned(workspace, ALIGN))
            return CQ_EWORKSPACE;
        per_group = (double*)workspace;
    } else if (!aligned(per_group, 8)) {
        return CQ_EINVAL;
    }
    return hip_status(cqk::launch_proxy(w, d_eval, d_period, E, n_groups, n_policies, scales, module_offsets,
                                        n_modules, module_mean, macro, per_group, (hipStream_t)stream));
}

int32_t cq_proxy_worst_env_wmse_multi_spec(const float* w, const float* d_eval, int32_t group_len, int32_t qmin,
                                           int32_t qmax, int64_t d_period, int32_t E, int64_t n_groups,
                                           int32_t n_policies, const uint16_t* scales, const int64_t* module_offsets,
                                           int32_t n_modules, double* module_mean, double* macro, double* per_group,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!spec_ok(group_len, qmin, qmax)) return CQ_EINVAL;
    if (group_len == CQ_GROUP && qmin == -8 && qmax == 7)
        return cq_proxy_worst_env_wmse_multi(w, d_eval, d_period, E, n_groups, n_policies, scales, module_offsets,
                                             n_modules, module_mean, macro, per_group, workspace, workspace_bytes,
                                             stream);
    if (!groups_ok(w, d_eval, d_period, E, n_groups, 4)) return CQ_EINVAL;
    if (n_policies < 1 || n_policies > CQ_MAX_POLICIES) return CQ_EINVAL;
    if (n_modules < 1 || !module_offsets || !module_mean || !macro) return CQ_EINVAL;
    if (n_groups > 0 && !scales) return CQ_EINVAL;
    if ((n_groups + 15) / 16 > INT32_MAX || n_groups > INT64_MAX / 8 / n_policies) return CQ_EINVAL;
    if (!per_group) {
        if (!workspace || workspace_bytes < cq_proxy_workspace_size(n_groups * n_policies) ||
            !aligned(workspace, ALIGN))
            return CQ_EWORKSPACE;
        per_group = (double*)workspace;
    } else if (!aligned(per_group, 8)) {
        return CQ_EINVAL;
    }
    return hip_status(cqk::launch_proxy_spec(w, d_eval, d_period, group_len, qmin, qmax, E, n_groups, n_policies,
                                             scales, module_offsets, n_modules, module_mean, macro, per_group,
                                             (hipStream_t)stream));
}

int32_t cq_proxy_worst_env_wmse(const float* w, const float* d_eval, int64_t d_period, int32_t E, int64_t n_groups,
                                const uint16_t* scales, const int64_t* module_offsets, int32_t n_modules,
                                double* module_mean, double* macro, double* per_group, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return cq_proxy_worst_env_wmse_multi(w, d_eval, d_period, E, n_groups, 1, scales, module_offsets, n_modules,
                                         module_mean, macro, per_group, workspace, workspace_bytes, stream);
}

int32_t cq_w4a16_matmul(const uint16_t* x, const int32_t* qweight, const uint16_t* scales, int64_t M, int64_t out,
                        int64_t in, float* y, void* stream) {
    if (M < 0 || out < 0 || in < 0 || in % CQ_GROUP != 0) return CQ_EINVAL;
    if (M == 0 || out == 0) return CQ_OK;
    if (in == 0) return CQ_EINVAL;
    if ((M + 63) / 64 > 65535 || (out + 63) / 64 > INT32_MAX) return CQ_EINVAL;
    if (!x || !qweight || !scales || !y) return CQ_EINVAL;
    if (!aligned(x, 16) || !aligned(qweight, 4) || !aligned(scales, 2) || !aligned(y, 4)) return CQ_EINVAL;
    return hip_status(cqk::launch_w4a16(x, qweight, scales, M, out, in, y, (hipStream_t)stream));
}

size_t cq_diagonals_workspace_size(int32_t E, int64_t T, int64_t in) {
    if (E < 1 || E > CQ_MAX_ENVS || T < 1 || in < CQ_GROUP || in % CQ_GROUP != 0 || in > (int64_t)1 << 24) return 0;
    return round_up((size_t)E * (size_t)cqk::diag_chunks(E, T, in) * (size_t)in * 8u) + round_up((size_t)E * (size_t)in * 8u);
}

int32_t cq_environment_diagonals(const uint16_t* x, int32_t E, int64_t T, int64_t in, float* d, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    if (E < 1 || E > CQ_MAX_ENVS || T < 1 || in < CQ_GROUP || in % CQ_GROUP != 0 || in > (int64_t)1 << 24)
        return CQ_EINVAL;
    if (!x || !d || !aligned(x, 16) || !aligned(d, 4)) return CQ_EINVAL;
    const size_t need = cq_diagonals_workspace_size(E, T, in);
    if (!workspace || workspace_bytes < need || !aligned(workspace, ALIGN)) return CQ_EWORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    double* part = (double*)ws;
    double* msq = (double*)(ws + round_up((size_t)E * (size_t)cqk::diag_chunks(E, T, in) * (size_t)in * 8u));
    return hip_status(cqk::launch_diagonals(x, E, T, in, d, part, msq, (hipStream_t)stream));
}

size_t cq_heldout_workspace_size(int32_t n_boot, int32_t n_modules) {
    if (n_boot < 0 || n_modules < 1) return 0;
    return round_up((size_t)(n_boot + 1) * (size_t)n_modules * 8u) + round_up((size_t)n_boot * 8u) +
           round_up((size_t)n_boot * 4u);
}

int32_t cq_heldout_compare(const double* pa, const double* pb, int64_t n_groups, const int64_t* module_offsets,
                           int32_t n_modules, const int32_t* boot_idx, int32_t n_boot, double alpha,
                           int64_t* counts, double* effect, double* boot, double* ci, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (n_groups < 0 || n_modules < 1 || n_boot < 0 || n_boot > CQ_MAX_BOOT) return CQ_EINVAL;
    if (!(alpha > 0.0 && alpha < 1.0)) return CQ_EINVAL;
    if (n_groups > 0 && (!pa || !pb || !aligned(pa, 8) || !aligned(pb, 8))) return CQ_EINVAL;
    if (!module_offsets || !aligned(module_offsets, 8) || !counts || !effect || !ci) return CQ_EINVAL;
    if (n_boot > 0 && (!boot_idx || !boot || !aligned(boot_idx, 4))) return CQ_EINVAL;
    if ((int64_t)(n_boot + 1) * n_modules > INT32_MAX) return CQ_EINVAL;
    if (!workspace || workspace_bytes < cq_heldout_workspace_size(n_boot, n_modules) || !aligned(workspace, ALIGN))
        return CQ_EWORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    double* mm = (double*)ws;
    double* reps = (double*)(ws + round_up((size_t)(n_boot + 1) * (size_t)n_modules * 8u));
    int32_t* rank = (int32_t*)((uint8_t*)reps + round_up((size_t)n_boot * 8u));
    return hip_status(cqk::launch_heldout(pa, pb, n_groups, module_offsets, n_modules, boot_idx, n_boot, alpha,
                                          counts, effect, boot, ci, mm, reps, rank, (hipStream_t)stream));
}

int32_t cq_probe_valu_fma(int32_t iters, int32_t blocks, int32_t mode, float* out, uint64_t* clocks,
                          double* wall_clock_hz, void* stream) {
    if (iters < 1 || blocks < 1 || (mode < 0 || mode > 2) || !out || !clocks || !wall_clock_hz) return CQ_EINVAL;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CQ_EHIP;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return CQ_EHIP;
    *wall_clock_hz = 1e3 * (double)khz;
    return hip_status(cqk::launch_fma_probe(iters, blocks, mode, out, clocks, (hipStream_t)stream));
}

}  // extern "C"
