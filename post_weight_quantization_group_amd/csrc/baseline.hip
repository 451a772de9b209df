// AbsMax baseline scale policy for gfx950.
//
// The matched baseline checkpoint of the pages uses AbsMax scales
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Measured result" and
// "Held-out reconstruction proxy"); the pages do not print its formula.  Read
// as s = binary16(round-to-nearest-even(fl32(max_i |w_i| / 7))), a result of
// 0 becoming the smallest positive scale and an overflow the largest finite.
// Without the objective, one 128-thread workgroup per group: a max-reduce,
// one division, the conversion and the codes.  With it, one thread per
// (group, environment): the thread reads its group's weights, forms the same
// scale, and adds its environment's terms d_e (w - s q)^2 for i = 0..127 in
// index order with every operation rounded on its own, so each environment's
// sum is the sequential binary64 definition bit for bit; environment 0's
// thread writes the codes and the scale, and the maximum over environments
// goes through LDS.
#include "device.h"
#include "launch.h"

namespace cqk {

__device__ __forceinline__ uint32_t absmax_bits(float m) {
    uint32_t b = f32_to_half_bits_rne(m / 7.0f);
    if (b == 0u) b = BITS_FIRST;
    if (b > BITS_LAST) b = BITS_LAST;
    return b;
}

__global__ __launch_bounds__(128) void absmax_kernel(const float* __restrict__ w, int64_t group_offset,
                                                     uint16_t* scales, int8_t* codes) {
    __shared__ float red[2];
    const int64_t g = (int64_t)blockIdx.x + group_offset;
    const int tid = threadIdx.x;
    const float v = w[g * G + tid];
    float m = wave_max_f(fabsf(v));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(red[0], red[1]);
    const uint32_t b = absmax_bits(m);
    if (codes) codes[g * G + tid] = (int8_t)exact_code(v, half_bits_value(b));
    if (tid == 0) scales[g] = (uint16_t)b;
}

__device__ __forceinline__ float abs_max4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}
__device__ __forceinline__ double absmax_term(float wf, float df, double s, double inv) {
    // the operations of env_error_f64 for one weight
    const double wi = (double)wf;
    double r = __builtin_rint(wi * inv);
    r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
    const double sq = s * r;
    const double t = wi - sq;
    const double t2 = t * t;
    return (double)df * t2;
}
__device__ __forceinline__ uint32_t code_byte(float wv, float s) {
    return (uint32_t)(uint8_t)(int8_t)exact_code(wv, s);
}

// blockDim.x = 256; the workgroup holds gpb = 256 / E groups, thread c = (c / E, c % E).
__global__ __launch_bounds__(256) void absmax_objective_kernel(const float* __restrict__ w,
                                                               const float* __restrict__ d, int64_t d_period,
                                                               int E, int gpb, int64_t n_groups,
                                                               uint16_t* scales, int8_t* codes,
                                                               double* objective) {
    __shared__ double fe[256];
    const int c = threadIdx.x;
    const int gl = c / E, e = c - gl * E;
    const int64_t g = (int64_t)blockIdx.x * gpb + gl;
    const bool live = gl < gpb && g < n_groups;
    if (live) {
        const float4* wr = (const float4*)(w + g * G);
        float m = 0.0f;
#pragma unroll 8
        for (int k = 0; k < G / 4; ++k) m = fmaxf(m, abs_max4(wr[k]));
        const uint32_t b = absmax_bits(m);
        const float s = half_bits_value(b);
        const double s64 = (double)s, inv = 1.0 / s64;
        const float4* dr = (const float4*)(d + (g % d_period) * (int64_t)(E * G) + (int64_t)e * G);
        double F = 0.0;
#pragma unroll 4
        for (int k = 0; k < G / 4; ++k) {
            const float4 v = wr[k], dv = dr[k];
            F = F + absmax_term(v.x, dv.x, s64, inv);
            F = F + absmax_term(v.y, dv.y, s64, inv);
            F = F + absmax_term(v.z, dv.z, s64, inv);
            F = F + absmax_term(v.w, dv.w, s64, inv);
        }
        fe[c] = F;
        if (e == 0) {
            scales[g] = (uint16_t)b;
            if (codes) {
                uint4* cr = (uint4*)(codes + g * G);
#pragma unroll 2
                for (int k = 0; k < G / 16; ++k) {
                    uint32_t q[4];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const float4 v = wr[4 * k + h];
                        q[h] = code_byte(v.x, s) | (code_byte(v.y, s) << 8) | (code_byte(v.z, s) << 16) |
                               (code_byte(v.w, s) << 24);
                    }
                    cr[k] = make_uint4(q[0], q[1], q[2], q[3]);
                }
            }
        }
    }
    __syncthreads();
    if (live && e == 0) {
        double F = fe[c];
        for (int k = 1; k < E; ++k) F = fe[c + k] > F ? fe[c + k] : F;
        objective[g] = F;
    }
}

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st) {
    if (objective) {
        const int gpb = BLOCK / E;
        const int64_t blocks = (n_groups + gpb - 1) / gpb;
        hipLaunchKernelGGL(absmax_objective_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, st, w, d, d_period, E,
                           gpb, n_groups, scales, codes, objective);
        return hipGetLastError();
    }
    const int64_t step = 1ll << 30;
    for (int64_t off = 0; off < n_groups; off += step) {
        const int64_t n = n_groups - off < step ? n_groups - off : step;
        hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)n), dim3(128), 0, st, w, off, scales, codes);
    }
    return hipGetLastError();
}

}  // namespace cqk
