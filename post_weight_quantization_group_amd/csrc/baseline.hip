// AbsMax baseline scale policy for gfx950.
//
// The matched baseline checkpoint of the pages uses AbsMax scales
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Measured result" and
// "Held-out reconstruction proxy"); the pages do not print its formula.  Read
// as s = binary16(round-to-nearest-even(fl32(max_i |w_i| / 7))), a result of
// 0 becoming the smallest positive scale and an overflow the largest finite.
// Without the objective, one 128-thread workgroup per group: a max-reduce,
// one division, the conversion and the codes.  With it, one thread per
// (group, environment): the thread loads its group's weights into registers
// (all loads in flight at once), forms the same scale, and adds its
// environment's terms d_e (w - s q)^2 for i = 0..127 in index order with every
// operation rounded on its own, so each environment's sum is the sequential
// binary64 definition bit for bit; the group's E threads share the codes (each
// a contiguous share), environment 0's thread writes the scale, and the
// maximum over environments goes through LDS.  When E is a power of two up to
// 32 a group's threads are adjacent lanes of one wave and also share the
// binary64 codes and squared residuals (absmax_shared_kernel).
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
    // the product is finite (no NaN), so max/min clip exactly as the comparisons do
    const double r = __builtin_fmin(__builtin_fmax(__builtin_rint(wi * inv), -8.0), 7.0);
    const double sq = s * r;
    const double t = wi - sq;
    const double t2 = t * t;
    return (double)df * t2;
}
__device__ __forceinline__ uint32_t code_byte(float wv, float s) {
    return (uint32_t)(uint8_t)(int8_t)exact_code(wv, s);
}

// blockDim.x = 256; the workgroup holds gpb = 256 / E groups, thread c = (c / E, c % E).  A thread
// holds its group's 128 weights in registers (every load in flight at once), forms the scale, then
// loads its environment's diagonals in two halves and adds the terms in index order.
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
        float4 wv[G / 4];
#pragma unroll
        for (int k = 0; k < G / 4; ++k) wv[k] = wr[k];
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < G / 4; ++k) m = fmaxf(m, abs_max4(wv[k]));
        const uint32_t b = absmax_bits(m);
        const float s = half_bits_value(b);
        const double s64 = (double)s, inv = 1.0 / s64;
        const float4* dr = (const float4*)(d + (g % d_period) * (int64_t)(E * G) + (int64_t)e * G);
        double F = 0.0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float4 dv[G / 8];
#pragma unroll
            for (int k = 0; k < G / 8; ++k) dv[k] = dr[h * (G / 8) + k];
#pragma unroll
            for (int k = 0; k < G / 8; ++k) {
                const float4 v = wv[h * (G / 8) + k];
                F = F + absmax_term(v.x, dv[k].x, s64, inv);
                F = F + absmax_term(v.y, dv[k].y, s64, inv);
                F = F + absmax_term(v.z, dv[k].z, s64, inv);
                F = F + absmax_term(v.w, dv[k].w, s64, inv);
            }
        }
        fe[c] = F;
        if (e == 0) scales[g] = (uint16_t)b;
        if (codes) {
            // the group's E threads share its codes: thread e takes weights [e per, (e + 1) per)
            const int per = (G + E - 1) / E, i0 = e * per, i1 = i0 + per < G ? i0 + per : G;
            if (per % 4 == 0 && G % E == 0) {
                // four codes per 16-byte load and 4-byte store
                const float4* wg = (const float4*)(w + g * G);
                uint32_t* cg = (uint32_t*)(codes + g * G);
#pragma unroll 8
                for (int j = i0 / 4; j < i1 / 4; ++j) {
                    const float4 v = wg[j];
                    cg[j] = code_byte(v.x, s) | (code_byte(v.y, s) << 8) | (code_byte(v.z, s) << 16) |
                            (code_byte(v.w, s) << 24);
                }
            } else {
                const float* wg = w + g * G;
                int8_t* cg = codes + g * G;
#pragma unroll 8
                for (int i = i0; i < i1; ++i) cg[i] = (int8_t)exact_code(wg[i], s);
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

// Another quantizer (group length G <= 256, codes in [qmin, qmax] with qmax >= 1): the scale
// fp16(fl32(max|w| / qmax)), 0 -> 0x0001, overflow -> 0x7BFF (the largest magnitude maps to the
// largest positive code, as max|w| / 7 does for [-8, 7]).  One thread per (group, environment) as
// above, the weights read in index order; the codes shared by the group's threads; with the
// objective, each environment's sum i = 0..G-1 with every operation rounded on its own.
__global__ __launch_bounds__(256) void absmax_spec_kernel(const float* __restrict__ w, const float* __restrict__ d,
                                                          int64_t d_period, int G, int qmin, int qmax, int E, int gpb,
                                                          int64_t n_groups, uint16_t* scales, int8_t* codes,
                                                          double* objective) {
    __shared__ double fe[256];
    const int c = threadIdx.x;
    const int gl = c / E, e = c - gl * E;
    const int64_t g = (int64_t)blockIdx.x * gpb + gl;
    const bool live = gl < gpb && g < n_groups;
    if (live) {
        const float* wg = w + g * G;
        float m = 0.0f;
        for (int i = 0; i < G; ++i) m = fmaxf(m, fabsf(wg[i]));
        uint32_t b = f32_to_half_bits_rne(m / (float)qmax);
        if (b == 0u) b = BITS_FIRST;
        if (b > BITS_LAST) b = BITS_LAST;
        const float s = half_bits_value(b);
        if (e == 0) scales[g] = (uint16_t)b;
        if (codes) {
            const int per = (G + E - 1) / E, i0 = e * per, i1 = i0 + per < G ? i0 + per : G;
            for (int i = i0; i < i1; ++i)
                codes[g * G + i] = (int8_t)exact_code_range(wg[i], s, (float)qmin, (float)qmax);
        }
        if (objective) {
            const double s64 = (double)s;
            fe[c] = env_error_f64_n(wg, d + (g % d_period) * (int64_t)(E * G) + (int64_t)e * G, 1, G, s64,
                                    1.0 / s64, (double)qmin, (double)qmax);
        }
    }
    __syncthreads();
    if (objective && live && e == 0) {
        double F = fe[c];
        for (int k = 1; k < E; ++k) F = fe[c + k] > F ? fe[c + k] : F;
        objective[g] = F;
    }
}

hipError_t launch_absmax_spec(const float* w, const float* d, int64_t d_period, int G, int qmin, int qmax, int E,
                              int64_t n_groups, uint16_t* scales, int8_t* codes, double* objective, hipStream_t st) {
    const int Eu = objective ? E : 1;  // without the objective one thread per group
    const int gpb = BLOCK / Eu;
    const int64_t blocks = (n_groups + gpb - 1) / gpb;
    hipLaunchKernelGGL(absmax_spec_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, st, w, d, d_period, G, qmin, qmax,
                       Eu, gpb, n_groups, scales, codes, objective);
    return hipGetLastError();
}

// The value of lane j of this lane's group of E adjacent lanes (E a power of two up to 32): a DPP
// move within the quad for E <= 4, a lane shuffle beyond.
template <int E>
__device__ __forceinline__ uint32_t group_lane(uint32_t v, int j) {
    if constexpr (E == 4) {
        switch (j) {  // quad_perm [j, j, j, j]
            case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
            case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
            case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
            default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
        }
    } else if constexpr (E == 2) {  // quad_perm [j, j, 2 + j, 2 + j]
        return (uint32_t)(j == 0 ? __builtin_amdgcn_mov_dpp((int)v, 0xA0, 0xF, 0xF, false)
                                 : __builtin_amdgcn_mov_dpp((int)v, 0xF5, 0xF, 0xF, false));
    } else {
        const int lane = threadIdx.x & 63;
        return (uint32_t)__shfl((int)v, (lane & ~(E - 1)) + j, 64);
    }
}
template <int E>
__device__ __forceinline__ double group_lane(double v, int j) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = group_lane<E>((uint32_t)u, j), hi = group_lane<E>((uint32_t)(u >> 32), j);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// E a power of two from 2 to 32: a group's E threads are adjacent lanes of one wave, so they share
// the codes and squared residuals.  Lane e forms them for the weights i = E k + e and the group's
// lanes pass them round, so that each environment's thread adds the 128 terms d_e (w - s q)^2 in
// index order from the same values with the same operations as above (the same sums bit for bit),
// with 1/E of the binary64 code work per thread.  Lanes of a group past n_groups read group 0 and
// write nothing, so that every lane takes part in the exchanges.
template <int E>
__global__ __launch_bounds__(256) void absmax_shared_kernel(const float* __restrict__ w, const float* __restrict__ d,
                                                            int64_t d_period, int64_t n_groups, uint16_t* scales,
                                                            int8_t* codes, double* objective) {
    constexpr int GPB = BLOCK / E, K = G / E;
    __shared__ double fe[BLOCK];
    const int c = threadIdx.x, e = c & (E - 1);
    const int64_t g = (int64_t)blockIdx.x * GPB + c / E;
    const bool live = g < n_groups;
    const int64_t gs = live ? g : 0;
    const float* wg = w + gs * G;
    float wq[K];  // weights E k + e
#pragma unroll
    for (int k = 0; k < K; ++k) wq[k] = wg[E * k + e];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) m = fmaxf(m, fabsf(wq[k]));
#pragma unroll
    for (int o = 1; o < E; o <<= 1) m = fmaxf(m, lane_xor(m, o));
    const uint32_t b = absmax_bits(m);
    const float s = half_bits_value(b);
    if (live && e == 0) scales[g] = (uint16_t)b;
    if (live && codes)
#pragma unroll
        for (int k = 0; k < K; ++k) codes[g * G + E * k + e] = (int8_t)exact_code(wq[k], s);
    const double s64 = (double)s, inv = 1.0 / s64;
    const float4* dr = (const float4*)(d + (gs % d_period) * (int64_t)(E * G) + (int64_t)e * G);
    double F = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float dl[G / 2];
#pragma unroll
        for (int q = 0; q < G / 8; ++q) {
            const float4 v = dr[h * (G / 8) + q];
            dl[4 * q] = v.x; dl[4 * q + 1] = v.y; dl[4 * q + 2] = v.z; dl[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int k = h * (K / 2); k < (h + 1) * (K / 2); ++k) {
            // the operations of env_error_f64 for weight E k + e, then the group's E of them in order
            const double wi = (double)wq[k];
            const double r = __builtin_fmin(__builtin_fmax(__builtin_rint(wi * inv), -8.0), 7.0);
            const double sq = s64 * r;
            const double t = wi - sq;
            const double t2 = t * t;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const double term = (double)dl[E * k + j - h * (G / 2)] * group_lane<E>(t2, j);
                F = F + term;
            }
        }
    }
    fe[c] = F;
    __syncthreads();
    if (live && e == 0) {
        double Fm = fe[c];
#pragma unroll
        for (int k = 1; k < E; ++k) Fm = fe[c + k] > Fm ? fe[c + k] : Fm;
        objective[g] = Fm;
    }
}

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st) {
    if (objective && (E & (E - 1)) == 0 && E >= 2 && E <= 32) {
        const int64_t blocks = (n_groups + BLOCK / E - 1) / (BLOCK / E);
        const dim3 grid((unsigned)blocks), block(BLOCK);
        switch (E) {
            case 2: hipLaunchKernelGGL(absmax_shared_kernel<2>, grid, block, 0, st, w, d, d_period, n_groups, scales, codes,
                                       objective); break;
            case 4: hipLaunchKernelGGL(absmax_shared_kernel<4>, grid, block, 0, st, w, d, d_period, n_groups, scales, codes,
                                       objective); break;
            case 8: hipLaunchKernelGGL(absmax_shared_kernel<8>, grid, block, 0, st, w, d, d_period, n_groups, scales, codes,
                                       objective); break;
            case 16: hipLaunchKernelGGL(absmax_shared_kernel<16>, grid, block, 0, st, w, d, d_period, n_groups, scales,
                                        codes, objective); break;
            default: hipLaunchKernelGGL(absmax_shared_kernel<32>, grid, block, 0, st, w, d, d_period, n_groups, scales,
                                        codes, objective); break;
        }
        return hipGetLastError();
    }
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
