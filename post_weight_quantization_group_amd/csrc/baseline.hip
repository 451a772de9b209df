// AbsMax baseline scale policy for gfx950.
//
// The matched baseline checkpoint of the pages uses AbsMax scales
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Measured result" and
// "Held-out reconstruction proxy"); the pages do not print its formula.  Read
// as s = binary16(round-to-nearest-even(fl32(max_i |w_i| / 7))), a result of
// 0 becoming the smallest positive scale and an overflow the largest finite.
// Without the objective, one 128-thread workgroup per group: a max-reduce,
// one division, the conversion and the codes.  With it, a 256-thread
// workgroup takes GB = max(1, 16 / E) consecutive groups: their weights and
// diagonal slices go to LDS in coalesced 16-byte loads, one wave per group
// forms max|w| and the scale, all threads form the terms d_e (w - s q)^2 of
// every (group, environment, weight) in LDS with every operation rounded on
// its own, and one lane per (group, environment) adds its 128 terms in index
// order, so each environment's sum is the sequential binary64 definition bit
// for bit; the maximum over environments follows in LDS.
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

// Groups per workgroup of the objective kernel: GB * E <= 16 sums (E <= 16), else one group.
__host__ __device__ constexpr int absmax_gb(int E) { return E >= 16 ? 1 : 16 / E; }
// Dynamic LDS of the objective kernel: weights [GB][G], diagonals [GB][E][G] (binary32), terms
// [GB * E][G + 1] (binary64; rows padded by one so that the summing lanes read distinct banks),
// then the scales' patterns, reciprocals and per-environment sums.
__host__ __device__ constexpr size_t absmax_lds(int E) {
    return (size_t)absmax_gb(E) * G * 4 + (size_t)absmax_gb(E) * E * G * 4 +
           (size_t)absmax_gb(E) * E * (G + 1) * 8 + (size_t)absmax_gb(E) * 16 + (size_t)absmax_gb(E) * E * 8;
}

__global__ __launch_bounds__(256) void absmax_objective_kernel(const float* __restrict__ w,
                                                               const float* __restrict__ d, int64_t d_period,
                                                               int E, int64_t group_offset, int64_t n_groups,
                                                               uint16_t* scales, int8_t* codes, double* objective) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int GB = absmax_gb(E);
    float* sw = (float*)lds;                                    // [GB][G]
    float* sd = sw + GB * G;                                    // [GB][E][G]
    double* st = (double*)(sd + GB * E * G);                    // [GB * E][G + 1]
    double* sinv = st + GB * E * (G + 1);                       // [GB]
    double* sfe = sinv + GB;                                    // [GB * E]
    uint32_t* sb = (uint32_t*)(sfe + GB * E);                   // [GB]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t g0 = group_offset + (int64_t)blockIdx.x * GB;
    const int ng = (int)(n_groups - g0 < GB ? n_groups - g0 : GB);

    // ---- staging: the groups' weights (contiguous) and each group's diagonal slice
    for (int j = tid; j < ng * (G / 4); j += BLOCK)
        ((float4*)sw)[j] = ((const float4*)(w + g0 * G))[j];
    for (int j = tid; j < ng * E * (G / 4); j += BLOCK) {
        const int gl = j / (E * (G / 4)), r = j - gl * (E * (G / 4));
        ((float4*)sd)[j] = ((const float4*)(d + ((g0 + gl) % d_period) * (int64_t)(E * G)))[r];
    }
    __syncthreads();

    // ---- max|w| and the scale, one wave per group
    for (int gl = wave; gl < ng; gl += BLOCK / 64) {
        const float m = wave_max_f(fmaxf(fabsf(sw[gl * G + lane]), fabsf(sw[gl * G + lane + 64])));
        if (lane == 0) {
            const uint32_t b = absmax_bits(m);
            sb[gl] = b;
            sinv[gl] = 1.0 / (double)half_bits_value(b);
        }
    }
    __syncthreads();

    // ---- every term, and the codes (four weights per thread, one 32-bit store)
    for (int j = tid; j < ng * E * G; j += BLOCK) {
        const int row = j / G, i = j - row * G, gl = row / E;
        const double s64 = (double)half_bits_value(sb[gl]);
        st[row * (G + 1) + i] = absmax_term(sw[gl * G + i], sd[row * G + i], s64, sinv[gl]);
    }
    if (codes) {
        for (int j = tid; j < ng * (G / 4); j += BLOCK) {
            const int gl = j / (G / 4);
            const float s = half_bits_value(sb[gl]);
            const float4 v = ((const float4*)sw)[j];
            ((uint32_t*)(codes + g0 * G))[j] = code_byte(v.x, s) | (code_byte(v.y, s) << 8) |
                                               (code_byte(v.z, s) << 16) | (code_byte(v.w, s) << 24);
        }
    }
    __syncthreads();

    // ---- each environment's sum in index order, then the maximum over environments
    if (tid < ng * E) {
        const double* tr = st + tid * (G + 1);
        double F = 0.0;
#pragma unroll 16
        for (int i = 0; i < G; ++i) F = F + tr[i];
        sfe[tid] = F;
    }
    __syncthreads();
    if (tid < ng) {
        double F = sfe[tid * E];
        for (int k = 1; k < E; ++k) F = sfe[tid * E + k] > F ? sfe[tid * E + k] : F;
        objective[g0 + tid] = F;
        scales[g0 + tid] = (uint16_t)sb[tid];
    }
}

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st) {
    if (objective) {
        const int gb = absmax_gb(E);
        const int64_t blocks = (n_groups + gb - 1) / gb;
        const int64_t step = 1ll << 30;  // grid.x is limited to 2^31 - 1 blocks
        for (int64_t off = 0; off < blocks; off += step) {
            const int64_t nb = blocks - off < step ? blocks - off : step;
            hipLaunchKernelGGL(absmax_objective_kernel, dim3((unsigned)nb), dim3(BLOCK), absmax_lds(E), st, w, d,
                               d_period, E, off * gb, n_groups, scales, codes, objective);
        }
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
