// Device helpers shared by the gfx950 kernels of the scale-selection library.
//
// Definitions followed (CliffQuant repository README, "What CliffQuant
// changes"): the admissible scales are the positive finite IEEE binary16
// values, the code of a weight is its quotient by the scale rounded half to
// even and then clipped to [-8, 7], the objective is the worst environment's
// diagonal-weighted squared error, and an exact tie goes to the lower bit
// pattern.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cqk {

constexpr int G = 128;                  // weights per group
constexpr uint32_t BITS_FIRST = 0x0001u; // 2^-24
constexpr uint32_t BITS_LAST = 0x7BFFu;  // 65504
constexpr uint32_t N_SCALES = 31743u;
constexpr int BLOCK = 256;

// Kernels are instantiated for 1, 2, 4, 8, 16 and 32 environments; other counts run the
// next size up with zero diagonals, which add 0 to every sum and never win a maximum.
inline int pad_envs(int E) {
    int p = 1;
    while (p < E) p <<= 1;
    return p;
}

constexpr uint8_t FLAG_BAD_INPUT = 1u, FLAG_NEAR_TIE = 2u, FLAG_EXACT_TIE = 4u,
                  FLAG_FALLBACK = 8u, FLAG_FP64_SWEEP = 16u;

// Exact binary32 value of a positive binary16 bit pattern (no reliance on the
// device's half-precision denormal mode).
__device__ __forceinline__ float half_bits_value(uint32_t b) {
    const uint32_t ex = b >> 10, man = b & 0x3FFu;
    if (ex == 0u) return (float)man * 5.9604644775390625e-08f;  // man * 2^-24
    return __uint_as_float(((ex + 112u) << 23) | (man << 13));   // rebias 15 -> 127
}

// The code rule with the quotient as one correctly rounded binary32 division.
__device__ __forceinline__ float exact_code(float w, float s) {
    const float x = w / s;
    const float r = __builtin_rintf(x);
    return __builtin_amdgcn_fmed3f(r, -8.0f, 7.0f);
}

// Per-environment error of one group at one scale in binary64, summed
// i = 0..127 in order with every operation rounded on its own.  The code
// decision uses the binary64 product w * (1/s).  A binary32 weight that is not
// exactly (m + 1/2) s differs from that binary32 number by at least half a
// binary32 spacing, so its quotient sits at least a quarter binary32 ulp of
// m + 1/2 (about 2^-26 relative) away from the half-integer; the product's
// relative error (2^-52) cannot cross it.  Every decision therefore equals the
// exact one -- and the binary32-division one -- except at exact half-integers,
// where both neighbouring codes give the same |w - s q| = s/2.
__device__ __forceinline__ double env_error_f64(const float* w, const float* d, int dstride,
                                                double s, double inv) {
    double F = 0.0;
#pragma unroll 8
    for (int i = 0; i < G; ++i) {
        const double wi = (double)w[i];
        double r = __builtin_rint(wi * inv);
        r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
        const double sq = s * r;
        const double t = wi - sq;
        const double t2 = t * t;
        const double term = (double)d[i * dstride] * t2;
        F = F + term;
    }
    return F;
}

// env_error_f64 with the codes given: q[i] is the exact code of w[i] at s.  Same operations in the
// same order, so the same value.
__device__ __forceinline__ double env_error_codes_f64(const float* w, const float* d, int dstride,
                                                      const int8_t* q, double s) {
    double F = 0.0;
#pragma unroll 8
    for (int i = 0; i < G; ++i) {
        const double wi = (double)w[i];
        const double sq = s * (double)q[i];
        const double t = wi - sq;
        const double t2 = t * t;
        const double term = (double)d[i * dstride] * t2;
        F = F + term;
    }
    return F;
}

// The code rule for the code range [qlo, qhi] (a quantizer specification): one correctly rounded
// binary32 division, round half to even, clip.
__device__ __forceinline__ float exact_code_range(float w, float s, float qlo, float qhi) {
    const float x = w / s;
    const float r = __builtin_rintf(x);
    return __builtin_amdgcn_fmed3f(r, qlo, qhi);
}

// env_error_f64 for a group of n weights and the code range [qlo, qhi]: the same operations in
// the same order (i = 0..n-1), the code decided by the binary64 product as argued there (the
// argument does not depend on the size of the quotient).
__device__ __forceinline__ double env_error_f64_n(const float* w, const float* d, int dstride, int n,
                                                  double s, double inv, double qlo, double qhi) {
    double F = 0.0;
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
        const double wi = (double)w[i];
        double r = __builtin_rint(wi * inv);
        r = r < qlo ? qlo : (r > qhi ? qhi : r);
        const double sq = s * r;
        const double t = wi - sq;
        const double t2 = t * t;
        const double term = (double)d[i * dstride] * t2;
        F = F + term;
    }
    return F;
}

// binary32 x >= 0 to the nearest binary16 pattern, ties to even; 0x7C00 on overflow.
__device__ __forceinline__ uint32_t f32_to_half_bits_rne(float x) {
    if (!(x < 65520.0f)) return 0x7C00u;
    if (x < 0x1p-14f) {
        // subnormal range: the pattern is x / 2^-24 rounded half to even (1024 = smallest normal)
        return (uint32_t)__builtin_rintf(x * 16777216.0f);
    }
    const uint32_t u = __float_as_uint(x);
    const uint32_t ex = (u >> 23) - 127u + 15u;  // in 1..30
    const uint32_t man = u & 0x7FFFFFu;
    uint32_t r = man >> 13;
    const uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
    return (ex << 10) + r;  // a carry out of the fraction bumps the exponent, as it should
}

// ---------------------------------------------------------------- lane exchange
// The value of lane (lane ^ m) for m = 1, 2, 4, 8 through DPP moves (quad_perm [1,0,3,2] and
// [2,3,0,1]; half-row mirror, i.e. xor 7, then quad_perm [3,2,1,0], i.e. xor 3; row rotate by 8),
// with no LDS round trip; a lane shuffle for larger m.  m is a constant once the callers' loops
// are unrolled.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int m) {
    switch (m) {
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
        case 4: return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false),
                                                          0x1B, 0xF, 0xF, false);
        case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
        default: return (uint32_t)__shfl_xor((int)v, m, 64);
    }
}
__device__ __forceinline__ float lane_xor(float v, int m) { return __uint_as_float(lane_xor(__float_as_uint(v), m)); }
__device__ __forceinline__ uint64_t lane_xor(uint64_t v, int m) {
    const uint32_t lo = lane_xor((uint32_t)v, m), hi = lane_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double lane_xor(double v, int m) {
    return __builtin_bit_cast(double, lane_xor(__builtin_bit_cast(uint64_t, v), m));
}
// The value of lane (lane - 1), 0 in lane 0 (DPP wave shift right by one).
__device__ __forceinline__ uint32_t lane_prev(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, true);
}
__device__ __forceinline__ float lane_prev(float v) { return __uint_as_float(lane_prev(__float_as_uint(v))); }
__device__ __forceinline__ double lane_prev(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = ((uint64_t)lane_prev((uint32_t)(u >> 32)) << 32) | lane_prev((uint32_t)u);
    return __builtin_bit_cast(double, r);
}
// Inclusive prefix sum over the 64 lanes of a wave through DPP: row_shr 1, 2, 4, 8 within each
// row of 16 lanes (lanes with no source add 0), then row_bcast15 and row_bcast31 carry the
// totals of the earlier rows.
__device__ __forceinline__ float wave_inclusive_sum_f32(float x) {
#define CQ_SCAN_STEP32(ctrl, rmask) \
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xF, true));
    CQ_SCAN_STEP32(0x111, 0xF)
    CQ_SCAN_STEP32(0x112, 0xF)
    CQ_SCAN_STEP32(0x114, 0xF)
    CQ_SCAN_STEP32(0x118, 0xF)
    CQ_SCAN_STEP32(0x142, 0xA)
    CQ_SCAN_STEP32(0x143, 0xC)
#undef CQ_SCAN_STEP32
    return x;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t u = lane_xor(v, o);
        v = u < v ? u : v;
    }
    return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, lane_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, lane_xor(v, o));
    return v;
}

// Block-wide reductions for 256 threads; `red` is caller LDS of >= 4 slots.
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* red) {
    v = wave_min_u64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = red[0];
#pragma unroll
    for (int k = 1; k < BLOCK / 64; ++k) r = red[k] < r ? red[k] : r;
    return r;
}
__device__ __forceinline__ float block_max_f(float v, float* red) {
    v = wave_max_f(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < BLOCK / 64; ++k) r = fmaxf(r, red[k]);
    return r;
}
__device__ __forceinline__ float block_min_f(float v, float* red) {
    v = wave_min_f(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < BLOCK / 64; ++k) r = fminf(r, red[k]);
    return r;
}

// Block-wide maxima of N values at once, in one barrier round; `red` holds >= 4 * N slots.
template <int N>
__device__ __forceinline__ void block_max_fn(float (&v)[N], float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] = fmaxf(v[k], lane_xor(v[k], o));
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k) red[(threadIdx.x >> 6) * N + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float r = red[k];
#pragma unroll
        for (int w = 1; w < BLOCK / 64; ++w) r = fmaxf(r, red[w * N + k]);
        v[k] = r;
    }
}

// Block-wide minima of N 64-bit values at once, in one barrier round; `red` holds >= 4 * N slots.
template <int N>
__device__ __forceinline__ void block_min_u64n(uint64_t (&v)[N], uint64_t* red) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = wave_min_u64(v[k]);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k) red[(threadIdx.x >> 6) * N + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        uint64_t r = red[k];
#pragma unroll
        for (int w = 1; w < BLOCK / 64; ++w) r = red[w * N + k] < r ? red[w * N + k] : r;
        v[k] = r;
    }
}

// Key ordering (value, bit pattern) lexicographically for non-negative floats.
__device__ __forceinline__ uint64_t key_of(float v, uint32_t b) {
    return ((uint64_t)__float_as_uint(v) << 32) | (uint64_t)b;
}
__device__ __forceinline__ float key_value(uint64_t k) { return __uint_as_float((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_bits(uint64_t k) { return (uint32_t)(k & 0xFFFFFFFFu); }
constexpr uint64_t KEY_NONE = ~0ull;

}  // namespace cqk
