// AbsMax baseline scale policy for gfx950.
//
// The matched baseline checkpoint of the pages uses AbsMax scales
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Measured result" and
// "Held-out reconstruction proxy"); the pages do not print its formula.  Read
// as s = binary16(round-to-nearest-even(fl32(max_i |w_i| / 7))), a result of
// 0 becoming the smallest positive scale and an overflow the largest finite.
// One 128-thread workgroup per group: a max-reduce, one division, the
// conversion, the codes, and (optionally) the worst-environment objective at
// that scale in binary64.  For the objective every thread forms its weight's
// terms d_e (w - s q)^2 for all environments into LDS (the same operations as
// the sequential definition), then one thread per environment adds them in
// index order, so the value is the definition's bit for bit.
#include "device.h"
#include "launch.h"

namespace cqk {

__global__ __launch_bounds__(128) void absmax_kernel(const float* __restrict__ w, const float* __restrict__ d,
                                                     int64_t d_period, int E, int64_t group_offset,
                                                     uint16_t* scales, int8_t* codes, double* objective) {
    extern __shared__ double terms[];  // [E][G] when the objective is wanted
    __shared__ float red[2];
    __shared__ double fe[32];
    const int64_t g = (int64_t)blockIdx.x + group_offset;
    const int tid = threadIdx.x;
    const float v = w[g * G + tid];
    float m = wave_max_f(fabsf(v));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(red[0], red[1]);
    uint32_t b = f32_to_half_bits_rne(m / 7.0f);
    if (b == 0u) b = BITS_FIRST;
    if (b > BITS_LAST) b = BITS_LAST;
    const float s = half_bits_value(b);
    if (codes) codes[g * G + tid] = (int8_t)exact_code(v, s);
    if (tid == 0) scales[g] = (uint16_t)b;
    if (objective) {
        const float* dg = d + (g % d_period) * (int64_t)(E * G);
        const double s64 = (double)s, inv = 1.0 / s64;
        // the operations of env_error_f64 for this thread's weight
        const double wi = (double)v;
        double r = __builtin_rint(wi * inv);
        r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
        const double sq = s64 * r;
        const double t = wi - sq;
        const double t2 = t * t;
        for (int e = 0; e < E; ++e) terms[e * G + tid] = (double)dg[e * G + tid] * t2;
        __syncthreads();
        if (tid < E) {
            double F = 0.0;
#pragma unroll 8
            for (int i = 0; i < G; ++i) F = F + terms[tid * G + i];
            fe[tid] = F;
        }
        __syncthreads();
        if (tid == 0) {
            double F = fe[0];
            for (int e = 1; e < E; ++e) F = fe[e] > F ? fe[e] : F;
            objective[g] = F;
        }
    }
}

hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st) {
    const int64_t step = 1ll << 30;
    for (int64_t off = 0; off < n_groups; off += step) {
        const int64_t n = n_groups - off < step ? n_groups - off : step;
        const size_t lds = objective ? (size_t)E * G * sizeof(double) : 0;
        hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)n), dim3(128), lds, st, w, d, d_period, E, off,
                           scales, codes, objective);
    }
    return hipGetLastError();
}

}  // namespace cqk
