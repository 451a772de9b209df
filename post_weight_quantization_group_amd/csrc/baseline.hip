// AbsMax baseline scale policy for gfx950.
//
// The matched baseline checkpoint of the pages uses AbsMax scales
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Measured result" and
// "Held-out reconstruction proxy"); the pages do not print its formula.  Read
// as s = binary16(round-to-nearest-even(fl32(max_i |w_i| / 7))), a result of
// 0 becoming the smallest positive scale and an overflow the largest finite.
// One 128-thread workgroup per group: a max-reduce, one division, the
// conversion, the codes, and (optionally) the worst-environment objective at
// that scale in binary64.
#include "device.h"
#include "launch.h"

namespace cqk {

__global__ __launch_bounds__(128) void absmax_kernel(const float* __restrict__ w, const float* __restrict__ d,
                                                     int64_t d_period, int E, int64_t group_offset,
                                                     uint16_t* scales, int8_t* codes, double* objective) {
    __shared__ float sw[G];
    __shared__ float red[2];
    __shared__ double fe[32];
    const int64_t g = (int64_t)blockIdx.x + group_offset;
    const int tid = threadIdx.x;
    const float v = w[g * G + tid];
    sw[tid] = v;
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
        const double s64 = (double)s;
        if (tid < E) fe[tid] = env_error_f64(sw, dg + tid * G, 1, s64, 1.0 / s64);
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
        hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)n), dim3(128), 0, st, w, d, d_period, E, off,
                           scales, codes, objective);
    }
    return hipGetLastError();
}

}  // namespace cqk
