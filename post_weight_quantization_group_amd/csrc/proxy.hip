// Module-macro worst-environment weighted MSE for gfx950
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Held-out
// reconstruction proxy"; CliffQuant README, "Held-out reconstruction proxy").
//
//   p_g   = max_e (1/128) sum_i d_eval[e][i] (w_i - s_g q_i(s_g))^2   (binary64)
//   mean over each module's groups, then the mean over modules.
//
// Stage 1: one wave per group, two weights per lane; each lane forms its two
// squared residuals once and the E environment sums are wave-reduced in
// binary64.  Stage 2: one workgroup per module sums its p_g in a fixed order.
// Stage 3: one workgroup averages the module means in a fixed order.  Every
// reduction order is fixed, so repeated runs are bit-identical.
#include "device.h"
#include "launch.h"

namespace cqk {

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += lane_xor(v, o);
    return v;
}

__global__ __launch_bounds__(256) void proxy_group_kernel(const float* __restrict__ w, const float* __restrict__ d,
                                                          int64_t d_period, int E, int64_t n_groups,
                                                          const uint16_t* __restrict__ scales,
                                                          double* __restrict__ per_group) {
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= n_groups) return;
    const float* dg = d + (g % d_period) * (int64_t)E * G;
    const float2 wv = ((const float2*)(w + g * G))[lane];
    const double s = (double)half_bits_value(scales[g]);
    const double inv = 1.0 / s;
    double t2[2];
    const float wl[2] = {wv.x, wv.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const double wi = (double)wl[h];
        double r = __builtin_rint(wi * inv);
        r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
        const double t = wi - s * r;
        t2[h] = t * t;
    }
    double worst = 0.0;
    for (int e = 0; e < E; ++e) {
        const float2 dv = ((const float2*)(dg + e * G))[lane];
        double part = (double)dv.x * t2[0] + (double)dv.y * t2[1];
        part = wave_sum_f64(part);
        worst = e == 0 ? part : (part > worst ? part : worst);
    }
    if (lane == 0) per_group[g] = worst / 128.0;
}

__global__ __launch_bounds__(256) void proxy_module_kernel(const double* __restrict__ per_group,
                                                           const int64_t* __restrict__ off, int64_t n_groups,
                                                           double* __restrict__ module_mean) {
    __shared__ double red[256];
    const int m = blockIdx.x;
    const int64_t lo = off[m], hi = off[m + 1];
    const bool valid = lo >= 0 && hi <= n_groups && lo < hi;
    // each thread sums a contiguous run of the module's groups (four interleaved accumulators,
    // the loads independent of the adds), then a fixed tree: repeated runs are bit-identical
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (valid) {
        const int64_t per = (hi - lo + 255) / 256;
        const int64_t b = lo + (int64_t)threadIdx.x * per;
        const int64_t e = b + per < hi ? b + per : hi;
        int64_t g = b;
#pragma unroll 4
        for (; g + 4 <= e; g += 4) {
            acc[0] += per_group[g];
            acc[1] += per_group[g + 1];
            acc[2] += per_group[g + 2];
            acc[3] += per_group[g + 3];
        }
        for (; g < e; ++g) acc[0] += per_group[g];
    }
    red[threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) module_mean[m] = valid ? red[0] / (double)(hi - lo) : __builtin_nan("");
}

__global__ __launch_bounds__(256) void proxy_macro_kernel(const double* __restrict__ module_mean, int n_modules,
                                                          double* __restrict__ macro) {
    __shared__ double red[256];
    double acc = 0.0;
    for (int m = threadIdx.x; m < n_modules; m += 256) acc += module_mean[m];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) *macro = red[0] / (double)n_modules;
}

hipError_t launch_proxy(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                        const uint16_t* scales, const int64_t* module_offsets, int n_modules,
                        double* module_mean, double* macro, double* per_group, hipStream_t st) {
    if (n_groups > 0) {
        const int64_t blocks = (n_groups + 3) / 4;
        hipLaunchKernelGGL(proxy_group_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, d, d_period, E,
                           n_groups, scales, per_group);
    }
    hipLaunchKernelGGL(proxy_module_kernel, dim3((unsigned)n_modules), dim3(256), 0, st, per_group,
                       module_offsets, n_groups, module_mean);
    hipLaunchKernelGGL(proxy_macro_kernel, dim3(1), dim3(256), 0, st, module_mean, n_modules, macro);
    return hipGetLastError();
}

}  // namespace cqk
