// Separately normalized environment diagonals from calibration activations, for gfx950
// (CliffQuant README, "What CliffQuant changes": each channel's sensitivity weighted by its
// activations, per calibration environment, each environment normalized on its own; model card, "Calibration and evaluation
// data": four environments of calibration windows, a 16-bit model runtime).
//
// Reading where the pages are silent: d_{e,i} = (1/T) sum_t x_{t,i}^2 over environment e's T
// tokens, divided by its mean over the channels i, in binary64, rounded once to binary32 and
// written in the solver's layout [in/128][E][128].
//
// The pass over the activations is HBM-bound (2 bytes per element, one binary64 fma each):
//   1. partial sums: a workgroup takes 512 channels (64 lanes x 8 bf16, one 16-byte load per
//      lane per row, eight rows in flight) of a chunk of rows; its four waves take every fourth
//      row and meet in LDS in a fixed order;
//   2. per channel, the chunks' sums in order, divided by T;
//   3. per environment, one workgroup: the mean over channels (fixed-order reduction), then the
//      normalized values.
// Every order is fixed, so repeated runs are bit-identical.
#include "device.h"
#include "launch.h"

namespace cqk {
namespace {

constexpr int DIAG_COLS = 512;  // channels per workgroup in the partial pass

__device__ __forceinline__ double bf16_value(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

// grid (in / DIAG_COLS rounded up, n_chunks, E); 256 threads
__global__ __launch_bounds__(256) void diag_partial_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t in,
                                                           int64_t rows_per_chunk, int n_chunks,
                                                           double* __restrict__ part) {
    __shared__ double red[3][64 * 8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.z, chunk = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * DIAG_COLS + 8 * lane;  // this lane's first channel
    const bool live = c0 < in;
    const int64_t r0 = (int64_t)chunk * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < T ? r0 + rows_per_chunk : T;
    double acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0;
    if (live) {
        const uint16_t* base = x + ((int64_t)e * T) * in + c0;
        int64_t r = r0 + wave;
#pragma unroll 1
        for (; r + 28 < r1; r += 32) {  // eight rows per wave in flight
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(base + (r + 4 * u) * in);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const double lo = bf16_value(w[h] & 0xFFFFu), hi = bf16_value(w[h] >> 16);
                    acc[2 * h] = __builtin_fma(lo, lo, acc[2 * h]);
                    acc[2 * h + 1] = __builtin_fma(hi, hi, acc[2 * h + 1]);
                }
            }
        }
        for (; r < r1; r += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(base + r * in);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const double lo = bf16_value(w[h] & 0xFFFFu), hi = bf16_value(w[h] >> 16);
                acc[2 * h] = __builtin_fma(lo, lo, acc[2 * h]);
                acc[2 * h + 1] = __builtin_fma(hi, hi, acc[2 * h + 1]);
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) red[wave - 1][lane * 8 + k] = acc[k];
    }
    __syncthreads();
    if (wave == 0 && live) {
        double* out = part + ((int64_t)e * n_chunks + chunk) * in + c0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            out[k] = ((acc[k] + red[0][lane * 8 + k]) + red[1][lane * 8 + k]) + red[2][lane * 8 + k];
    }
}

// thread per (e, channel)
__global__ __launch_bounds__(256) void diag_reduce_kernel(const double* __restrict__ part, int E, int n_chunks,
                                                          int64_t in, int64_t T, double* __restrict__ msq) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)E * in) return;
    const int64_t e = t / in, i = t % in;
    const double* p = part + e * n_chunks * in + i;
    // eight interleaved accumulators (the loads independent of the adds), combined in a fixed order
    double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] += p[(int64_t)(c + k) * in];
    }
    for (; c < n_chunks; ++c) s[0] += p[(int64_t)c * in];
    msq[t] = (((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]))) / (double)T;
}

// one 256-thread workgroup per environment
__global__ __launch_bounds__(256) void diag_normalize_kernel(const double* __restrict__ msq, int E, int64_t in,
                                                             float* __restrict__ d) {
    __shared__ double red[4];
    const int e = blockIdx.x;
    const double* m = msq + (int64_t)e * in;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < in; i += 256) s += m[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += lane_xor(s, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const double mean = (((red[0] + red[1]) + red[2]) + red[3]) / (double)in;
    for (int64_t i = threadIdx.x; i < in; i += 256)
        d[((i / G) * E + e) * G + (i % G)] = (float)(m[i] / mean);
}

}  // namespace

int64_t diag_chunks(int E, int64_t T, int64_t in) {
    // about 512 workgroups in the partial pass (each wave keeps eight 1 KB rows in flight), each
    // with at least 32 rows: few enough chunks for a short second pass
    const int64_t tiles = (in + DIAG_COLS - 1) / DIAG_COLS * E;
    int64_t n = (512 + tiles - 1) / tiles;
    const int64_t max_n = (T + 31) / 32;
    n = n < max_n ? n : max_n;
    return n < 1 ? 1 : n;
}

hipError_t launch_diagonals(const uint16_t* x, int E, int64_t T, int64_t in, float* d, double* part, double* msq,
                            hipStream_t st) {
    const int64_t n_chunks = diag_chunks(E, T, in);
    const int64_t rows = (T + n_chunks - 1) / n_chunks;
    const dim3 grid((unsigned)((in + DIAG_COLS - 1) / DIAG_COLS), (unsigned)n_chunks, (unsigned)E);
    hipLaunchKernelGGL(diag_partial_kernel, grid, dim3(256), 0, st, x, T, in, rows, (int)n_chunks, part);
    hipLaunchKernelGGL(diag_reduce_kernel, dim3((unsigned)((E * in + 255) / 256)), dim3(256), 0, st, part, E,
                       (int)n_chunks, in, T, msq);
    hipLaunchKernelGGL(diag_normalize_kernel, dim3((unsigned)E), dim3(256), 0, st, msq, E, in, d);
    return hipGetLastError();
}

}  // namespace cqk
