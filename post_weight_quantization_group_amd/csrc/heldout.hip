// Held-out comparison of two scale policies on the proxy's per-group values, for gfx950
// (CliffQuant README, "Held-out reconstruction proxy": CliffQuant's wins, ties and losses
// against Pooled-WMSE by group, and a bootstrap of the effect that resamples groups within each
// module, with the same draws for both policies, and its 95% interval).
//
// Readings where the pages are silent: A wins a group when p_A < p_B, ties when p_A == p_B;
// the effect is the mean over modules of each module's mean of (p_B - p_A); replicate r
// resamples each module's groups with replacement, the same draw for both policies, the draws
// being an input (boot_idx); the interval is the linear-interpolation percentile of the sorted
// replicates.  Every sum runs left to right in binary64, so the results are the sequential
// definition bit for bit.
//
// Launches: counts (one workgroup); module means with row 0 the identity draw, either from LDS (the
// differences and each row's draws staged there, one thread per module) or, for more than 4,096
// groups, one thread per (row, module) from global memory; macro means, one thread per row; a rank
// sort of the replicates under a total order (NaN last, ties by index): ranks counted over key
// tiles on a 2-D grid and added with integer atomics, then a scatter; the two percentiles.
#include "device.h"
#include "launch.h"

namespace cqk {
namespace {

constexpr int COUNT_THREADS = 1024;

__global__ __launch_bounds__(COUNT_THREADS) void heldout_counts_kernel(const double* __restrict__ pa,
                                                                       const double* __restrict__ pb,
                                                                       int64_t n, int64_t* __restrict__ counts) {
    __shared__ uint64_t red[3][COUNT_THREADS / 64];
    uint64_t c[3] = {0, 0, 0};
    for (int64_t g = threadIdx.x; g < n; g += COUNT_THREADS) {
        const double a = pa[g], b = pb[g];
        c[0] += a < b ? 1u : 0u;
        c[1] += a == b ? 1u : 0u;
        c[2] += a > b ? 1u : 0u;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) c[k] += lane_xor(c[k], o);
        if ((threadIdx.x & 63) == 0) red[k][threadIdx.x >> 6] = c[k];
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        uint64_t t = 0;
        for (int w = 0; w < COUNT_THREADS / 64; ++w) t += red[threadIdx.x][w];
        counts[threadIdx.x] = (int64_t)t;
    }
}

// Row 0: the identity draw (the point estimate); row r + 1: replicate r.
__global__ __launch_bounds__(256) void heldout_module_means_kernel(const double* __restrict__ pa,
                                                                   const double* __restrict__ pb,
                                                                   int64_t n, const int64_t* __restrict__ off,
                                                                   int M, const int32_t* __restrict__ idx,
                                                                   int B, double* __restrict__ mm) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)(B + 1) * M) return;
    const int row = (int)(t / M), m = (int)(t % M);
    const int64_t lo = off[m], hi = off[m + 1];
    double v = __builtin_nan("");
    if (lo >= 0 && hi <= n && lo < hi) {
        const int32_t* draw = row == 0 ? nullptr : idx + (int64_t)(row - 1) * n;
        // a draw outside the module marks the row bad and reads the module's first group instead,
        // so the loop has no early exit and the loads of later steps issue ahead of the adds
        bool ok = true;
        double acc = 0.0;
#pragma unroll 4
        for (int64_t j = lo; j < hi; ++j) {
            int64_t g = draw ? (int64_t)draw[j] : j;
            const bool in = g >= lo && g < hi;
            ok = ok && in;
            g = in ? g : lo;
            const double dv = pb[g] - pa[g];
            acc = j == lo ? dv : acc + dv;
        }
        if (ok) v = acc / (double)(hi - lo);
    }
    mm[t] = v;
}

// The same sums with the differences (once) and each row's draws staged in LDS: one workgroup per
// MEANS_ROWS rows, one thread per module summing from LDS in the same order.  n <= MEANS_LDS_N.
constexpr int MEANS_ROWS = 16;
constexpr int MEANS_LDS_N = 4096;

__global__ __launch_bounds__(256) void heldout_module_means_lds_kernel(const double* __restrict__ pa,
                                                                       const double* __restrict__ pb, int n,
                                                                       const int64_t* __restrict__ off, int M,
                                                                       const int32_t* __restrict__ idx, int B,
                                                                       double* __restrict__ mm) {
    __shared__ double diff[MEANS_LDS_N];
    __shared__ int32_t draw[MEANS_LDS_N];
    for (int g = threadIdx.x; g < n; g += 256) diff[g] = pb[g] - pa[g];
    const int r0 = blockIdx.x * MEANS_ROWS;
    const int r1 = r0 + MEANS_ROWS < B + 1 ? r0 + MEANS_ROWS : B + 1;
    for (int row = r0; row < r1; ++row) {
        __syncthreads();
        if (row == 0) {
            for (int j = threadIdx.x; j < n; j += 256) draw[j] = j;
        } else {
            const int32_t* src = idx + (int64_t)(row - 1) * n;
            for (int j = threadIdx.x; j < n; j += 256) draw[j] = src[j];
        }
        __syncthreads();
        for (int m = threadIdx.x; m < M; m += 256) {
            const int64_t lo = off[m], hi = off[m + 1];
            double v = __builtin_nan("");
            if (lo >= 0 && hi <= n && lo < hi) {
                bool ok = true;
                double acc = 0.0;
#pragma unroll 4
                for (int64_t j = lo; j < hi; ++j) {
                    int64_t g = draw[j];
                    const bool in = g >= lo && g < hi;
                    ok = ok && in;
                    g = in ? g : lo;
                    const double dv = diff[g];
                    acc = j == lo ? dv : acc + dv;
                }
                if (ok) v = acc / (double)(hi - lo);
            }
            mm[(int64_t)row * M + m] = v;
        }
    }
}

__global__ __launch_bounds__(256) void heldout_macro_kernel(const double* __restrict__ mm, int M, int B,
                                                            double* __restrict__ effect,
                                                            double* __restrict__ reps, int32_t* __restrict__ rank) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row > B) return;
    const double* r = mm + (int64_t)row * M;
    double acc = r[0];
    for (int m = 1; m < M; ++m) acc = acc + r[m];
    const double v = acc / (double)M;
    if (row == 0) {
        *effect = v;
    } else {
        reps[row - 1] = v;
        rank[row - 1] = 0;  // the rank counters the next launch adds into
    }
}

// Total order on binary64 values with every NaN last: flip the sign bit of non-negative
// values and every bit of negative ones.
__device__ __forceinline__ uint64_t order_key(double v) {
    if (__builtin_isnan(v)) return ~0ull;
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int RANK_TILE = 1024;

// grid (B / 256 rounded up, B / RANK_TILE rounded up): workgroup (x, y) counts, for its 256
// replicates, the replicates of key tile y ordered before them, and adds the count to their rank
// (integer sums: the same total in any order).
__global__ __launch_bounds__(256) void heldout_rank_kernel(const double* __restrict__ reps, int B,
                                                           int32_t* __restrict__ rank) {
    __shared__ uint64_t tile[RANK_TILE];
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t ki = order_key(i < B ? reps[i] : 0.0);
    const int t0 = blockIdx.y * RANK_TILE;
    const int tn = B - t0 < RANK_TILE ? B - t0 : RANK_TILE;
    for (int k = threadIdx.x; k < tn; k += blockDim.x) tile[k] = order_key(reps[t0 + k]);
    __syncthreads();
    int cnt = 0;
#pragma unroll 8
    for (int k = 0; k < tn; ++k) {
        const uint64_t kj = tile[k];
        cnt += (kj < ki || (kj == ki && t0 + k < i)) ? 1 : 0;
    }
    if (i < B && cnt > 0) atomicAdd(&rank[i], cnt);
}

__global__ __launch_bounds__(256) void heldout_scatter_kernel(const double* __restrict__ reps,
                                                              const int32_t* __restrict__ rank, int B,
                                                              double* __restrict__ sorted) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < B) sorted[rank[i]] = reps[i];
}

__device__ __forceinline__ double percentile_sorted(const double* v, int B, double q) {
    const double pos = q * (double)(B - 1);
    const int lo = (int)__builtin_floor(pos);
    const double t = pos - (double)lo;
    if (lo + 1 >= B) return v[B - 1];
    return v[lo] + (v[lo + 1] - v[lo]) * t;
}

__global__ void heldout_ci_kernel(const double* __restrict__ sorted, int B, double alpha, double* __restrict__ ci) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    if (B == 0 || __builtin_isnan(sorted[B - 1])) {
        ci[0] = ci[1] = __builtin_nan("");
        return;
    }
    ci[0] = percentile_sorted(sorted, B, alpha / 2.0);
    ci[1] = percentile_sorted(sorted, B, 1.0 - alpha / 2.0);
}

__global__ void heldout_nan_kernel(double* __restrict__ ci) {
    if (threadIdx.x == 0 && blockIdx.x == 0) ci[0] = ci[1] = __builtin_nan("");
}

}  // namespace

hipError_t launch_heldout(const double* pa, const double* pb, int64_t n, const int64_t* off, int M,
                          const int32_t* idx, int B, double alpha, int64_t* counts, double* effect,
                          double* boot, double* ci, double* mm, double* reps, int32_t* rank, hipStream_t st) {
    hipLaunchKernelGGL(heldout_counts_kernel, dim3(1), dim3(COUNT_THREADS), 0, st, pa, pb, n, counts);
    if (n <= MEANS_LDS_N) {
        hipLaunchKernelGGL(heldout_module_means_lds_kernel, dim3((unsigned)((B + 1 + MEANS_ROWS - 1) / MEANS_ROWS)),
                           dim3(256), 0, st, pa, pb, (int)n, off, M, idx, B, mm);
    } else {
        const int64_t rows = (int64_t)(B + 1) * M;
        hipLaunchKernelGGL(heldout_module_means_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, pa,
                           pb, n, off, M, idx, B, mm);
    }
    hipLaunchKernelGGL(heldout_macro_kernel, dim3((unsigned)((B + 1 + 255) / 256)), dim3(256), 0, st, mm, M, B,
                       effect, reps, rank);
    if (B > 0) {
        hipLaunchKernelGGL(heldout_rank_kernel, dim3((unsigned)((B + 255) / 256), (unsigned)((B + RANK_TILE - 1) / RANK_TILE)),
                           dim3(256), 0, st, reps, B, rank);
        hipLaunchKernelGGL(heldout_scatter_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, reps, rank, B,
                           boot);
        hipLaunchKernelGGL(heldout_ci_kernel, dim3(1), dim3(64), 0, st, boot, B, alpha, ci);
    } else {
        hipLaunchKernelGGL(heldout_nan_kernel, dim3(1), dim3(64), 0, st, ci);
    }
    return hipGetLastError();
}

}  // namespace cqk
