// Internal launchers of the gfx950 kernels (host side, C++ linkage).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "search_args.h"

namespace cqk {

hipError_t launch_absmax_spec(const float* w, const float* d, int64_t d_period, int G, int qmin, int qmax, int E,
                              int64_t n_groups, uint16_t* scales, int8_t* codes, double* objective, hipStream_t st);
hipError_t launch_absmax(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups,
                         uint16_t* scales, int8_t* codes, double* objective, hipStream_t st);

hipError_t launch_pack_spec(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in, int bits,
                            int group_len, int32_t* qweight, uint16_t* scales, hipStream_t st);
hipError_t launch_pack(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                       int32_t* qweight, uint16_t* scales, hipStream_t st);

// Shapes of the matrices one multi-matrix packing launch takes (passed by value as the kernel
// argument; 2 KB).
constexpr int PACK_MAX_MATS = 256;
struct PackShapes {
    int32_t n;
    int32_t out[PACK_MAX_MATS];
    int32_t in[PACK_MAX_MATS];
};
hipError_t launch_pack_multi(const int8_t* codes, const uint16_t* grp_scales, const PackShapes& m,
                             int32_t* qweight, uint16_t* scales, hipStream_t st);

// W4A16 matmul y [M][out] = x [M][in] (bf16) times the GPTQ-v1 tensors dequantized.
hipError_t launch_w4a16(const uint16_t* x, const int32_t* qw, const uint16_t* scales, int64_t M, int64_t out,
                        int64_t in, float* y, hipStream_t st);

// Environment diagonals from bf16 activations [E][T][in] into d [in/128][E][128]; part
// (E * diag_chunks * in) and msq (E * in) are workspace.
int64_t diag_chunks(int E, int64_t T, int64_t in);
hipError_t launch_diagonals(const uint16_t* x, int E, int64_t T, int64_t in, float* d, double* part, double* msq,
                            hipStream_t st);

// Held-out comparison of two policies' per-group values: counts, effect, sorted bootstrap
// replicates and the percentile interval; mm ((B + 1) * M), reps (B) and rank (B) are workspace.
hipError_t launch_heldout(const double* pa, const double* pb, int64_t n, const int64_t* off, int M,
                          const int32_t* idx, int B, double alpha, int64_t* counts, double* effect,
                          double* boot, double* ci, double* mm, double* reps, int32_t* rank, hipStream_t st);

hipError_t launch_proxy_spec(const float* w, const float* d, int64_t d_period, int G, int qmin, int qmax, int E,
                             int64_t n_groups, int P, const uint16_t* scales, const int64_t* module_offsets,
                             int n_modules, double* module_mean, double* macro, double* per_group, hipStream_t st);
hipError_t launch_proxy(const float* w, const float* d, int64_t d_period, int E, int64_t n_groups, int P,
                        const uint16_t* scales, const int64_t* module_offsets, int n_modules,
                        double* module_mean, double* macro, double* per_group, hipStream_t st);

// Vector-unit issue probe: `blocks` workgroups of 256 threads, each thread 8 independent chains of
// `iters` fp32 fmas in the form `mode` selects (0: v_fma_f32, 1: v_fmac_f32, 2: v_fma_f32 with a scalar operand); out [blocks * 256] floats, clocks [2 * blocks] (shader cycles, wall ticks).
hipError_t launch_fma_probe(int iters, int blocks, int mode, float* out, uint64_t* clocks, hipStream_t st);

}  // namespace cqk
