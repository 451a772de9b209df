// Vector-unit issue probe for gfx950: the fp32 fma rate the chip reaches, and the clock it holds,
// against which the full-grid search's issue rate and its fraction of the published fp32 peak are
// read.  Each thread runs eight independent fma chains (no packed fp32: the build turns it off),
// so every vector instruction of the loop is one v_fma_f32 over 64 lanes and the dependent
// latency is hidden by the chains and the waves.  Thread 0 of every workgroup reads the shader
// clock and the constant-rate wall clock at its start and end.  Two forms of the same fma are timed
// (below): the vector unit's rate depends on the instruction's encoding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace cqk {
namespace {

constexpr int PROBE_BLOCK = 256;
constexpr int PROBE_CHAINS = 8;

// MODE 0: x = fma(x, c, y) with c and y in vector registers: the three-operand encoding,
// v_fma_f32 (the destination is not the addend).  MODE 1: x = fma(y, c, x): the
// accumulate-into-destination encoding, v_fmac_f32 (the form of the full-grid search's
// environment sums).  MODE 2: x = fma(x, a, b) with a and b kernel arguments: v_fma_f32 with a
// scalar-register operand (one per instruction; the other is copied to a vector register).
template <int MODE>
__global__ __launch_bounds__(PROBE_BLOCK) void fma_probe_kernel(int iters, float a, float b, float* out,
                                                               uint64_t* clocks) {
    const int tid = threadIdx.x;
    uint64_t c0 = 0, r0 = 0;
    if (tid == 0) {
        c0 = clock64();
        r0 = wall_clock64();
    }
    float x[PROBE_CHAINS], y[PROBE_CHAINS];
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k) {
        x[k] = (float)(tid + k) * 0x1p-10f;
        y[k] = (float)(k + 1) * b + (float)(tid & 1) * 0.0f;  // vector registers (not folded to scalars)
    }
    // a in a vector register (the product with the lane's parity is not folded away)
    const float c = a + (float)(tid & 1) * 0.0f;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < PROBE_CHAINS; ++k) {
            if (MODE == 0) x[k] = __builtin_fmaf(x[k], c, y[k]);
            else if (MODE == 1) x[k] = __builtin_fmaf(y[k], c, x[k]);
            else x[k] = __builtin_fmaf(x[k], a, b);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k) s += x[k];
    out[(int64_t)blockIdx.x * PROBE_BLOCK + tid] = s;
    if (tid == 0) {
        const uint64_t c1 = clock64(), r1 = wall_clock64();
        clocks[2 * (int64_t)blockIdx.x] = c1 - c0;
        clocks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_fma_probe(int iters, int blocks, int mode, float* out, uint64_t* clocks, hipStream_t st) {
    // a = 1 - 2^-20 and b = 2^-20 keep every chain near its start value (modes 0 and 2) or let it
    // grow by at most 8 x 2^-20 per step (mode 1): no overflow or denormal slows a lane
    const float a = 1.0f - 0x1p-20f, b = 0x1p-20f;
    const dim3 grid((unsigned)blocks), block(PROBE_BLOCK);
    if (mode == 0) hipLaunchKernelGGL(fma_probe_kernel<0>, grid, block, 0, st, iters, a, b, out, clocks);
    else if (mode == 1) hipLaunchKernelGGL(fma_probe_kernel<1>, grid, block, 0, st, iters, a, b, out, clocks);
    else hipLaunchKernelGGL(fma_probe_kernel<2>, grid, block, 0, st, iters, a, b, out, clocks);
    return hipGetLastError();
}

}  // namespace cqk
