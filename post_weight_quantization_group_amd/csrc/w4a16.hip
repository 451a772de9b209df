// W4A16 matmul over the GPTQ-v1 tensors, for gfx950: the consumer check of the packed output
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Quantization configuration": GPTQ v1,
// 4 bits, group size 128, symmetric, 16-bit activations).
//
//   y[m][o] = sum_g s[g][o] * sum_{k in group g} x[m][k] * (u[k][o] - 8)
//
// with u the nibble of qweight and s the binary16 scale.  The inner sums are a dense contraction
// on the matrix cores: bf16 activations times the codes u - 8, which are small integers and so
// exact in bf16, through v_mfma_f32_32x32x8bf16_1k with fp32 accumulation (every product exact);
// the group's scale then enters with one fp32 fma per output.
//
// A 256-thread workgroup computes a 64 x 64 tile of y (four waves, each a 32 x 32 MFMA tile).
// Per group it stages the x tile [64][128] and the dequantized codes, transposed to [64][128]
// so that each lane reads its four consecutive k at once, in LDS; 16 MFMA steps cover the group.
// Lane layout of the instruction (checked on gfx950): lane l holds A[l % 32][4 (l / 32) + j] and
// B[4 (l / 32) + j][l % 32], j = 0..3; result register r of lane l is D[8 (r / 4) + 4 (l / 32) +
// r % 4][l % 32].  Each lane's 16 results share one output column, hence one scale per group.
#include "device.h"
#include "launch.h"

namespace cqk {
namespace {

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TM = 64, TN = 64, KG = 128;
constexpr int XS = KG + 8;  // LDS row stride (bf16) of both tiles: rows 16 bytes apart in banks

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ scales, int64_t M, int64_t out,
                                                    int64_t in, float* __restrict__ y) {
    __shared__ __align__(16) uint16_t xs[TM * XS];  // [m][k]
    __shared__ __align__(16) uint16_t bs[TN * XS];  // [n][k], the codes u - 8 as bf16
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    const int64_t n_groups = in / KG;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int64_t g = 0; g < n_groups; ++g) {
        __syncthreads();
        // x tile: 64 rows x 128 bf16 = 1,024 16-byte pieces, four per thread
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int piece = tid + 256 * p, row = piece >> 4, col = (piece & 15) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + row < M) v = *reinterpret_cast<const uint4*>(x + (m0 + row) * in + g * KG + col);
            *reinterpret_cast<uint4*>(xs + row * XS + col) = v;
        }
        // codes: 16 qweight rows x 64 outputs, one word (8 codes of one output) per (row, output)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int item = tid + 256 * p, r = item >> 6, n = item & 63;
            uint32_t word = 0x88888888u;  // code 0 outside the matrix
            if (n0 + n < out) word = (uint32_t)qw[(g * (KG / 8) + r) * out + n0 + n];
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = (float)((int)((word >> (8 * j)) & 0xFu) - 8);
                const float hi = (float)((int)((word >> (8 * j + 4)) & 0xFu) - 8);
                h[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
            }
            *reinterpret_cast<uint4*>(bs + n * XS + 8 * r) = make_uint4(h[0], h[1], h[2], h[3]);
        }
        __syncthreads();
        f32x16 part;
#pragma unroll
        for (int r = 0; r < 16; ++r) part[r] = 0.0f;
        const uint16_t* arow = xs + (wm + (lane & 31)) * XS + 4 * (lane >> 5);
        const uint16_t* brow = bs + (wn + (lane & 31)) * XS + 4 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KG / 8; ++ks) {
            const bf16x4 a = *reinterpret_cast<const bf16x4*>(arow + 8 * ks);
            const bf16x4 b = *reinterpret_cast<const bf16x4*>(brow + 8 * ks);
            part = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, part, 0, 0, 0);
        }
        const int64_t col = n0 + wn + (lane & 31);
        const float s = col < out ? half_bits_to_float(scales[g * out + col]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(s, part[r], acc[r]);
    }
    const int64_t col = n0 + wn + (lane & 31);
    if (col < out) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < M) y[row * out + col] = acc[r];
        }
    }
}

}  // namespace

hipError_t launch_w4a16(const uint16_t* x, const int32_t* qw, const uint16_t* scales, int64_t M, int64_t out,
                        int64_t in, float* y, hipStream_t st) {
    const dim3 grid((unsigned)((out + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    hipLaunchKernelGGL(w4a16_kernel, grid, dim3(256), 0, st, x, qw, scales, M, out, in, y);
    return hipGetLastError();
}

}  // namespace cqk
