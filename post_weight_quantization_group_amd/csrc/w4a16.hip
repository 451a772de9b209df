// W4A16 matmul over the GPTQ-v1 tensors, for gfx950: the consumer check of the packed output
// (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Quantization configuration": GPTQ v1,
// 4 bits, group size 128, symmetric, 16-bit activations).
//
//   y[m][o] = sum_g s[g][o] * sum_{k in group g} x[m][k] * (u[k][o] - 8)
//
// with u the nibble of qweight and s the binary16 scale.  The inner sums are a dense contraction
// on the matrix cores: bf16 activations times the codes u - 8, which are small integers and so
// exact in bf16, through gfx950's v_mfma_f32_32x32x16_bf16 with fp32 accumulation (every product
// exact);
// the group's scale then enters with one fp32 fma per output.
//
// A 256-thread workgroup computes a 128 x 128 tile of y (four waves, each a 64 x 64 block of
// 2 x 2 MFMA tiles of 32 x 32).  Per group it stages the x tile [128][128] and the dequantized
// codes, transposed to [128][128] so that each lane reads its eight consecutive k at once, in
// LDS; 8 MFMA steps per tile cover the group, while the next group's tiles are already being
// loaded.
// Lane layout of the instruction (checked on gfx950): lane l holds A[l % 32][8 (l / 32) + j] and
// B[8 (l / 32) + j][l % 32], j = 0..7; result register r of lane l is D[8 (r / 4) + 4 (l / 32) +
// r % 4][l % 32].  Each lane's 16 results share one output column, hence one scale per group.
#include "device.h"
#include "launch.h"

namespace cqk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TN = 128, KG = 128;
constexpr int XS = KG + 8;  // LDS row stride (bf16) of both tiles: rows 16 bytes apart in banks

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// 8 codes of one output (one qweight word) as bf16 pairs: code k of the word is nibble k, minus 8.
// u XOR 8 read as a signed 4-bit field is u - 8; its binary32 value is a small integer, whose upper
// half is its bf16 pattern, and one byte permute packs two of them.
__device__ __forceinline__ uint4 codes_bf16(uint32_t word) {
    const uint32_t v = word ^ 0x88888888u;
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = (float)((int32_t)(v << (28 - 8 * j)) >> 28);
        const float hi = (float)((int32_t)(v << (24 - 8 * j)) >> 28);
        h[j] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    return make_uint4(h[0], h[1], h[2], h[3]);
}

// A (64 MT) x 128 tile of y per workgroup: four waves as 2 x 2 blocks of (32 MT) x 64, each an
// MT x 2 arrangement of 32 x 32 MFMA tiles (MT = 2 for throughput; MT = 1 for a few rows, where
// the larger tile would mostly multiply padding).  The dequantized codes of a group are staged once
// per workgroup and serve all its rows; the next group's x tile and code words are loaded into
// registers while the current group's MFMAs run.
template <int MT>
__global__ __launch_bounds__(256, 2) void w4a16_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ scales, int64_t M, int64_t out,
                                                    int64_t in, float* __restrict__ y) {
    constexpr int TMB = 64 * MT;
    __shared__ __align__(16) uint16_t xs[TMB * XS];  // [m][k]
    __shared__ __align__(16) uint16_t bs[TN * XS];   // [n][k], the codes u - 8 as bf16
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // workgroups are dealt to the eight XCDs in turn: all column tiles of a row block go to one XCD,
    // so that its L2 serves the row block's activations to all of them
    const int64_t nx = gridDim.x, ny = gridDim.y, L = (int64_t)blockIdx.y * nx + blockIdx.x;
    int64_t bx = L % nx, by = L / nx;
    if (ny % 8 == 0) {
        const int64_t j = L >> 3;
        by = 8 * (j / nx) + (L & 7);
        bx = j % nx;
    }
    const int64_t m0 = by * TMB, n0 = bx * TN;
    const int wm = (wave >> 1) * 32 * MT, wn = (wave & 1) * 64;
    const int64_t n_groups = in / KG;
    uint4 xv[4 * MT];
    uint32_t qv[8];
    auto fetch = [&](int64_t g) {
#pragma unroll
        for (int p = 0; p < 4 * MT; ++p) {  // TMB rows x 128 bf16: 16 TMB 16-byte pieces
            const int piece = tid + 256 * p, row = piece >> 4, col = (piece & 15) * 8;
            xv[p] = make_uint4(0, 0, 0, 0);
            if (m0 + row < M) xv[p] = *reinterpret_cast<const uint4*>(x + (m0 + row) * in + g * KG + col);
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {  // 16 qweight rows x 128 outputs
            const int item = tid + 256 * p, r = item >> 7, n = item & 127;
            qv[p] = 0x88888888u;  // code 0 outside the matrix
            if (n0 + n < out) qv[p] = (uint32_t)qw[(g * (KG / 8) + r) * out + n0 + n];
        }
    };
    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.0f;
    fetch(0);
    for (int64_t g = 0; g < n_groups; ++g) {
        __syncthreads();  // the previous group's MFMAs have read the tiles
#pragma unroll
        for (int p = 0; p < 4 * MT; ++p) {
            const int piece = tid + 256 * p, row = piece >> 4, col = (piece & 15) * 8;
            *reinterpret_cast<uint4*>(xs + row * XS + col) = xv[p];
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int item = tid + 256 * p, r = item >> 7, n = item & 127;
            *reinterpret_cast<uint4*>(bs + n * XS + 8 * r) = codes_bf16(qv[p]);
        }
        __syncthreads();
        if (g + 1 < n_groups) fetch(g + 1);
        f32x16 part[MT][2];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[i][t][r] = 0.0f;
        const uint16_t* arow = xs + (wm + (lane & 31)) * XS + 8 * (lane >> 5);
        const uint16_t* brow = bs + (wn + (lane & 31)) * XS + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KG / 16; ++ks) {
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(brow + 16 * ks);
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(brow + 32 * XS + 16 * ks);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * i * XS + 16 * ks);
                part[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, part[i][0], 0, 0, 0);
                part[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, part[i][1], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t col = n0 + wn + 32 * t + (lane & 31);
            const float sc = col < out ? half_bits_to_float(scales[g * out + col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][t][r] = __builtin_fmaf(sc, part[i][t][r], acc[i][t][r]);
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t col = n0 + wn + 32 * t + (lane & 31);
        if (col < out) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < M) y[row * out + col] = acc[i][t][r];
                }
        }
    }
}

}  // namespace

hipError_t launch_w4a16(const uint16_t* x, const int32_t* qw, const uint16_t* scales, int64_t M, int64_t out,
                        int64_t in, float* y, hipStream_t st) {
    if (M <= 64) {
        const dim3 grid((unsigned)((out + TN - 1) / TN), (unsigned)((M + 63) / 64));
        hipLaunchKernelGGL(w4a16_kernel<1>, grid, dim3(256), 0, st, x, qw, scales, M, out, in, y);
    } else {
        const dim3 grid((unsigned)((out + TN - 1) / TN), (unsigned)((M + 127) / 128));
        hipLaunchKernelGGL(w4a16_kernel<2>, grid, dim3(256), 0, st, x, qw, scales, M, out, in, y);
    }
    return hipGetLastError();
}

}  // namespace cqk
