// GPTQ-v1 packer for gfx950 (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model
// card, "Quantization configuration": GPTQ v1, 4-bit, group size 128,
// symmetric; the scale policy changes, the packed format does not).
//
//   qweight[r][o] (int32, [in/8][out]): nibble j = codes[o][8r+j] + 8
//   scales[c][o]  (uint16, [in/128][out]) = grp_scales[o][c]
//
// The groups run along `in` while both outputs are `out`-contiguous, so each
// 256-thread workgroup transposes a tile of 64 output rows x 128 input
// channels (one group column) through LDS: the codes tile is read as 16-byte
// row segments and the 16 x 64 qweight words are written as full 256-byte
// rows.  The LDS row stride is 132 bytes so that the 64 lanes reading one
// word each fall in distinct banks.
#include "device.h"
#include "launch.h"

namespace cqk {

constexpr int PT_ROWS = 64;
constexpr int PT_STRIDE = 132;  // bytes per LDS row (128 + 4)

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ grp_scales,
                                                   int64_t out, int64_t in, int32_t* __restrict__ qweight,
                                                   uint16_t* __restrict__ scales) {
    __shared__ __align__(16) uint8_t tile[PT_ROWS * PT_STRIDE];
    const int tid = threadIdx.x;
    const int64_t o0 = (int64_t)blockIdx.x * PT_ROWS;
    const int64_t c = blockIdx.y;  // group column
    const int64_t ngc = in / G;
    // load: 64 rows x 128 bytes, thread -> (row, 32-byte quarter) as two 16-byte loads
    {
        const int row = tid >> 2, q = tid & 3;
        const int64_t o = o0 + row;
        if (o < out) {
            const int4* src = (const int4*)(codes + o * in + c * G + q * 32);
            const int4 v0 = src[0], v1 = src[1];
            uint32_t* dst = (uint32_t*)(tile + row * PT_STRIDE + q * 32);
            dst[0] = (uint32_t)v0.x; dst[1] = (uint32_t)v0.y; dst[2] = (uint32_t)v0.z; dst[3] = (uint32_t)v0.w;
            dst[4] = (uint32_t)v1.x; dst[5] = (uint32_t)v1.y; dst[6] = (uint32_t)v1.z; dst[7] = (uint32_t)v1.w;
        }
    }
    __syncthreads();
    // store: 16 qweight rows x 64 columns; lane -> column, wave -> rows
    const int col = tid & 63;
    const int64_t o = o0 + col;
    if (o < out) {
        const uint8_t* trow = tile + col * PT_STRIDE;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rl = (tid >> 6) + 4 * k;  // 0..15 within the group
            const uint32_t lo = *(const uint32_t*)(trow + rl * 8);
            const uint32_t hi = *(const uint32_t*)(trow + rl * 8 + 4);
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                word |= ((((lo >> (8 * j)) & 0xFFu) + 8u) & 0xFu) << (4 * j);
                word |= ((((hi >> (8 * j)) & 0xFFu) + 8u) & 0xFu) << (4 * (j + 4));
            }
            qweight[(c * 16 + rl) * out + o] = (int32_t)word;
        }
        if (tid < 64) scales[c * out + o] = grp_scales[o * ngc + c];
    }
}

hipError_t launch_pack(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                       int32_t* qweight, uint16_t* scales, hipStream_t st) {
    if (out == 0 || in == 0) return hipSuccess;
    const dim3 grid((unsigned)((out + PT_ROWS - 1) / PT_ROWS), (unsigned)(in / G));
    hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, st, codes, grp_scales, out, in, qweight, scales);
    return hipGetLastError();
}

}  // namespace cqk
