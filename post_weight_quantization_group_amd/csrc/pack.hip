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

// Several matrices in one launch: matrix k's codes, group scales and outputs follow those of
// matrices 0..k-1 back to back (offsets from the prefix sums of out * in).  Each workgroup forms
// the tile and element prefix sums of the (at most 256) shapes once, then loops over tiles,
// finding each tile's matrix by a binary search of the prefix; a tile is the same 64 x 128
// transpose as in pack_kernel.
__global__ __launch_bounds__(256) void pack_multi_kernel(const int8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ grp_scales, PackShapes m,
                                                         int64_t total_tiles, int32_t* __restrict__ qweight,
                                                         uint16_t* __restrict__ scales) {
    __shared__ __align__(16) uint8_t tile[PT_ROWS * PT_STRIDE];
    __shared__ int64_t tpre[PACK_MAX_MATS + 1], epre[PACK_MAX_MATS + 1];
    const int tid = threadIdx.x;
    // inclusive scans (Hillis-Steele) of the tiles and the elements of each matrix
    int64_t tv = 0, ev = 0;
    if (tid < m.n) {
        tv = (int64_t)((m.out[tid] + PT_ROWS - 1) / PT_ROWS) * (m.in[tid] / G);
        ev = (int64_t)m.out[tid] * m.in[tid];
    }
    tpre[tid + 1] = tv;
    epre[tid + 1] = ev;
    if (tid == 0) { tpre[0] = 0; epre[0] = 0; }
    __syncthreads();
    for (int o = 1; o < PACK_MAX_MATS; o <<= 1) {
        const int64_t a = tid + 1 > o ? tpre[tid + 1 - o] : 0, b = tid + 1 > o ? epre[tid + 1 - o] : 0;
        __syncthreads();
        tpre[tid + 1] += a;
        epre[tid + 1] += b;
        __syncthreads();
    }
    for (int64_t t = blockIdx.x; t < total_tiles; t += gridDim.x) {
        int lo = 0, hi = m.n - 1;  // the last k with tpre[k] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tpre[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int k = lo;
        const int64_t out = m.out[k], in = m.in[k], ngc = in / G;
        const int64_t local = t - tpre[k];
        const int64_t rt = (out + PT_ROWS - 1) / PT_ROWS;
        const int64_t c = local / rt, o0 = (local - c * rt) * PT_ROWS;
        const int8_t* cm = codes + epre[k];
        const uint16_t* gm = grp_scales + epre[k] / G;
        int32_t* qm = qweight + epre[k] / 8;
        uint16_t* sm = scales + epre[k] / G;
        {
            const int row = tid >> 2, q = tid & 3;
            const int64_t o = o0 + row;
            if (o < out) {
                const int4* src = (const int4*)(cm + o * in + c * G + q * 32);
                const int4 v0 = src[0], v1 = src[1];
                uint32_t* dst = (uint32_t*)(tile + row * PT_STRIDE + q * 32);
                dst[0] = (uint32_t)v0.x; dst[1] = (uint32_t)v0.y; dst[2] = (uint32_t)v0.z; dst[3] = (uint32_t)v0.w;
                dst[4] = (uint32_t)v1.x; dst[5] = (uint32_t)v1.y; dst[6] = (uint32_t)v1.z; dst[7] = (uint32_t)v1.w;
            }
        }
        __syncthreads();
        const int col = tid & 63;
        const int64_t o = o0 + col;
        if (o < out) {
            const uint8_t* trow = tile + col * PT_STRIDE;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int rl = (tid >> 6) + 4 * kk;
                const uint32_t lo32 = *(const uint32_t*)(trow + rl * 8);
                const uint32_t hi32 = *(const uint32_t*)(trow + rl * 8 + 4);
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    word |= ((((lo32 >> (8 * j)) & 0xFFu) + 8u) & 0xFu) << (4 * j);
                    word |= ((((hi32 >> (8 * j)) & 0xFFu) + 8u) & 0xFu) << (4 * (j + 4));
                }
                qm[(c * 16 + rl) * out + o] = (int32_t)word;
            }
            if (tid < 64) sm[c * out + o] = gm[o * ngc + c];
        }
        __syncthreads();
    }
}

hipError_t launch_pack_multi(const int8_t* codes, const uint16_t* grp_scales, const PackShapes& m,
                             int32_t* qweight, uint16_t* scales, hipStream_t st) {
    int64_t total = 0;
    for (int k = 0; k < m.n; ++k) total += (int64_t)((m.out[k] + PT_ROWS - 1) / PT_ROWS) * (m.in[k] / G);
    if (total == 0) return hipSuccess;
    const int64_t grid = total < 8192 ? total : 8192;
    hipLaunchKernelGGL(pack_multi_kernel, dim3((unsigned)grid), dim3(256), 0, st, codes, grp_scales, m, total,
                       qweight, scales);
    return hipGetLastError();
}

// Other field widths and group lengths (bits in {2, 4, 8}, any group length): the same transpose of
// 64 output rows through LDS over 128-channel tiles (the last one may be shorter; `in` is a multiple
// of 32 / bits, hence of 4), then one qweight word per (field row, output): field j of the word for
// channels (32/bits) r .. (32/bits) r + 32/bits - 1 is code + 2^(bits-1) modulo 2^bits.
__global__ __launch_bounds__(256) void pack_spec_kernel(const int8_t* __restrict__ codes, int64_t out, int64_t in,
                                                        int bits, int32_t* __restrict__ qweight) {
    __shared__ uint32_t tile[PT_ROWS][33];  // 64 rows x 128 code bytes, one padding word per row
    const int tid = threadIdx.x;
    const int64_t o0 = (int64_t)blockIdx.x * PT_ROWS, c0 = (int64_t)blockIdx.y * 128;
    const int nch = (int)(in - c0 < 128 ? in - c0 : 128);
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // 64 rows x 32 four-byte words
        const int idx = tid + 256 * k, row = idx >> 5, wc = idx & 31;
        uint32_t v = 0;
        if (o0 + row < out && 4 * wc < nch) v = *(const uint32_t*)(codes + (o0 + row) * in + c0 + 4 * wc);
        tile[row][wc] = v;
    }
    __syncthreads();
    const int per = 32 / bits, col = tid & 63, nr = nch / per;
    const uint32_t mask = (1u << bits) - 1u, bias = 1u << (bits - 1);
    const int64_t o = o0 + col;
    if (o < out)
        for (int rl = tid >> 6; rl < nr; rl += 4) {
            uint32_t word = 0;
            for (int j = 0; j < per; ++j) {
                const int ch = rl * per + j;
                const uint32_t byte = (tile[col][ch >> 2] >> (8 * (ch & 3))) & 0xFFu;
                word |= ((byte + bias) & mask) << (bits * j);
            }
            qweight[(c0 / per + rl) * out + o] = (int32_t)word;
        }
}

// scales[c][o] = grp_scales[o][c], one thread per output element (output-fastest).
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ grp_scales, int64_t out,
                                                          int64_t ngc, uint16_t* __restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= ngc * out) return;
    const int64_t c = t / out, o = t - c * out;
    scales[t] = grp_scales[o * ngc + c];
}

hipError_t launch_pack_spec(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in, int bits,
                            int group_len, int32_t* qweight, uint16_t* scales, hipStream_t st) {
    if (out == 0 || in == 0) return hipSuccess;
    const dim3 grid((unsigned)((out + PT_ROWS - 1) / PT_ROWS), (unsigned)((in + 127) / 128));
    hipLaunchKernelGGL(pack_spec_kernel, grid, dim3(256), 0, st, codes, out, in, bits, qweight);
    const int64_t ngc = in / group_len, n = ngc * out;
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, grp_scales, out, ngc,
                       scales);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t* codes, const uint16_t* grp_scales, int64_t out, int64_t in,
                       int32_t* qweight, uint16_t* scales, hipStream_t st) {
    if (out == 0 || in == 0) return hipSuccess;
    const dim3 grid((unsigned)((out + PT_ROWS - 1) / PT_ROWS), (unsigned)(in / G));
    hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, st, codes, grp_scales, out, in, qweight, scales);
    return hipGetLastError();
}

}  // namespace cqk
