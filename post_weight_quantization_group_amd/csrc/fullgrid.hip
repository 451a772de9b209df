// Full-grid exhaustive FP16 scale search for gfx950: every one of the 31,743
// positive finite binary16 scales, every weight, every environment.
//
// This is the independent enumerator the pages describe next to the production
// solver (CliffQuant repository README, "What CliffQuant changes": a separate
// reference evaluates every one of the 31,743 binary16 values; README and model
// card, "Verification": solver cases matched exhaustive FP16 enumeration).  No
// scale is skipped, no range of the grid is cut off and no term is taken in
// closed form: for each group the kernel forms the binary32 objective at all
// 31,743 patterns from all G weights, then rescores in binary64 every pattern
// the binary32 error bound cannot rule out.
//
// The quantizer is a parameter (README, "Use the solver": a quantizer
// specification with qmin and qmax, and groups of any length): codes are
// clip(round-half-even(w/s), qmin, qmax), groups hold G <= 256 weights.
//
// Work split.  One 256-thread workgroup per group (below 1,024 groups, several
// workgroups per group, each on a share of the chunks, and a merge).  Weights
// and diagonals are staged in LDS as one row per weight: the pre-scaled weight
// and its E diagonals behind one address.  Each wave takes chunks of 64*NS
// consecutive patterns, NS per lane, and runs all G weights against its NS
// scales with the E per-environment sums in registers:
//     x = w' * r (r the reciprocal of s', below),  q = rint(x) (clipped when the
//     chunk can clip),  e = fma(-s', q, w'),  e^2,  then E fmas into the sums.
// A chunk cannot clip when every |w'| is at most (range end + 1/4) times its
// smallest scale; the clip is then left out (it cannot change any code).  In a
// chunk that can clip, a weight whose |w'| is at least (range end - 1/4) times
// the chunk's largest scale has the range end as its code at every scale of the
// chunk: its terms are formed from that code, without the quotient (the vector
// path keeps its rows in clip-ratio order, so these weights are one run).  In any
// chunk, a weight with |w'| at most (1 - 2^-20)/2 times the chunk's smallest scale
// has code 0 at every scale of the chunk (|x~| < 1/2); these weights end the row
// order, and their terms too are formed from their code, 0, without the quotient.
// Every term keeps the value the quotient path gives it, and its residual, square
// and E weighted fmas are still formed at every scale.
// Patterns are rotated over the lanes from chunk to chunk so that scales a power
// of two apart (which tie exactly when one outlier alone carries a code) land in
// different lanes.  Each lane keeps its best three (value, pattern) keys per
// policy; minimax F = max_e F_e and pooled P = sum_e F_e come from the same sums.
//
// Exactness (u = 2^-24).  The binary32 value is a screen with a proven bound:
//   * weights are pre-scaled by 2^k (max |w'| in [1, 2)) and scales by the same
//     2^k, which changes no quotient and no code; a range check guarantees that
//     every nonzero term d e^2 is a normal binary32 number (else the group goes
//     to the binary64 sweep below);
//   * r is the hardware estimate r0 = (1/s')(1 + t0), |t0| <= 2^-23, refined by
//     one Newton step with fmas: fma(-s', r0, 1) is exactly -t0 (a multiple of
//     2^-47 below 2^-23 in magnitude) and r = fma(r0, -t0, r0) = RN((1/s')(1 - t0^2)),
//     within (u + 2^-46) of 1/s' relatively; so x~ = RN(w' r) = x (1 + t) with
//     |t| <= 2 u + 2^-46 + u^2 < 2.0001 u, as for a correctly rounded reciprocal.
//     The code from x~ differs from the exact one only when x lies within 2.0001 u |x|
//     of a half-integer, |x| <= X = max(-qmin, qmax) + 1/2; both codes then leave
//     |x - q| within 1/2 -+ 2.0001 u X, so the term grows by a factor of at most
//     1 + 16.001 u X and never shrinks (the exact code is the nearer one);
//   * e is exact unless clipped (then one rounding); e^2 and the G fmas of the
//     sum give every term at most G + 3 roundings on its way into F_e.
//   So (1 - (G+3)u) F <= F~ <= (1 + (G+3)u)(1 + 16.001 u X) F, and the pooled sum
//   meets E - 1 more roundings.  Every pattern whose value is at most the
//   smallest one times the host-computed ratio (these bounds, with margin) is
//   rescored in binary64 in the definition's order, which decides the winner
//   and the lower-bit-pattern tie; the rescored value equals the oracle's bit
//   for bit.  A zero binary32 value is exact (every term is normal or zero), so
//   when the smallest value is 0 the lowest such pattern wins directly.  When a
//   lane's third key lies inside the bound (it may have dropped a fourth), or
//   more than CAP patterns survive, the group goes to the binary64 sweep.
#include <type_traits>

#include "device.h"
#include "search_args.h"

namespace cqk {
namespace full {

// Scales per lane per chunk: eight up to E = 4, then fewer so that the NS * E sums stay at 32
// registers.  A wave's chunk is 64 * NS consecutive patterns.
constexpr int ns_for(int E) { return E <= 4 ? 8 : 32 / E; }
constexpr int chunk_for(int E) { return 64 * ns_for(E); }
constexpr int nchunk_for(int E) { return ((int)N_SCALES + chunk_for(E) - 1) / chunk_for(E); }
constexpr int CAP = 256;                                // shortlist capacity per group
// The screen's LDS row of a weight: the pre-scaled weight, then from float doff_for(E) its E
// diagonals; one address serves a weight and its diagonals.  The vector path reads the diagonals
// as 16-byte broadcasts (offset 4, rows of a multiple of four floats); the matrix-core path
// (E >= 16) reads one float per lane, so its rows are packed (offset 1), which keeps six
// workgroups per CU within the LDS at E = 16.
constexpr int doff_for(int E) { return E >= 16 ? 1 : 4; }
constexpr int row_for(int E) { return E < 4 ? 8 : E + doff_for(E); }
constexpr int GMAX = 256;                               // longest group
constexpr uint8_t TAG_MINIMAX = 1, TAG_POOLED = 2;

constexpr int min_blocks_for(int E) { return E <= 4 ? 5 : (E == 8 ? 4 : (E == 16 ? 2 : 1)); }
// From sixteen environments on, the E weighted sums of each term run on the matrix cores: per
// weight and scale slot one v_mfma_f32_4x4x1f32 per four environments (below).  Measured on
// gfx950, the matrix-core instructions do not overlap the vector work of the chunk, and per
// multiply-add they cost what a vector fma costs: at E = 4 the matrix-core variant took 18.7 ms
// per 28,672-group matrix against 15.1 ms on the vector unit alone, at E = 16 41.6 ms against
// 45.7 ms for 32,768 groups (its E fmas per term are most of the work there, and the operands
// come from one 4-byte LDS read per four environments instead of 16-byte broadcasts).
constexpr bool use_mfma(int E) { return E >= 16; }
// The vector path orders its rows by clip ratio and gives a clipping chunk's weights that keep one
// code their own run (below); the matrix-core path keeps the rows in index order.
constexpr bool sorted_rows(int E) { return !use_mfma(E); }
typedef float v4f __attribute__((ext_vector_type(4)));

template <int E>
struct Smem {
    float w[GMAX];                  // the weights as given (rescoring, codes)
    // row i: w'_i = w_i 2^k (the screen's weight), zeros up to doff_for(E), then d[0..E-1][i] (the
    // environments past the call's E and the padding of E < 4 are zeros)
    __align__(16) float rows[GMAX * row_for(E)];
    float redf[4 * 8];
    uint64_t redk[4 * 4];
    uint32_t cand_b[CAP];
    uint8_t cand_tag[CAP];
    double cand_F[CAP];
    double cand_P[CAP];
    double pairF[BLOCK];
    int n_cand;
    int overflow;
    int n_key[2];                   // slices: keys stored per policy
    uint32_t ov_bits[2];            // slices: the smallest value not kept (binary32 bits)
    float thr[2];                   // each policy's shortlist threshold (-1: decided by the zero rule)
    uint32_t win_b[2];
    double win_F[2];
    uint8_t win_flags[2];
};
static_assert(sizeof(double) * CAP >= sizeof(int) * GMAX, "the staging ranks and clip ratios live in cand_F and cand_P");

// The value of a finite binary16 pattern by one hardware conversion (exact).
__device__ __forceinline__ float half_value_hw(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ void top3_insert(uint64_t (&k)[3], uint64_t v) {
    if (v < k[2]) {
        if (v < k[1]) {
            k[2] = k[1];
            if (v < k[0]) { k[1] = k[0]; k[0] = v; }
            else k[1] = v;
        } else {
            k[2] = v;
        }
    }
}

// A value held in a vector register: keeps the clip bounds out of scalar registers, which the
// hot loop's v_med3 would otherwise read through the scalar operand port.
__device__ __forceinline__ float in_vgpr(float x) {
    float r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
    return r;
}

// How a run of weights forms its codes in a chunk: the quotient, rounded, then clipped (CLIP); the
// same without the clip, for weights that cannot leave the range at any scale of the chunk (FREE);
// or, for weights that clip at every scale of the chunk, the range end on their side, kept in the
// row (FIXED); or, for weights whose code is 0 at every scale of the chunk, that 0 (ZERO, from a
// register the compiler cannot see through, so that the residual, the square and the E weighted
// sums are still formed at every scale).  Every mode gives each term exactly the value the clipped
// path gives it.
enum TermMode { FREE = 0, CLIP = 1, FIXED = 2, ZERO = 3 };

// One run of rows [0, n): every lane runs the n weights against its NS scales, the per-environment
// sums in registers.  The weight and its E diagonals are LDS broadcasts shared by the NS scales.
template <int E, int NS, int MODE>
__device__ __forceinline__ void chunk_terms(const float* __restrict__ rows, int n,
                                            const float (&nsv)[NS], const float (&inv)[NS], float qlo, float qhi,
                                            float (&acc)[NS][E]) {
    constexpr int RS = row_for(E);
    // rows in flight per iteration: fewer in the runs of clipping chunks from E = 8 on (measured)
    constexpr int UNROLL = MODE == FIXED || (MODE == CLIP && E > 4) ? 2 : 4;
#pragma unroll UNROLL
    for (int i = 0; i < n; ++i) {
        const float* row = rows + i * RS;
        const float wi = row[0];
        float di[E];
#pragma unroll
        for (int e = 0; e < E; ++e) di[e] = row[doff_for(E) + e];
        // the code this row keeps over the chunk
        const float qi = MODE == FIXED ? row[1] : (MODE == ZERO ? in_vgpr(0.0f) : 0.0f);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            float r = qi;
            if (MODE != FIXED && MODE != ZERO) {
                r = __builtin_rintf(wi * inv[t]);
                if (MODE == CLIP) r = __builtin_amdgcn_fmed3f(r, qlo, qhi);
            }
            const float ev = __builtin_fmaf(nsv[t], r, wi);
            const float e2 = ev * ev;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[t][e] = __builtin_fmaf(di[e], e2, acc[t][e]);
        }
    }
}

// The same run with the environment sums on the matrix cores.  v_mfma_f32_4x4x1f32 treats the
// wave as 16 blocks of four lanes: block b forms D[i][j] = C[i][j] + A_(4b+i) * B_(4b+j), kept in
// register i of lane 4b+j.  With A the diagonal of environment 4k + (lane & 3) and B the lane's own
// e^2, register i of lane L accumulates environment 4k + i of L's own scale: the same sums as the
// vector path, one fused multiply-add per term, and the vector unit is left the quotient, the
// rounding, the clip, the residual and the square.
template <int E, int NS, int MODE>
__device__ __forceinline__ void chunk_terms_mf(const float* __restrict__ rows, int n,
                                               const float (&nsv)[NS], const float (&inv)[NS], float qlo,
                                               float qhi, int lane4, v4f (&acc)[NS][E / 4]) {
    static_assert(MODE != FIXED, "the matrix-core rows hold no code");
    constexpr int RS = row_for(E);
    for (int i = 0; i < n; ++i) {
        const float* row = rows + i * RS;
        const float wi = row[0];
        float dl[E / 4];
#pragma unroll
        for (int k = 0; k < E / 4; ++k) dl[k] = row[doff_for(E) + 4 * k + lane4];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            float r = __builtin_rintf(wi * inv[t]);
            if (MODE == CLIP) r = __builtin_amdgcn_fmed3f(r, qlo, qhi);
            const float ev = __builtin_fmaf(nsv[t], r, wi);
            const float e2 = ev * ev;
#pragma unroll
            for (int k = 0; k < E / 4; ++k) acc[t][k] = __builtin_amdgcn_mfma_f32_4x4x1f32(dl[k], e2, acc[t][k], 0, 0, 0);
        }
    }
}

// The runs of a clipping chunk on the vector path.  With s0 <= s <= s1 the chunk's scales and
// u = 2^-24 (the quotient x~ within 2.0001 u |x| of w'/s, as for the screen's bound):
//   * w' >= (qmax - 1/4) s1 (1 + 2^-20) > 0 gives x~ > qmax - 1/4 at every scale: code qmax;
//   * w' <= (qmin + 1/4) s1 (1 + 2^-20) < 0 gives x~ < qmin + 1/4 at every scale: code qmin.
// The thresholds themselves take two roundings (4 u in all), far inside the 2^-20 margin.  The
// rows are in descending order of |w| over the end of the range on its side (staging), so the
// weights with one code over the chunk lead: the chunk runs [0, f) with each row's own code, f the
// first row that meets neither condition, and [f, G) clipped.  (A third run, the unclipped tail,
// would save one instruction on about 8% of the terms but pushes the kernel past the registers of
// five workgroups per CU.)  The sums meet the terms in row order whatever the runs.  The
// matrix-core rows hold no code: that path clips the whole chunk.
// The lane index through a vector move of its own, so that addresses formed from it are formed
// where they are used, not held in registers across the chunk loop.
__device__ __forceinline__ int fresh_lane() {
    int r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// The first row of the suffix of rows whose code is 0 at every scale of the chunk.  With s0 the
// chunk's smallest scale, |w'| <= s0 (1 - 2^-20) / 2 gives |x~| < 1/2 at every scale of the chunk
// (x~ within 2.0001 u |x| of w'/s, the threshold itself one rounding), so the code is 0, which lies
// in every code range.  The rows are in clip-ratio order, not in |w| order, so the suffix starts
// after the last row that does not qualify.
__device__ __forceinline__ int zero_run_start(const float* __restrict__ rows, int RS, int G, float s0) {
    const int lane = fresh_lane();
    const float tz = 0.5f * s0 * (1.0f - 0x1p-20f);
    int last = -1;
    for (int k0 = 0; k0 < G; k0 += 64) {
        const int k = k0 + lane;
        const float x = k < G ? rows[k * RS] : 0.0f;
        const uint64_t m = __ballot(k < G && !(fabsf(x) <= tz));
        if (m != 0) last = k0 + 63 - (int)__builtin_clzll(m);
    }
    return last + 1;
}

__device__ __forceinline__ int fixed_run_end(const float* __restrict__ rows, int RS, int G, int qmin, int qmax,
                                             float s1) {
    const int lane = fresh_lane();
    // the range ends through a vector move of its own: formed here, per chunk, not held in
    // registers across the chunk loop
    const float tA = qmin < 0 ? (in_vgpr((float)qmin) + 0.25f) * s1 * (1.0f + 0x1p-20f) : -__builtin_inff();
    const float tF = qmax > 0 ? (in_vgpr((float)qmax) - 0.25f) * s1 * (1.0f + 0x1p-20f) : __builtin_inff();
    for (int k0 = 0; k0 < G; k0 += 64) {
        const int k = k0 + lane;
        const float x = k < G ? rows[k * RS] : 0.0f;
        const uint64_t m = __ballot(k < G && !(x >= tF || x <= tA));
        if (m != 0) return k0 + (int)__builtin_ctzll(m);
    }
    return G;
}

// binary64 rescoring of shortlist entries [0, n): cand_F = max_e F_e, cand_P = (sum_e F_e)/E,
// each F_e summed i = 0..G-1 in the definition's order (the oracle's value bit for bit).
template <int E>
__device__ void rescore(Smem<E>& sm, int n, int G, int E_real, double qlo, double qhi) {
    constexpr int PER = BLOCK / E;
    const int t = threadIdx.x;
    for (int base = 0; base < n; base += PER) {
        const int nb = min(PER, n - base);
        if (t < nb * E) {
            const int j = base + t / E, e = t % E;
            const double s = (double)half_bits_value(sm.cand_b[j]);
            sm.pairF[t] = env_error_f64_n(sm.w, sm.rows + doff_for(E) + e, row_for(E), G, s, 1.0 / s, qlo, qhi);
        }
        __syncthreads();
        if (t < nb) {
            double F = sm.pairF[t * E], P = sm.pairF[t * E];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                const double v = sm.pairF[t * E + e];
                F = v > F ? v : F;
                P = P + v;
            }
            sm.cand_F[base + t] = F;
            sm.cand_P[base + t] = P / (double)E_real;
        }
        __syncthreads();
    }
}

// One wave: the lexicographic (value, bits) winner among the entries tagged `tag`, and its
// flags (more than one entry: near tie; another pattern with the same value: exact tie).
template <int E>
__device__ void pick_winner(Smem<E>& sm, int n, uint8_t tag, int slot) {
    const int lane = threadIdx.x & 63;
    uint64_t bv = ~0ull;
    uint32_t bb = 0xFFFFFFFFu;
    int count = 0;
    for (int j = lane; j < n; j += 64) {
        if (!(sm.cand_tag[j] & tag)) continue;
        const double v = tag == TAG_MINIMAX ? sm.cand_F[j] : sm.cand_P[j];
        const uint64_t vb = __builtin_bit_cast(uint64_t, v);  // values are >= 0: bits order as values
        const uint32_t b = sm.cand_b[j];
        ++count;
        if (vb < bv || (vb == bv && b < bb)) { bv = vb; bb = b; }
    }
    const uint64_t best_v = wave_min_u64(bv);
    const uint32_t best_b = (uint32_t)wave_min_u64(bv == best_v ? (uint64_t)bb : ~0ull);
    int tie = 0;
    for (int j = lane; j < n; j += 64) {
        if (!(sm.cand_tag[j] & tag)) continue;
        const double v = tag == TAG_MINIMAX ? sm.cand_F[j] : sm.cand_P[j];
        if (__builtin_bit_cast(uint64_t, v) == best_v && sm.cand_b[j] != best_b) tie = 1;
    }
#pragma unroll
    for (int k = 0; k < 6; ++k) {  // lane distances 32, 16, .., 1 (a counted loop, fully unrolled)
        count += (int)lane_xor((uint32_t)count, 32 >> k);
        tie |= (int)lane_xor((uint32_t)tie, 32 >> k);
    }
    if (lane == 0) {
        sm.win_b[slot] = best_b;
        sm.win_F[slot] = __builtin_bit_cast(double, best_v);
        sm.win_flags[slot] = (uint8_t)((count > 1 ? FLAG_NEAR_TIE : 0) | (tie ? FLAG_EXACT_TIE : 0));
    }
}

__device__ __forceinline__ void append_cand(uint32_t* cb, uint8_t* ct, int* n, uint32_t b, uint8_t tag) {
    const int j = atomicAdd(n, 1);
    if (j < CAP) { cb[j] = b; ct[j] = tag; }
}

__device__ __forceinline__ void queue_f64(const FullArgs& a, int64_t g) {
    const int j = atomicAdd(a.fb_count, 1);
    a.fb_list[j] = (int32_t)g;
}

// Staging and input checks for group g: w and the screen rows into LDS, the pre-scale 2^k and the
// chunk clip threshold.  Returns 0 (screen it), 1 (a non-finite or negative input) or 2 (outside
// the binary32 screen's guaranteed range).  Every workgroup of a group computes the same.
template <int E>
__device__ int stage_group(const FullArgs& a, int64_t g, Smem<E>& sm, float& pk_out, float& cmax_out) {
    const int tid = threadIdx.x;
    const int G = a.G;
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);

    // ---- staging (environments a.E..E-1 are zero padding).  On the vector path the screen's rows
    // go in descending order of the clip ratio |w| / (range end on w's side) (ties by index), so
    // that in a chunk the weights that clip at every scale come first: weight i's row is its rank,
    // the number of weights ahead of it.  The order changes no term, only the order of each sum's
    // additions, which the screen's bound does not depend on.  A NaN weight may give two weights
    // one rank (always within 0..G-1); such a group is rejected below before any row is read.
    constexpr int RS = row_for(E);
    int* rank = reinterpret_cast<int*>(sm.cand_F);  // free until the shortlist is rescored
    if constexpr (sorted_rows(E)) {
        static_assert(doff_for(E) >= 2, "a sorted row keeps its clip code in slot 1");
        float* ratio = reinterpret_cast<float*>(sm.cand_P);
        for (int i = tid; i < G; i += BLOCK) {
            const float x = wg[i];
            sm.w[i] = x;
            ratio[i] = x > 0.0f ? (a.qmax > 0 ? x / (float)a.qmax : 0.0f) : (a.qmin < 0 ? x / (float)a.qmin : 0.0f);
        }
        __syncthreads();
        for (int i = tid; i < G; i += BLOCK) {
            const float x = ratio[i];
            int r = 0;
            for (int j = 0; j < G; ++j) {
                const float y = ratio[j];
                r += (y > x || (y == x && j < i)) ? 1 : 0;
            }
            rank[i] = r;
        }
        __syncthreads();
        for (int j = tid; j < G * RS; j += BLOCK) {
            const int i = j / RS, f = j - i * RS, e = f - doff_for(E);
            sm.rows[rank[i] * RS + f] = (e >= 0 && e < a.E) ? dg[(int64_t)e * G + i] : 0.0f;
        }
    } else {
        for (int i = tid; i < G; i += BLOCK) {
            sm.w[i] = wg[i];
            rank[i] = i;
        }
        for (int j = tid; j < G * RS; j += BLOCK) {
            const int i = j / RS, f = j - i * RS, e = f - doff_for(E);
            sm.rows[j] = (e >= 0 && e < a.E) ? dg[(int64_t)e * G + i] : 0.0f;
        }
    }
    __syncthreads();

    // ---- input checks and ranges: bad, max|w|, max w+, max w-, min nonzero |w|, max d, min nonzero d
    float v[7] = {0.0f, 0.0f, 0.0f, 0.0f, -__builtin_inff(), 0.0f, -__builtin_inff()};
    for (int i = tid; i < G; i += BLOCK) {
        const float x = sm.w[i];
        if (!__builtin_isfinite(x)) v[0] = 1.0f;
        const float ax = fabsf(x);
        v[1] = fmaxf(v[1], ax);
        v[2] = fmaxf(v[2], x);
        v[3] = fmaxf(v[3], -x);
        if (ax > 0.0f) v[4] = fmaxf(v[4], -ax);
    }
    for (int j = tid; j < G * RS; j += BLOCK) {
        const float x = sm.rows[j];  // the weight slots are still zero here
        if (!(x >= 0.0f) || !__builtin_isfinite(x)) v[0] = 1.0f;
        else {
            v[5] = fmaxf(v[5], x);
            if (x > 0.0f) v[6] = fmaxf(v[6], -x);
        }
    }
    block_max_fn<7>(v, sm.redf);
    if (v[0] != 0.0f) return 1;
    const float wmax = v[1], wpos = v[2], wneg = v[3], wmin_nz = -v[4], dmax = v[5], dmin_nz = -v[6];

    // ---- power-of-two pre-scaling and the no-underflow / no-overflow guarantee: every nonzero
    // residual is at least the smaller of ulp(w') >= 2^-24 min|w'| and the binary16 grid spacing
    // 2^-24 * 2^k, so e^2 >= elb^2 must stay normal, also times the smallest nonzero diagonal
    int k = 0;
    if (wmax > 0.0f) {
        int ex;
        frexpf(wmax, &ex);
        k = min(100, max(-100, 1 - ex));
    }
    bool safe = dmax <= 0x1p100f;
    if (wmin_nz < __builtin_inff()) {
        const double elb = fmin(ldexp(1.0, k - 24), (double)wmin_nz * ldexp(1.0, k - 24));
        const double e2 = elb * elb;
        safe = safe && e2 >= 0x1p-120 && (dmin_nz == __builtin_inff() || (double)dmin_nz * e2 >= 0x1p-120);
    }
    if (!safe) return 2;
    const float pk = ldexpf(1.0f, k);
    for (int i = tid; i < G; i += BLOCK) {
        const float x = sm.w[i];
        sm.rows[rank[i] * RS] = x * pk;
        // the code the weight takes at every scale where it clips (the vector rows' slot 1)
        if (sorted_rows(E)) sm.rows[rank[i] * RS + 1] = x > 0.0f ? (float)a.qmax : (x < 0.0f ? (float)a.qmin : 0.0f);
    }
    if (tid == 0) {
        sm.n_cand = 0;
        sm.overflow = 0;
        sm.n_key[0] = sm.n_key[1] = 0;
        sm.ov_bits[0] = sm.ov_bits[1] = 0xFFFFFFFFu;
    }
    __syncthreads();
    // no weight clips in a chunk whose smallest scale s0 has w+ <= (qmax + 1/4) s0 and
    // w- <= (-qmin + 1/4) s0: |x~| stays below the range end plus 1/2
    const float cpos = wpos * pk / ((float)a.qmax + 0.25f), cneg = wneg * pk / (0.25f - (float)a.qmin);
    cmax_out = fmaxf(cpos, cneg) * (1.0f + 0x1p-20f);
    pk_out = pk;
    return 0;
}

// The outputs of a group with a non-finite or negative input.
__device__ void write_bad(const FullArgs& a, int64_t g) {
    const int tid = threadIdx.x;
    if (a.codes)
        for (int i = tid; i < a.G; i += BLOCK) a.codes[g * a.G + i] = 0;
    if (tid == 0) {
        if (a.scales) a.scales[g] = 0;
        if (a.objective) a.objective[g] = __builtin_nan("");
        if (a.pscales) a.pscales[g] = 0;
        if (a.pobjective) a.pobjective[g] = __builtin_nan("");
        if (a.flags) a.flags[g] = FLAG_BAD_INPUT | a.flag_or;
    }
}

// The binary32 screen of the chunks c with (c / 4) % S == slice (all of them when S = 1): every
// lane's best three (value, pattern) keys per policy.
template <int E>
__device__ void screen_keys(const FullArgs& a, Smem<E>& sm, float pk, float cmax, int slice, int S,
                            uint64_t (&mk)[3], uint64_t (&qk)[3]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, G = a.G;
    const float qlo = in_vgpr((float)a.qmin), qhi = in_vgpr((float)a.qmax);
    constexpr int NS = ns_for(E), CHUNK = chunk_for(E), NCHUNK = nchunk_for(E);
#pragma unroll
    for (int r = 0; r < 3; ++r) { mk[r] = KEY_NONE; qk[r] = KEY_NONE; }
    for (int c = wave + 4 * slice; c < NCHUNK; c += 4 * S) {
        const float s0 = half_value_hw(BITS_FIRST + (uint32_t)(c * CHUNK)) * pk;
        const bool clips = !(cmax <= s0);
        int end = 0;  // clipping chunks on the vector path: rows [0, end) keep one code over the chunk
        if (sorted_rows(E) && clips) {
            const float s1 = half_value_hw(min(BITS_FIRST + (uint32_t)(c * CHUNK + CHUNK - 1), BITS_LAST)) * pk;
            end = fixed_run_end(sm.rows, row_for(E), G, a.qmin, a.qmax, s1);
        }
        float nsv[NS], inv[NS];
        float acc[NS][E];
        const int rot = (lane + 5 * c) & 63;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const uint32_t b = min(BITS_FIRST + (uint32_t)(c * CHUNK + rot + 64 * t), BITS_LAST);
            const float s = half_value_hw(b) * pk;
            nsv[t] = -s;
            // hardware reciprocal and one Newton step: within one binary32 rounding of 1/s, the
            // accuracy the error bound assumes
            const float r0 = __builtin_amdgcn_rcpf(s);
            inv[t] = __builtin_fmaf(r0, __builtin_fmaf(-s, r0, 1.0f), r0);
        }
        if constexpr (use_mfma(E)) {
            v4f am[NS][E / 4];
#pragma unroll
            for (int t = 0; t < NS; ++t)
#pragma unroll
                for (int k = 0; k < E / 4; ++k) am[t][k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            if (!clips)
                chunk_terms_mf<E, NS, FREE>(sm.rows, G, nsv, inv, qlo, qhi, lane & 3, am);
            else
                chunk_terms_mf<E, NS, CLIP>(sm.rows, G, nsv, inv, qlo, qhi, lane & 3, am);
#pragma unroll
            for (int t = 0; t < NS; ++t)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[t][e] = am[t][e / 4][e % 4];
        } else {
#pragma unroll
            for (int t = 0; t < NS; ++t)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[t][e] = 0.0f;
            // rows [zs, G) have code 0 at every scale of the chunk (after any FIXED prefix: those
            // rows clip, so zs >= end)
            const int zs = zero_run_start(sm.rows, row_for(E), G, s0);
            const int mid = zs > end ? zs : end;
            if (!clips) {
                if (mid > 0) chunk_terms<E, NS, FREE>(sm.rows, mid, nsv, inv, qlo, qhi, acc);
            } else {
                if (end > 0) chunk_terms<E, NS, FIXED>(sm.rows, end, nsv, inv, qlo, qhi, acc);
                if (mid > end) chunk_terms<E, NS, CLIP>(sm.rows + end * row_for(E), mid - end, nsv, inv, qlo, qhi, acc);
            }
            if (mid < G) chunk_terms<E, NS, ZERO>(sm.rows + mid * row_for(E), G - mid, nsv, inv, qlo, qhi, acc);
        }
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const uint32_t b = BITS_FIRST + (uint32_t)(c * CHUNK + rot + 64 * t);
            if (b > BITS_LAST) continue;
            // the sums are +0 or positive: their maximum is that of their bit patterns
            uint32_t Fb = __float_as_uint(acc[t][0]);
            float Ps = acc[t][0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                const float x = acc[t][e];
                Fb = max(Fb, __float_as_uint(x));
                Ps = Ps + x;
            }
            const float Fm = __uint_as_float(Fb);
            if (a.want_minimax) top3_insert(mk, key_of(Fm, b));
            if (a.want_pooled) top3_insert(qk, key_of(Ps, b));
        }
    }
}

// After the shortlist (sm.cand_*, sm.n_cand, sm.overflow, and win_b of the zero rule): the binary64
// sweep when the screen was inconclusive, else rescoring, the lower-bit-pattern rule and outputs.
template <int E>
__device__ void decide_and_write(const FullArgs& a, int64_t g, Smem<E>& sm) {
    const int tid = threadIdx.x, wave = tid >> 6, G = a.G;
    const int n = sm.n_cand;
    if (sm.overflow || n > CAP) {
        if (tid == 0) queue_f64(a, g);
        return;
    }
    if (sorted_rows(E) && n > 0) {
        // the diagonals back in index order (the screen's rows are in clip-ratio order):
        // rescoring adds each environment's terms over i = 0..G-1
        constexpr int RS = row_for(E);
        const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);
        for (int j = tid; j < G * RS; j += BLOCK) {
            const int i = j / RS, f = j - i * RS, e = f - doff_for(E);
            sm.rows[j] = (e >= 0 && e < a.E) ? dg[(int64_t)e * G + i] : 0.0f;
        }
        __syncthreads();
    }
    rescore<E>(sm, n, G, a.E, (double)a.qmin, (double)a.qmax);
    if (wave < 2) {
        const bool want = wave == 0 ? a.want_minimax : a.want_pooled;
        if (want && sm.win_b[wave] == 0xFFFFFFFFu)
            pick_winner<E>(sm, n, wave == 0 ? TAG_MINIMAX : TAG_POOLED, wave);
    }
    __syncthreads();
    const float fqlo = (float)a.qmin, fqhi = (float)a.qmax;
    const int cp = a.want_minimax ? 0 : 1;  // the policy whose codes are written
    const float sc = half_bits_value(sm.win_b[cp]);
    if (a.codes)
        for (int i = tid; i < G; i += BLOCK) a.codes[g * G + i] = (int8_t)exact_code_range(sm.w[i], sc, fqlo, fqhi);
    if (tid == 0) {
        if (a.want_minimax) {
            a.scales[g] = (uint16_t)sm.win_b[0];
            if (a.objective) a.objective[g] = sm.win_F[0];
            if (a.flags) a.flags[g] = sm.win_flags[0] | a.flag_or;
        }
        if (a.want_pooled) {
            if (a.pscales) a.pscales[g] = (uint16_t)sm.win_b[1];
            if (a.pobjective) a.pobjective[g] = sm.win_F[1];
            if (!a.want_minimax && a.flags) a.flags[g] = sm.win_flags[1] | a.flag_or;
        }
    }
}

// The zero rule or the shortlist threshold of one policy from its smallest key M1 and runner-up
// S2: a zero binary32 value is exact (every term is normal or zero), so the lowest such pattern
// wins with value 0; otherwise every key within the ratio of M1 is rescored.  One thread per
// policy.
template <int E>
__device__ float policy_threshold(const FullArgs& a, Smem<E>& sm, int pol, uint64_t M1, uint64_t S2) {
    const float m = key_value(M1);
    if (m == 0.0f) {
        sm.win_b[pol] = key_bits(M1);
        sm.win_F[pol] = 0.0;
        sm.win_flags[pol] = (S2 != KEY_NONE && key_value(S2) == 0.0f) ? (FLAG_NEAR_TIE | FLAG_EXACT_TIE) : 0;
        return -1.0f;  // nothing to rescore
    }
    sm.win_b[pol] = 0xFFFFFFFFu;  // decided by rescoring
    return m * a.ratio;
}

// One workgroup per group: the whole grid, the shortlist from every lane's keys, the decision.
template <int E>
__device__ void screen_group(const FullArgs& a, int64_t g, Smem<E>& sm) {
    const int tid = threadIdx.x;
    float pk, cmax;
    // A workgroup starts beside others that keep the SIMDs busy with the screen, and the oldest
    // waves issue first: its staging runs at a raised wave priority, so that it joins the screen
    // soon instead of waiting for issue slots.
    __builtin_amdgcn_s_setprio(3);
    const int st = stage_group<E>(a, g, sm, pk, cmax);
    __builtin_amdgcn_s_setprio(0);
    if (st == 1) { write_bad(a, g); return; }
    if (st == 2) { if (tid == 0) queue_f64(a, g); return; }
    uint64_t mk[3], qk[3];
    screen_keys<E>(a, sm, pk, cmax, 0, 1, mk, qk);

    // ---- each policy's smallest key, its runner-up, and the shortlist
    uint64_t kv[2] = {mk[0], qk[0]};
    block_min_u64n<2>(kv, sm.redk);
    uint64_t kv2[2] = {mk[0] == kv[0] ? mk[1] : mk[0], qk[0] == kv[1] ? qk[1] : qk[0]};
    block_min_u64n<2>(kv2, sm.redk + 8);
    if (tid == 0) {
        for (int pol = 0; pol < 2; ++pol)
            if (pol == 0 ? a.want_minimax : a.want_pooled) sm.thr[pol] = policy_threshold<E>(a, sm, pol, kv[pol], kv2[pol]);
    }
    __syncthreads();
    for (int pol = 0; pol < 2; ++pol) {
        if (!(pol == 0 ? a.want_minimax : a.want_pooled)) continue;
        const uint64_t* kk = pol == 0 ? mk : qk;
        const float T = sm.thr[pol];
        if (T < 0.0f) continue;
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            if (kk[r] != KEY_NONE && key_value(kk[r]) <= T) {
                if (r == 2) sm.overflow = 1;
                else append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(kk[r]), pol == 0 ? TAG_MINIMAX : TAG_POOLED);
            }
        }
    }
    __syncthreads();
    decide_and_write<E>(a, g, sm);
}

template <int E>
__global__ __launch_bounds__(BLOCK, min_blocks_for(E)) void full_screen_kernel(FullArgs a) {
    __shared__ Smem<E> sm;
    screen_group<E>(a, (int64_t)blockIdx.x + a.group_offset, sm);
}

// List mode: the groups a.list[0 .. *a.list_count - 1], each workgroup taking every gridDim.x-th
// entry (the count is known only on the device).  Every return inside screen_group is taken by the
// whole workgroup, and the barrier keeps one group's LDS from being restaged under another's reads.
// The loop around the search needs more registers than one group does: fewer workgroups per CU
// (three at E = 4, one fewer elsewhere) keep it free of spills.
constexpr int list_blocks_for(int E) { return E == 4 ? 3 : (min_blocks_for(E) > 1 ? min_blocks_for(E) - 1 : 1); }
template <int E>
__global__ __launch_bounds__(BLOCK, list_blocks_for(E)) void full_list_kernel(FullArgs a) {
    __shared__ Smem<E> sm;
    const int cnt = *a.list_count;
    for (int k = blockIdx.x; k < cnt; k += gridDim.x) {
        screen_group<E>(a, (int64_t)a.list[k], sm);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ few groups: slices
// Below about a thousand groups one workgroup per group leaves most CUs idle, so a group's chunks
// are split over S workgroups (slices).  Slice s screens the chunks c with (c / 4) % S == s and
// leaves in its SlicePart, per policy: its smallest and second keys; every key within the ratio
// of its own smallest (up to SLICE_KEYS); and the smallest value it could not keep (a lane's third
// key within that ratio, which may hide a fourth; or its smallest value when the keys overflowed).
// The merge takes the group's smallest key over the slices: the global threshold is no larger than
// any slice's, so every key within it is stored unless a slice's unkept value lies within it too,
// which sends the group to the binary64 sweep.
template <int E>
__global__ __launch_bounds__(BLOCK, min_blocks_for(E)) void full_slice_kernel(FullArgs a) {
    __shared__ Smem<E> sm;
    const int S = a.slices, tid = threadIdx.x;
    const int64_t g = (int64_t)blockIdx.x / S;
    const int slice = (int)(blockIdx.x % S);
    SlicePart& P = a.parts[blockIdx.x];
    float pk, cmax;
    __builtin_amdgcn_s_setprio(3);  // as in the one-workgroup path: staging beside busy waves
    const int st = stage_group<E>(a, g, sm, pk, cmax);
    __builtin_amdgcn_s_setprio(0);
    if (st != 0) return;  // the merge stages the group again
    uint64_t mk[3], qk[3];
    screen_keys<E>(a, sm, pk, cmax, slice, S, mk, qk);
    uint64_t kv[2] = {mk[0], qk[0]};
    block_min_u64n<2>(kv, sm.redk);
    uint64_t kv2[2] = {mk[0] == kv[0] ? mk[1] : mk[0], qk[0] == kv[1] ? qk[1] : qk[0]};
    block_min_u64n<2>(kv2, sm.redk + 8);
#pragma unroll
    for (int pol = 0; pol < 2; ++pol) {
        const uint64_t* kk = pol == 0 ? mk : qk;
        const float T = key_value(kv[pol]) * a.ratio;  // 0 when the slice's smallest value is 0
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            if (kk[r] != KEY_NONE && key_value(kk[r]) <= T) {
                if (r == 2) {
                    atomicMin(&sm.ov_bits[pol], __float_as_uint(key_value(kk[r])));
                } else {
                    const int j = atomicAdd(&sm.n_key[pol], 1);
                    if (j < SLICE_KEYS) P.keys[pol][j] = kk[r];
                }
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        P.status = 0;
#pragma unroll
        for (int pol = 0; pol < 2; ++pol) {
            const int n = sm.n_key[pol];
            P.n[pol] = (uint32_t)(n < SLICE_KEYS ? n : SLICE_KEYS);
            // keys lost to the list's capacity: no stored value above the slice's smallest is sure
            P.ov[pol] = n > SLICE_KEYS ? __float_as_uint(key_value(kv[pol])) : sm.ov_bits[pol];
            P.m1[pol] = kv[pol];
            P.s2[pol] = kv2[pol];
        }
    }
}

template <int E>
__global__ __launch_bounds__(BLOCK) void full_merge_kernel(FullArgs a) {
    __shared__ Smem<E> sm;
    const int S = a.slices, tid = threadIdx.x;
    const int64_t g = blockIdx.x;
    float pk, cmax;
    const int st = stage_group<E>(a, g, sm, pk, cmax);
    if (st == 1) { write_bad(a, g); return; }
    if (st == 2) { if (tid == 0) queue_f64(a, g); return; }
    const SlicePart* parts = a.parts + g * S;
    const int lane = tid & 63, wave = tid >> 6;
    float* pre = reinterpret_cast<float*>(sm.pairF);  // [2][64]: inclusive prefix sums of the key counts
    if (wave < 2 && (wave == 0 ? a.want_minimax : a.want_pooled)) {
        // wave 0 minimax, wave 1 pooled: lane sl < S holds slice sl's smallest and second keys,
        // its unkept value and its count of stored keys (S <= 32)
        const int pol = wave;
        const bool in = lane < S;
        const uint64_t m = in ? parts[lane].m1[pol] : KEY_NONE;
        const uint64_t m2 = in ? parts[lane].s2[pol] : KEY_NONE;
        const uint32_t ov = in ? parts[lane].ov[pol] : 0xFFFFFFFFu;
        const float cnt = in ? (float)parts[lane].n[pol] : 0.0f;  // at most 128: exact
        // the group's smallest key and its runner-up (the slices screen disjoint patterns, so
        // the keys are distinct)
        const uint64_t M1 = wave_min_u64(m);
        const uint64_t S2 = wave_min_u64(m == M1 ? m2 : m);
        float T = 0.0f;
        if (lane == 0) T = policy_threshold<E>(a, sm, pol, M1, S2);
        T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(T)));
        if (lane == 0) sm.thr[pol] = T;
        // a slice's unkept value within the threshold sends the group to the binary64 sweep
        if (T >= 0.0f && in && ov != 0xFFFFFFFFu && __uint_as_float(ov) <= T) sm.overflow = 1;
        pre[pol * 64 + lane] = wave_inclusive_sum_f32(cnt);
    }
    __syncthreads();
    // every stored key within the threshold joins the shortlist.  The stored keys of both policies
    // form one index range, minimax first (one round of loads): entry j of a policy's keys, in
    // slice order, is key j - (keys before slice sl) of the slice sl it falls in, found by a binary
    // search of the prefix sums
    int tot[2];
#pragma unroll
    for (int pol = 0; pol < 2; ++pol) {
        const bool live = (pol == 0 ? a.want_minimax : a.want_pooled) && sm.thr[pol] >= 0.0f;
        tot[pol] = live ? (int)pre[pol * 64 + S - 1] : 0;
    }
    for (int j = tid; j < tot[0] + tot[1]; j += BLOCK) {
        const int pol = j < tot[0] ? 0 : 1, jj = pol == 0 ? j : j - tot[0];
        const float* pp = pre + pol * 64;
        int lo = 0, hi = S - 1;  // pp[S - 1] = tot[pol] > jj
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((int)pp[mid] > jj) hi = mid;
            else lo = mid + 1;
        }
        const int k = jj - (lo == 0 ? 0 : (int)pp[lo - 1]);
        const uint64_t key = parts[lo].keys[pol][k];
        if (key_value(key) <= sm.thr[pol])
            append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(key), pol == 0 ? TAG_MINIMAX : TAG_POOLED);
    }
    __syncthreads();
    decide_and_write<E>(a, g, sm);
}

// ------------------------------------------------------------------ binary64 sweep
// Every scale in binary64, each environment summed in the definition's order; the lexicographic
// (value, bits) minimum and the runner-up value give the answer with no screen at all.  For the
// groups whose binary32 screen could not be guaranteed or was inconclusive (flat objectives with
// thousands of exactly tied patterns among them).  One 1,024-thread workgroup per group, one scale
// per thread at a time: each weight's code, residual and square once, then its term added to the
// E environments' running sums, so that every sum still runs i = 0..G-1 with every operation
// rounded on its own.
constexpr int F64_BLOCK = 1024, F64_WAVES = F64_BLOCK / 64;

template <int E>
struct F64Smem {
    float w[GMAX];
    float dt[GMAX * E];  // [i][e]
    double rv[F64_WAVES], rv2[F64_WAVES], pv[F64_WAVES], pv2[F64_WAVES];
    uint32_t rb[F64_WAVES], pb[F64_WAVES];
};

__device__ __forceinline__ bool lex_less(double v, uint32_t b, double v2, uint32_t b2) {
    return v < v2 || (v == v2 && b < b2);
}

// Fold (v, b) into a (best, best bits, second value) triple.
__device__ __forceinline__ void fold(double v, uint32_t b, double& bv, uint32_t& bb, double& sv) {
    if (lex_less(v, b, bv, bb)) { sv = bv; bv = v; bb = b; }
    else if (v < sv) sv = v;
}
// Merge another triple: the lexicographic best of the two bests, and the smallest value of the rest.
__device__ __forceinline__ void merge3(double v, uint32_t b, double s, double& bv, uint32_t& bb, double& sv) {
    fold(v, b, bv, bb, sv);
    sv = s < sv ? s : sv;
}
// The triple over the 64 lanes of a wave (every lane ends with it).
__device__ __forceinline__ void wave_merge3(double& bv, uint32_t& bb, double& sv) {
#pragma unroll
    for (int k = 0; k < 6; ++k) {  // lane distances 32, 16, .., 1
        const int o = 32 >> k;
        const double v = lane_xor(bv, o), s = lane_xor(sv, o);
        const uint32_t b = lane_xor(bb, o);
        merge3(v, b, s, bv, bb, sv);
    }
}

template <int E>
__device__ void f64_group(const FullArgs& a, int64_t g, F64Smem<E>& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, G = a.G;
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);
    for (int i = tid; i < G; i += F64_BLOCK) sm.w[i] = wg[i];
    for (int j = tid; j < E * G; j += F64_BLOCK) {
        const int e = j / G, i = j - e * G;
        sm.dt[i * E + e] = e < a.E ? dg[j] : 0.0f;
    }
    __syncthreads();
    const double qlo = (double)a.qmin, qhi = (double)a.qmax;
    double bF = __builtin_inf(), sF = __builtin_inf(), bP = __builtin_inf(), sP = __builtin_inf();
    uint32_t bFb = 0xFFFFFFFFu, bPb = 0xFFFFFFFFu;
    for (uint32_t b = BITS_FIRST + tid; b <= BITS_LAST; b += F64_BLOCK) {
        const double s = (double)half_bits_value(b), inv = 1.0 / s;
        double f[E];
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = 0.0;
        for (int i = 0; i < G; ++i) {
            // the operations of env_error_f64_n for weight i, shared by the environments
            const double wi = (double)sm.w[i];
            double r = __builtin_rint(wi * inv);
            r = r < qlo ? qlo : (r > qhi ? qhi : r);
            const double sq = s * r;
            const double t = wi - sq;
            const double t2 = t * t;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double term = (double)sm.dt[i * E + e] * t2;
                f[e] = f[e] + term;
            }
        }
        double F = f[0], P = f[0];
#pragma unroll
        for (int e = 1; e < E; ++e) {
            F = f[e] > F ? f[e] : F;
            P = P + f[e];
        }
        P = P / (double)a.E;
        fold(F, b, bF, bFb, sF);
        fold(P, b, bP, bPb, sP);
    }
    wave_merge3(bF, bFb, sF);
    wave_merge3(bP, bPb, sP);
    if (lane == 0) {
        sm.rv[wave] = bF; sm.rb[wave] = bFb; sm.rv2[wave] = sF;
        sm.pv[wave] = bP; sm.pb[wave] = bPb; sm.pv2[wave] = sP;
    }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < F64_WAVES; ++k) {
            merge3(sm.rv[k], sm.rb[k], sm.rv2[k], sm.rv[0], sm.rb[0], sm.rv2[0]);
            merge3(sm.pv[k], sm.pb[k], sm.pv2[k], sm.pv[0], sm.pb[0], sm.pv2[0]);
        }
    }
    __syncthreads();
    const uint32_t win = a.want_minimax ? sm.rb[0] : sm.pb[0];
    if (a.codes) {
        const float sc = half_bits_value(win);
        for (int i = tid; i < G; i += F64_BLOCK)
            a.codes[g * G + i] = (int8_t)exact_code_range(sm.w[i], sc, (float)a.qmin, (float)a.qmax);
    }
    if (tid == 0) {
        const uint8_t fF = FLAG_FP64_SWEEP | (sm.rv2[0] == sm.rv[0] ? (FLAG_NEAR_TIE | FLAG_EXACT_TIE) : 0);
        const uint8_t fP = FLAG_FP64_SWEEP | (sm.pv2[0] == sm.pv[0] ? (FLAG_NEAR_TIE | FLAG_EXACT_TIE) : 0);
        if (a.want_minimax) {
            a.scales[g] = (uint16_t)sm.rb[0];
            if (a.objective) a.objective[g] = sm.rv[0];
            if (a.flags) a.flags[g] = fF | a.flag_or;
        }
        if (a.want_pooled) {
            if (a.pscales) a.pscales[g] = (uint16_t)sm.pb[0];
            if (a.pobjective) a.pobjective[g] = sm.pv[0];
            if (!a.want_minimax && a.flags) a.flags[g] = fP | a.flag_or;
        }
    }
    __syncthreads();
}

template <int E>
__global__ __launch_bounds__(F64_BLOCK) void full_f64_kernel(FullArgs a) {
    __shared__ F64Smem<E> sm;
    const int cnt = *a.fb_count;
    for (int k = blockIdx.x; k < cnt; k += gridDim.x) f64_group<E>(a, (int64_t)a.fb_list[k], sm);
}

__global__ void full_zero_kernel(int32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

template <int E>
hipError_t launch_e(const FullArgs& a_in, int64_t n_groups, hipStream_t st) {
    FullArgs a = a_in;
    hipLaunchKernelGGL(full_zero_kernel, dim3(1), dim3(64), 0, st, a.fb_count);
    // few groups: S slices per group, about 2,048 workgroups in all, at most one chunk per wave
    constexpr int S_MAX = nchunk_for(E) / 4 < 32 ? nchunk_for(E) / 4 : 32;
    int S = 1;
    if (n_groups < 1024 && a.parts && !a.list) {
        S = (int)((2048 + n_groups - 1) / n_groups);
        S = S > S_MAX ? S_MAX : S;
        while (S > 1 && n_groups * S > SLICE_PARTS) --S;
    }
    a.slices = S;
    if (a.list) {
        // as many workgroups as stay resident (fewer when the list cannot be that long)
        const int64_t cap = 256 * list_blocks_for(E);
        const int64_t nb = n_groups < cap ? n_groups : cap;
        hipLaunchKernelGGL(full_list_kernel<E>, dim3((unsigned)nb), dim3(BLOCK), 0, st, a);
    } else if (S > 1) {
        hipLaunchKernelGGL(full_slice_kernel<E>, dim3((unsigned)(n_groups * S)), dim3(BLOCK), 0, st, a);
        hipLaunchKernelGGL(full_merge_kernel<E>, dim3((unsigned)n_groups), dim3(BLOCK), 0, st, a);
    } else {
        const int64_t step = 1ll << 30;  // grid.x is limited to 2^31 - 1 blocks
        for (int64_t off = 0; off < n_groups; off += step) {
            FullArgs b = a;
            b.group_offset = off;
            const int64_t n = n_groups - off < step ? n_groups - off : step;
            hipLaunchKernelGGL(full_screen_kernel<E>, dim3((unsigned)n), dim3(BLOCK), 0, st, b);
        }
    }
    const int fb_blocks = (int)(n_groups < 1024 ? n_groups : 1024);
    hipLaunchKernelGGL(full_f64_kernel<E>, dim3(fb_blocks), dim3(F64_BLOCK), 0, st, a);
    return hipGetLastError();
}

}  // namespace full

// The shortlist ratio for G weights, codes in [qmin, qmax] and E environments: (1 + hi)/(1 - lo)
// with the bounds of the header, widened by 8 u for the roundings of the threshold itself and
// rounded up to binary32.
float fullgrid_ratio(int G, int qmin, int qmax, int E) {
    const double u = 0x1p-24;
    const double X = (double)(-qmin > qmax ? -qmin : qmax) + 0.5;
    // the matrix cores' accumulation is taken at one binary32 ulp (2u) per step, whatever its
    // rounding of the one fused product and sum
    const double acc_u = full::use_mfma(pad_envs(E)) ? 2.0 * u : u;
    const double hi = (1.0 + 1.0001 * (G * acc_u + (3 + E) * u)) * (1.0 + 16.001 * X * u) - 1.0;
    const double lo = 1.0001 * (G * acc_u + (3 + E) * u);
    const double r = (1.0 + hi) / (1.0 - lo) * (1.0 + 8.0 * u);
    float f = (float)r;
    if ((double)f < r) f = nextafterf(f, 2.0f);
    return f;
}

hipError_t launch_fullgrid(const FullArgs& a_in, int E, int64_t n_groups, hipStream_t st) {
    FullArgs a = a_in;
    a.E = E;
    if (n_groups == 0) return hipSuccess;
    switch (pad_envs(E)) {
        case 1: return full::launch_e<1>(a, n_groups, st);
        case 2: return full::launch_e<2>(a, n_groups, st);
        case 4: return full::launch_e<4>(a, n_groups, st);
        case 8: return full::launch_e<8>(a, n_groups, st);
        case 16: return full::launch_e<16>(a, n_groups, st);
        case 32: return full::launch_e<32>(a, n_groups, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cqk
