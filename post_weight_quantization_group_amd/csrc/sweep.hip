// Exhaustive FP16 scale sweep for gfx950.
//
// For every group the kernel decides among all 31,743 positive finite binary16
// scales (CliffQuant repository README, "What CliffQuant changes": the
// independent reference enumerates every one of them; model card
// "Verification").  It considers every pattern up to the top pattern b_top, the
// smallest scale >= 2 max|w|: from there on every code is 0, the objective is
// the same binary64 value at every pattern, and b_top wins all those exact ties
// by the lower-bit-pattern rule (about 40% of the grid on typical weights).
// Work split: one 256-thread workgroup per group; weights and diagonals are
// staged in LDS, sorted by a clip key; each wave takes chunks of 64*NS
// consecutive scale patterns, NS = 2 per lane, with the per-environment sums
// in registers.  Within a chunk the sorted weights fall
// into four consecutive ranges: code 0 at every scale of the chunk (their
// terms d w^2 enter as one prefix sum), never clipped, possibly clipped, and
// code 7 or -8 throughout (no quotient needed).  Chunks are taken outward from
// the chunk of max|w|/9, and a chunk whose proven lower bound exceeds the
// best value already screened is skipped (screen_keys): branch and bound, with
// the outputs of the full screen.
//
// Exactness.  The sweep runs in binary32 with a proven error bound and is a
// screen only:
//   * weights are pre-scaled by 2^k (max |w'| in [1,2)) and scales by the same
//     2^k -- the quotient and the codes are unchanged and every error term
//     stays in the normal binary32 range (groups for which that cannot be
//     guaranteed go to the binary64 sweep);
//   * the code uses x = w' * inv with inv within 1 ulp of 1/s' (hardware
//     reciprocal plus a Newton step), so |x~ - x| <= 3u|x|; it can differ from
//     the exact code only within 26 u of a half-integer (|x| <= 8.5), which
//     raises that term by at most 208 u (u = 2^-24) and never lowers it;
//   * e = fma(-s', q, w') is exact unless clipped (then one rounding), and
//     every term meets at most 129 more roundings on its way into the sum
//     (e^2, then one fma per later weight, the code-0 prefix sums included),
//     which puts the sum within (1 +- u)^131 of the exact value.
//   So the binary32 value F~ satisfies (1-131u) F <= F~ <= (1+340u) F, and
//   every scale whose F~ is within the factor 1.00004 (> 1 + 472u) of the smallest F~ is
//   rescored in binary64 (same summation order as the definition's plain
//   sequential sum), which decides the winner and the lower-bit-pattern tie.
//   When the smallest F~ is 0 the group's zero-error scales are exact and the
//   lowest such pattern wins directly.  A lane keeps its best three scales; if
//   its third is inside the bound (it may have dropped a fourth), or more than
//   256 scales survive, the group is queued for the binary64 sweep.
#include "device.h"
#include "search_args.h"

namespace cqk {

// Scales per lane per chunk, and workgroups per CU.  Two scales per lane (chunks of 128
// patterns) keep the chunks narrow, so fewer weights change code within one and the chunk bounds
// are tight, and leave room for many waves per SIMD: the screen's dependent LDS loads and
// binary64 chains need the latency hiding more than they suffer from the few spills this costs.
// Measured on gfx950 with chunk skipping: 128-pattern chunks beat 256 by 7-8% at E = 4, 64
// (one scale per lane) lose 30%.
constexpr int ns_for(int E) { return 2; }
constexpr int min_blocks_for(int E) { return E <= 2 ? 8 : (E == 4 ? 7 : (E == 8 ? 5 : (E == 16 ? 4 : 2))); }
constexpr int CAP = 256;                     // shortlist capacity per group
constexpr float SCREEN_RATIO = 1.00004f;
constexpr uint8_t TAG_MINIMAX = 1, TAG_POOLED = 2;

template <int E>
struct SweepSmem {
    float w[G];
    __align__(16) float dt[G * E];    // [i][e], definition order (rescoring)
    // screen order (sort by the clip key, see stage_group)
    __align__(16) float ws[G];        // pre-scaled weights
    __align__(16) float ds[G * E];    // their diagonals [r][e]
    float ks[G];                      // clip keys, ascending
    float qs[G];                      // the code a weight takes once it is clipped (7 or -8)
    // per wave, per chunk (screen_keys): the code a weight keeps over the chunk (127 if it
    // changes), and the list of weights whose code changes, never-clipped ones first
    int8_t qc[4][G];
    uint8_t vlist[4][G];
    int8_t rq[32][G];                 // rescoring: the codes of a batch of shortlisted scales
    __align__(16) float kz[(G + 1) * E];  // kz[m][e]: binary32 sum of d w'^2 over the first m weights
    float redf[4 * 5];
    uint64_t redk[8];
    uint32_t cand_b[CAP];
    uint8_t cand_tag[CAP];
    __align__(16) double cand_F[CAP];
    double cand_P[CAP];
    __align__(16) double pairF[BLOCK];
    int n_cand;
    int overflow;
    // the screen's work counters: chunks handed out upwards from c_start and downwards from
    // c_start - 1, and the limits beyond which every chunk is known to be skippable
    int next_up, next_down;
    int lim_up, lim_down;
    uint32_t win_b[2];
    double win_F[2];
    uint8_t win_flags[2];
    uint32_t ovbits;
    uint64_t mrg_m1[2];
    uint32_t b_top;                   // last pattern screened (top_pattern)
    int c_start;                      // the chunk screened first (around max|w|/9)
    uint32_t u_bits[2];               // smallest minimax / pooled binary32 value screened so far
};

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

// Weights [i0, i1) whose code is the clipped one, qs (7 or -8), at every scale of the chunk:
// e = fma(-s', q, w'), e^2, one fma per environment; no quotient.
template <int E, int NS>
__device__ __forceinline__ void sweep_range_clipped(const float* __restrict__ ws, const float* __restrict__ qs,
                                                    const float* __restrict__ ds, int i0, int i1,
                                                    const float (&nsv)[NS], float (&acc)[NS][E]) {
#pragma unroll 2
    for (int i = i0; i < i1; ++i) {
        const float wi = ws[i], qi = qs[i];
        float di[E];
#pragma unroll
        for (int e = 0; e < E; ++e) di[e] = ds[i * E + e];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const float ev = __builtin_fmaf(nsv[t], qi, wi);
            const float e2 = ev * ev;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[t][e] = __builtin_fmaf(di[e], e2, acc[t][e]);
        }
    }
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The weights of [r0, G) that keep one code q over the chunk in closed form: the fixed-code
// range [m_c, G) (q = 7 or -8) and, below m_c, those with qc != 127.  They add
// Q_e(s) = A_e - 2 B_e s + C_e s^2 with A = sum d w'^2, B = sum d w' q, C = sum d q^2 (all
// terms >= 0: q is 0 or has the sign of w').
// The sums run in binary64, 64/E lanes per environment and a butterfly over those lanes; each
// lane returns the sums of environment lane % E.  Q is used only when its binary64 error, at
// most 2^-45 (A + 2 B s + C s^2) (fewer than 140 roundings of 2^-53 along any path), is below
// 2^-31 of min Q over the chunk [s_lo, s_hi]: then Q~ = Q (1 +- 2^-31) at every scale of the
// chunk and the screen's bound is unchanged.  Otherwise the range is summed term by term.
// qlo is the computed min of Q over the chunk (Q at the clamped vertex; A when C = 0); when Q is
// used, every exact Q over the chunk is at least qlo (1 - 2^-31).
template <int E>
__device__ __forceinline__ bool fixed_code_sums(const SweepSmem<E>& sm, int r0, int m_c, float s_lo, float s_hi,
                                                double& A, double& B, double& C, double& qlo) {
    constexpr int P = 64 / E;  // lanes per environment
    const int lane = threadIdx.x & 63, e = lane % E, wave = threadIdx.x >> 6;
    A = 0.0; B = 0.0; C = 0.0;
    for (int r = r0 + lane / E; r < G; r += P) {
        const int qcode = r < m_c ? (int)sm.qc[wave][r] : 0;
        if (qcode == 127) continue;  // its code changes within the chunk: summed term by term
        const double wv = (double)sm.ws[r], dv = (double)sm.ds[r * E + e];
        const double q = r < m_c ? (double)qcode : (double)sm.qs[r];
        const double dw = dv * wv;  // exact (24 + 24 bits)
        A = __builtin_fma(dw, wv, A);
        B = __builtin_fma(dw, q, B);
        C = __builtin_fma(dv, q * q, C);
    }
#pragma unroll
    for (int o = E; o < 64; o <<= 1) {
        A += lane_xor(A, o);
        B += lane_xor(B, o);
        C += lane_xor(C, o);
    }
    bool ok = true;
    qlo = A;
    if (C > 0.0) {
        const double lo = (double)s_lo, hi = (double)s_hi;
        const double M = __builtin_fma(hi, __builtin_fma(hi, C, 2.0 * B), A);
        const double r0 = __builtin_amdgcn_rcp(C);
        double v = B * __builtin_fma(r0, __builtin_fma(-C, r0, 1.0), r0);  // the vertex, to ~2^-50
        v = v < lo ? lo : (v > hi ? hi : v);
        const double qmin = __builtin_fma(v, __builtin_fma(v, C, -2.0 * B), A);
        ok = M * 0x1p-13 <= qmin;  // 2^-45 M <= 2^-32 qmin, with room for the rounded vertex
        qlo = qmin;
    }
    return __ballot(!ok) == 0;
}

// The listed weights vl[i0..i1) of the screen order against the lane's NS scales, with the
// per-environment sums in registers: q = rne(w' * (1/s')) (clipped when CLIP), e = fma(-s', q, w'),
// e^2, then one fma per environment.  The weight and its E diagonals are LDS broadcasts shared by
// all NS scales of the lane.
template <int E, int NS, bool CLIP>
__device__ __forceinline__ void sweep_list(const float* __restrict__ ws, const float* __restrict__ ds,
                                           const uint8_t* __restrict__ vl, int i0, int i1,
                                           const float (&nsv)[NS], const float (&inv)[NS], float (&acc)[NS][E]) {
#pragma unroll 2
    for (int i = i0; i < i1; ++i) {
        const int r = vl[i];
        const float wi = ws[r];
        float di[E];
#pragma unroll
        for (int e = 0; e < E; ++e) di[e] = ds[r * E + e];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const float x = wi * inv[t];
            float q = __builtin_rintf(x);
            if (CLIP) q = __builtin_amdgcn_fmed3f(q, -8.0f, 7.0f);
            const float ev = __builtin_fmaf(nsv[t], q, wi);
            const float e2 = ev * ev;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[t][e] = __builtin_fmaf(di[e], e2, acc[t][e]);
        }
    }
}

// Which weights of [m_z, m_c) keep one code over the chunk's scales [s_lo, s_hi]: the codes at
// both ends agree (codes are monotone in s).  The quotients use reciprocals within 1 ulp, so
// x~ = x (1 +- 3u); a code is taken only when x~ is farther than 2^-20 max(1, |x~|) from a
// half-integer, where it equals the exact code.  Anything closer counts as changing, which is
// always safe.  Writes the kept code to qc (127 when it changes) and lists the weights whose code
// changes (all of them when `all`), in screen order, so that the never-clipped ones (r < m_u)
// come first; returns the list length and their number in n_u.
template <int E>
__device__ __forceinline__ int classify_chunk(SweepSmem<E>& sm, int m_z, int m_u, int m_c, float inv_lo, float inv_hi,
                                              bool all, int& n_u) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
    int n = 0;
    n_u = 0;
    for (int base = m_z; base < m_c; base += 64) {
        const int r = base + lane;
        bool var = false;
        if (r < m_c) {
            var = all;
            if (!all) {
                const float w = sm.ws[r];
                const float xl = w * inv_lo, xh = w * inv_hi;
                const float rl = __builtin_rintf(xl), rh = __builtin_rintf(xh);
                const float ml = 0.5f - 0x1p-20f * fmaxf(1.0f, fabsf(xl));
                const float mh = 0.5f - 0x1p-20f * fmaxf(1.0f, fabsf(xh));
                const float ql = __builtin_amdgcn_fmed3f(rl, -8.0f, 7.0f), qh = __builtin_amdgcn_fmed3f(rh, -8.0f, 7.0f);
                var = ql != qh || fabsf(xl - rl) >= ml || fabsf(xh - rh) >= mh;
                sm.qc[wave][r] = var ? (int8_t)127 : (int8_t)ql;
            }
        }
        const uint64_t m = __ballot(var);
        if (var) sm.vlist[wave][n + __popcll(m & below)] = (uint8_t)r;
        n += (int)__popcll(m);
        n_u += (int)__popcll(__ballot(var && r < m_u));
    }
    __builtin_amdgcn_wave_barrier();
    return n;
}

// binary64 rescoring of the first n shortlist entries: cand_F = max_e F_e,
// cand_P = (sum_e F_e)/E, each F_e summed in the definition's order.
template <int E>
__device__ void rescore(SweepSmem<E>& sm, int n, int E_real) {
    constexpr int PER = BLOCK / E < 32 ? BLOCK / E : 32;
    const int t = threadIdx.x;
    for (int base = 0; base < n; base += PER) {
        const int nb = min(PER, n - base);
        // the batch's codes from all threads first; each (scale, environment) sum then runs the
        // definition's operations in its order
        for (int j = t; j < nb * G; j += BLOCK) {
            const int c = j / G, i = j % G;
            sm.rq[c][i] = (int8_t)exact_code(sm.w[i], half_bits_value(sm.cand_b[base + c]));
        }
        __syncthreads();
        if (t < nb * E) {
            const int c = t / E, e = t % E;
            const double s = (double)half_bits_value(sm.cand_b[base + c]);
            sm.pairF[t] = env_error_codes_f64(sm.w, sm.dt + e, E, sm.rq[c], s);
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

// One wave: the lexicographic (value, bits) winner among shortlist entries with `tag`, the
// number of such entries and whether another pattern has the same value.  Each lane takes every
// 64th entry; the lanes' winners meet in a DPP reduction under the same order.  Lane 0 writes.
template <int E>
__device__ void pick_winner(SweepSmem<E>& sm, int n, uint8_t tag, int slot) {
    const int lane = threadIdx.x & 63;
    uint32_t bb = 0xFFFFFFFFu;
    double bF = __builtin_inf();
    int count = 0;
    for (int j = lane; j < n; j += 64) {
        if (!(sm.cand_tag[j] & tag)) continue;
        const double v = tag == TAG_MINIMAX ? sm.cand_F[j] : sm.cand_P[j];
        const uint32_t b = sm.cand_b[j];
        ++count;
        if (v < bF || (v == bF && b < bb)) { bF = v; bb = b; }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double v = lane_xor(bF, o);
        const uint32_t b = lane_xor(bb, o);
        if (v < bF || (v == bF && b < bb)) { bF = v; bb = b; }
        count += (int)lane_xor((uint32_t)count, o);
    }
    bool tie = false;
    for (int j = lane; j < n; j += 64) {
        if (!(sm.cand_tag[j] & tag)) continue;
        const double v = tag == TAG_MINIMAX ? sm.cand_F[j] : sm.cand_P[j];
        if (v == bF && sm.cand_b[j] != bb) tie = true;
    }
    tie = __ballot(tie) != 0;
    if (lane == 0) {
        sm.win_b[slot] = bb;
        sm.win_F[slot] = bF;
        sm.win_flags[slot] = (uint8_t)((count > 1 ? FLAG_NEAR_TIE : 0) | (tie ? FLAG_EXACT_TIE : 0));
    }
}

// The smallest pattern whose scale is at least 2 max|w| (BITS_LAST when there is none).  From
// there on every code is 0 (|w/s| <= 1/2 rounds to 0), so every residual is w itself and the
// objective is the same binary64 value at every larger pattern: those patterns tie with this one
// and lose to it by the lower-bit-pattern rule.  The sweep stops here.
__device__ __forceinline__ uint32_t top_pattern(float wmax) {
    const float t = 2.0f * wmax;
    if (!(t <= 65504.0f)) return BITS_LAST;
    uint32_t b = f32_to_half_bits_rne(t);
    b = b < BITS_FIRST ? BITS_FIRST : (b > BITS_LAST ? BITS_LAST : b);
    while (b > BITS_FIRST && half_bits_value(b - 1) >= t) --b;
    while (b < BITS_LAST && half_bits_value(b) < t) ++b;
    return b;
}

// Flags of a winner at the top pattern: every larger pattern ties with it exactly.
__device__ __forceinline__ uint8_t top_tie_flags(uint32_t win, uint32_t b_top) {
    return (win == b_top && b_top < BITS_LAST) ? (uint8_t)(FLAG_NEAR_TIE | FLAG_EXACT_TIE) : (uint8_t)0;
}

__device__ __forceinline__ void append_cand(uint32_t* cb, uint8_t* ct, int* n, uint32_t b, uint8_t tag) {
    const int j = atomicAdd(n, 1);
    if (j < CAP) { cb[j] = b; ct[j] = tag; }
}

// ------------------------------------------------------------------ stages of one group
// Stage w (definition order), the pre-scaled copy and d; check the inputs.  Returns 0 when the
// binary32 screen can run, 1 for bad input, 2 when the group lies outside the screen's
// guaranteed range.  The result is the same in every workgroup that stages the same group.
template <int E>
__device__ int stage_group(const SweepArgs& a, int64_t g, SweepSmem<E>& sm, float& pk_out, float& wmax_out) {
    const int tid = threadIdx.x;
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);
    // environments a.E..E-1 are zero padding
    if (tid < G) sm.w[tid] = wg[tid];
    for (int j = tid; j < E * G; j += BLOCK) sm.dt[(j % G) * E + j / G] = j / G < a.E ? dg[j] : 0.0f;
    __syncthreads();
    float bad = 0.0f, aw = 0.0f, wnz = __builtin_inff(), dmx = 0.0f, dnz = __builtin_inff();
    if (tid < G) {
        const float v = sm.w[tid];
        if (!__builtin_isfinite(v)) bad = 1.0f;
        aw = fabsf(v);
        if (aw > 0.0f) wnz = aw;
    }
    for (int j = tid; j < E * G; j += BLOCK) {
        const float v = sm.dt[j];
        if (!(v >= 0.0f) || !__builtin_isfinite(v)) bad = 1.0f;
        else {
            dmx = fmaxf(dmx, v);
            if (v > 0.0f) dnz = fminf(dnz, v);
        }
    }
    float red[5] = {bad, aw, -wnz, dmx, -dnz};  // minima as maxima of negations
    block_max_fn<5>(red, sm.redf);
    if (red[0] != 0.0f) return 1;
    const float wmax = red[1], wmin_nz = -red[2], dmax = red[3], dmin_nz = -red[4];

    // power-of-two pre-scaling and the no-underflow / no-overflow guarantee
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
    if (tid == 0) {
        sm.n_cand = 0;
        sm.overflow = 0;
        sm.next_up = 0;
        sm.next_down = 0;
        sm.lim_up = 0x7FFFFFFF;
        sm.lim_down = -1;
        const uint32_t b_top = top_pattern(wmax);
        sm.b_top = b_top;
        // the screen starts at the chunk of max|w|/9: the minimax optimum usually lies a little
        // below the AbsMax scale max|w|/7 (clipping the largest weight slightly pays), and
        // starting there screened 8% fewer chunks than starting at max|w|/7
        uint32_t b_a = f32_to_half_bits_rne(wmax * (1.0f / 9.0f));
        b_a = b_a < BITS_FIRST ? BITS_FIRST : (b_a > b_top ? b_top : b_a);
        sm.c_start = (int)((b_a - BITS_FIRST) / (uint32_t)(64 * ns_for(E)));
        sm.u_bits[0] = 0x7F800000u;
        sm.u_bits[1] = 0x7F800000u;
    }
    // Screen order: ascending clip key K = w'/6.5 (w' > 0) or |w'|/7.5 (otherwise), ties by
    // index.  For any chunk of scales [s_lo, s_hi], the weights whose code is 0 throughout, those
    // that never clip, those that may clip and those whose code is 7 or -8 throughout are then
    // four consecutive ranges of this order (screen_keys).
    // Scratch until the shortlist: the keys made unique as (key bits, index), which order as
    // (key, index) since keys are >= 0, and the partial ranks.
    uint64_t* ck = reinterpret_cast<uint64_t*>(sm.pairF);
    int* rk = reinterpret_cast<int*>(sm.cand_F);
    float wv = 0.0f, key = 0.0f;
    if (tid < G) {
        wv = sm.w[tid] * pk;
        key = wv > 0.0f ? wv * (1.0f / 6.5f) : fabsf(wv) * (1.0f / 7.5f);  // +0 for a zero weight
        ck[tid] = ((uint64_t)__float_as_uint(key) << 7) | (uint64_t)tid;
    }
    __syncthreads();
    {
        // rank = number of weights ordered before this one; each half of the block counts over
        // one half of the keys
        const int i = tid & (G - 1), h = tid >> 7;
        const uint64_t ki = ck[i];
        const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(ck + (G / 2) * h);
        int cnt = 0;
#pragma unroll 8
        for (int q = 0; q < G / 4; ++q) {
            const ulonglong2 v = k2[q];
            cnt += v.x < ki ? 1 : 0;
            cnt += v.y < ki ? 1 : 0;
        }
        rk[tid] = cnt;
    }
    __syncthreads();
    if (tid < G) {
        const int rank = rk[tid] + rk[tid + G];
        sm.ws[rank] = wv;
        sm.ks[rank] = key;
        sm.qs[rank] = wv > 0.0f ? 7.0f : -8.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) sm.ds[rank * E + e] = sm.dt[tid * E + e];
    }
    __syncthreads();
    // kz[m][e]: the code-0 terms d w'^2 (w'^2 rounded, then the product) of the first m weights
    // of the screen order, one wave per environment: lane l adds the terms of weights 2l and
    // 2l + 1, then an inclusive scan over the lanes.  Every term meets at most 10 roundings (a
    // chunk starts its sums from kz of its code-0 range).
    for (int e = tid >> 6; e < E; e += BLOCK / 64) {
        const int l = tid & 63;
        const float w0 = sm.ws[2 * l], w1 = sm.ws[2 * l + 1];
        const float t0 = sm.ds[(2 * l) * E + e] * (w0 * w0);
        const float t1 = sm.ds[(2 * l + 1) * E + e] * (w1 * w1);
        const float x = wave_inclusive_sum_f32(t0 + t1);
        sm.kz[(2 * l + 1) * E + e] = lane_prev(x) + t0;  // lane 0 adds 0
        sm.kz[(2 * l + 2) * E + e] = x;
        if (l == 0) sm.kz[e] = 0.0f;
    }
    __syncthreads();
    pk_out = pk;
    wmax_out = wmax;
    return 0;
}

__device__ __forceinline__ void write_bad(const SweepArgs& a, int64_t g) {
    const int tid = threadIdx.x;
    if (tid < G && a.codes) a.codes[g * G + tid] = 0;
    if (tid == 0) {
        if (a.scales) a.scales[g] = 0;
        if (a.objective) a.objective[g] = __builtin_nan("");
        if (a.pscales) a.pscales[g] = 0;
        if (a.pobjective) a.pobjective[g] = __builtin_nan("");
        if (a.flags) a.flags[g] = FLAG_BAD_INPUT;
    }
}

__device__ __forceinline__ void queue_fp64(const SweepArgs& a, int64_t g) {
    if (threadIdx.x == 0) {
        const int j = atomicAdd(a.fb_count, 1);
        a.fb_list[j] = (int32_t)g;
    }
}

// Lower bounds on each environment's objective at every scale of a chunk, summed in binary32
// from non-negative terms.  Z: the code-0 range [0, m_z) contributes its prefix sum kz (a
// non-decreasing function of the chunk's s_lo).  C: a weight that is clipped (code 7 or -8) at
// every scale of the chunk contributes d (|w'| - |q| s_hi)^2 when |w'| > |q| s_hi (its residual
// |w'| - |q| s only grows as s falls below s_hi): a non-increasing function of s_hi.  Every other
// term counts as 0, so Z + C bounds the chunk, Z bounds every chunk above it and C every chunk
// below it.  Any weight with |w'| > |q| s_hi has a clip key above the chunk's C threshold, so the
// range [m_c, G) holds all of them.  The lanes of environment lane % E split the weights; returns
// per lane the environment's C and Z.
template <int E>
__device__ __forceinline__ void chunk_lower_bounds(const SweepSmem<E>& sm, int m_z, int m_c, float s_hi,
                                                   float& lb_c, float& lb_z) {
    constexpr int P = 64 / E;
    const int lane = threadIdx.x & 63, e = lane % E;
    float v = 0.0f;
    for (int r = m_c + lane / E; r < G; r += P) {
        const float w = sm.ws[r];
        // |q| s_hi is exact (an 11-bit scale times 7 or 8): one rounding, the sign exact
        const float t = fmaxf(__builtin_fmaf(w > 0.0f ? -7.0f : -8.0f, s_hi, fabsf(w)), 0.0f);
        v = __builtin_fmaf(sm.ds[r * E + e], t * t, v);
    }
#pragma unroll
    for (int o = E; o < 64; o <<= 1) v += lane_xor(v, o);
    lb_c = v;
    lb_z = sm.kz[m_z * E + e];
}

// Maximum (minimax) and sum (pooled) over the environments of a per-lane value of environment
// lane % E; the same in all lanes.
template <int E>
__device__ __forceinline__ void env_max_sum(float v, float& mx, float& su) {
    mx = v;
    su = v;
#pragma unroll
    for (int o = 1; o < E; o <<= 1) {
        mx = fmaxf(mx, lane_xor(mx, o));
        su += lane_xor(su, o);
    }
}

// The binary32 screen over the chunks of one slice: each lane's best three (value, pattern) keys
// for minimax and for pooled.  The slice's chunks are c_start + slice + S v upwards and
// c_start - 1 - slice - S v downwards (v = 0, 1, ...); waves take them from two counters in LDS,
// each time from the side that has handed out fewer, so the chunks near the optimum come first.
// A chunk whose lower bound Z + C (chunk_lower_bounds) exceeds 1.001 times the smallest value
// screened so far (for each policy wanted) is skipped: all its binary32 values would exceed the
// shortlist threshold.  When C alone does on the way down (Z alone on the way up), so does every
// further chunk on that side, and that side stops.  With u = 2^-24: the computed bound is at most (1 + 150u) times an exact lower bound
// of F (at most 143 roundings of non-negative terms along any path), the screen's values are at
// least (1 - 131u) F (pooled: (1 - 131u)(1 - Eu)), and the threshold is at most 1.00004 (1 + u)
// times a value already screened, which is below 1.001 (1 - 350u).  Skipped
// scales are neither the minimum nor in the shortlist, nor can they push a shortlisted key out of
// a lane's best three, so the outputs are those of the full screen.
template <int E>
__device__ void screen_keys(const SweepArgs& a, SweepSmem<E>& sm, float pk, int slice, int S,
                            uint64_t (&mk)[3], uint64_t (&qk)[3]) {
    constexpr int NS = ns_for(E);
    constexpr int CHUNK = 64 * NS;                          // scales per wave per chunk
    // wave-uniform values read from LDS, held in scalar registers
    const uint32_t b_top = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.b_top);
    pk = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(pk)));
    const int nchunk = (int)((b_top - BITS_FIRST) / CHUNK) + 1;
    const int lane = threadIdx.x & 63;
    const float k0 = sm.ks[lane], k1 = sm.ks[lane + 64];
#pragma unroll
    for (int r = 0; r < 3; ++r) { mk[r] = KEY_NONE; qk[r] = KEY_NONE; }
    const int c_start = __builtin_amdgcn_readfirstlane(sm.c_start);
    volatile uint32_t* u_bits = sm.u_bits;
    for (;;) {
        int cl = -1, down = 0;
        if (lane == 0) {
            const int first = *(volatile int*)&sm.next_up <= *(volatile int*)&sm.next_down ? 0 : 1;
            for (int j = 0; j < 2 && cl < 0; ++j) {
                if ((first ^ j) == 0) {
                    const int cc = c_start + slice + S * atomicAdd(&sm.next_up, 1);
                    if (cc < nchunk && cc < *(volatile int*)&sm.lim_up) cl = cc;
                } else {
                    const int cc = c_start - 1 - slice - S * atomicAdd(&sm.next_down, 1);
                    if (cc >= 0 && cc > *(volatile int*)&sm.lim_down) { cl = cc; down = 1; }
                }
            }
        }
        const int c = __builtin_amdgcn_readfirstlane(cl);
        if (c < 0) break;
        const bool going_down = __builtin_amdgcn_readfirstlane(down) != 0;
        // The chunk's weight ranges (wave-uniform).  With K~ within 2u of the exact key and
        // 2^-20 margins on the thresholds:
        //   K~ <= s_lo/15:       |w'| <= 7.5 K < s_lo/2, code 0 at every scale of the chunk;
        //   K~ <  1.1333 s_lo:   x in (-8.5, 7.5) (7.367 s_lo or 8.5 s_lo bounds |w'|), never clipped;
        //   K~ >  s_hi:          w' > 6.5 s_hi or w' < -7.5 s_hi, code 7 or -8 throughout;
        //   otherwise:           the rounded code may clip.
        const float s_lo = half_bits_value(BITS_FIRST + (uint32_t)(c * CHUNK)) * pk;
        const float s_hi = half_bits_value(min(BITS_FIRST + (uint32_t)(c * CHUNK + CHUNK - 1), b_top)) * pk;
        const float tz = s_lo * ((1.0f / 15.0f) * (1.0f - 0x1p-20f));
        const float tu = s_lo * ((8.5f / 7.5f) * (1.0f - 0x1p-20f));
        const float tc = s_hi * (1.0f + 0x1p-20f);
        const int m_c = G - (int)(__popcll(__ballot(k0 > tc)) + __popcll(__ballot(k1 > tc)));
        const int m_u = min(m_c, (int)(__popcll(__ballot(k0 < tu)) + __popcll(__ballot(k1 < tu))));
        const int m_z = min(m_u, (int)(__popcll(__ballot(k0 <= tz)) + __popcll(__ballot(k1 <= tz))));
        {
            float lb_c, lb_z;
            chunk_lower_bounds<E>(sm, m_z, m_c, s_hi, lb_c, lb_z);
            float t_max, t_sum, o_max, o_sum;
            env_max_sum<E>(lb_c + lb_z, t_max, t_sum);
            env_max_sum<E>(going_down ? lb_c : lb_z, o_max, o_sum);
            const float um = 1.001f * __uint_as_float(u_bits[0]), up = 1.001f * __uint_as_float(u_bits[1]);
            const bool side = (!a.want_minimax || o_max > um) && (!a.want_pooled || o_sum > up);
            const bool skip = (!a.want_minimax || t_max > um) && (!a.want_pooled || t_sum > up);
            if (__builtin_amdgcn_readfirstlane((int)side)) {
                if (lane == 0) {
                    if (going_down) atomicMax(&sm.lim_down, c);
                    else atomicMin(&sm.lim_up, c);
                }
                continue;
            }
            if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
        }
        // The sums start from the terms that need no per-scale work: the code-0 ones (the same at
        // every scale, summed once in kz) and, when its closed form is accurate enough, the
        // fixed-code range: acc = fl32(kz + Q_e(s)), one rounding, which the screen's count of
        // at most 129 roundings per term covers.
        const float rl0 = __builtin_amdgcn_rcpf(s_lo), rh0 = __builtin_amdgcn_rcpf(s_hi);
        const float inv_lo = __builtin_fmaf(rl0, __builtin_fmaf(-s_lo, rl0, 1.0f), rl0);
        const float inv_hi = __builtin_fmaf(rh0, __builtin_fmaf(-s_hi, rh0, 1.0f), rh0);
        int n_u = 0;
        int n_var = classify_chunk<E>(sm, m_z, m_u, m_c, inv_lo, inv_hi, false, n_u);
        double fa = 0.0, fb = 0.0, fc = 0.0, fq = 0.0;
        const bool closed = fixed_code_sums<E>(sm, m_z, m_c, s_lo, s_hi, fa, fb, fc, fq);
        if (closed) {
            // A second lower bound, now that the fixed codes are summed: kz + min over the chunk
            // of Q (every other term counts as 0).  Same margins as the first.
            float t_max, t_sum;
            env_max_sum<E>((float)(fq + (double)sm.kz[m_z * E + lane % E]), t_max, t_sum);
            const bool skip = (!a.want_minimax || t_max > 1.001f * __uint_as_float(u_bits[0])) &&
                              (!a.want_pooled || t_sum > 1.001f * __uint_as_float(u_bits[1]));
            if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
        } else {
            n_var = classify_chunk<E>(sm, m_z, m_u, m_c, inv_lo, inv_hi, true, n_u);
        }
        float nsv[NS], inv[NS];
        float acc[NS][E];
        // Lane rotation: pattern b and b + 0x400k (the same fraction, 2^k times larger) would
        // otherwise share a lane; exact ties at power-of-two spacing (an outlier alone carrying a
        // code) then fill one lane's top three.  Rotating by 5 per chunk spreads them out.
        const int rot = (lane + 5 * c) & 63;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const uint32_t b = min(BITS_FIRST + (uint32_t)(c * CHUNK + rot + 64 * t), b_top);
            const float s = half_bits_value(b) * pk;
            nsv[t] = -s;
            // reciprocal within 1 binary32 ulp: hardware estimate plus one Newton step
            const float r0 = __builtin_amdgcn_rcpf(s);
            inv[t] = __builtin_fmaf(r0, __builtin_fmaf(-s, r0, 1.0f), r0);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float z = sm.kz[m_z * E + e];
            if (closed) {
                // fl32(z + Q(s)) with z added to A first (binary64, far inside the 2^-31)
                const double A = readlane_f64(fa, e) + (double)z;
                const double B2 = -2.0 * readlane_f64(fb, e), C = readlane_f64(fc, e);
#pragma unroll
                for (int t = 0; t < NS; ++t) {
                    const double sv = -(double)nsv[t];
                    acc[t][e] = (float)__builtin_fma(sv, __builtin_fma(sv, C, B2), A);
                }
            } else {
#pragma unroll
                for (int t = 0; t < NS; ++t) acc[t][e] = z;
            }
        }
        // the listed weights term by term: those whose code changes within the chunk, or all of
        // [m_z, m_c) and then the fixed-code range when the closed form is not accurate enough
        const uint8_t* vl = sm.vlist[threadIdx.x >> 6];
        sweep_list<E, NS, false>(sm.ws, sm.ds, vl, 0, n_u, nsv, inv, acc);
        sweep_list<E, NS, true>(sm.ws, sm.ds, vl, n_u, n_var, nsv, inv, acc);
        if (!closed) sweep_range_clipped<E, NS>(sm.ws, sm.qs, sm.ds, m_c, G, nsv, acc);
        float bm = __builtin_inff(), bp = __builtin_inff();
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const uint32_t b = BITS_FIRST + (uint32_t)(c * CHUNK + rot + 64 * t);
            if (b > b_top) continue;
            float Fm = acc[t][0], Ps = acc[t][0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                const float v = acc[t][e];
                Fm = fmaxf(Fm, v);
                Ps = Ps + v;
            }
            bm = fminf(bm, Fm);
            bp = fminf(bp, Ps);
            const uint64_t km = key_of(Fm, b), kq = key_of(Ps, b);
            if (a.want_minimax && km < mk[2]) top3_insert(mk, km);
            if (a.want_pooled && kq < qk[2]) top3_insert(qk, kq);
        }
        // values are >= 0, so their bit patterns order as the values do; the wave's minimum goes
        // in with one lane's atomic (64 lanes on one LDS word would serialise), and only when it
        // improves on the running minimum
        if (a.want_minimax) {
            const float m = wave_min_f(bm);
            if (lane == 0 && __float_as_uint(m) < u_bits[0]) atomicMin(&sm.u_bits[0], __float_as_uint(m));
        }
        if (a.want_pooled) {
            const float m = wave_min_f(bp);
            if (lane == 0 && __float_as_uint(m) < u_bits[1]) atomicMin(&sm.u_bits[1], __float_as_uint(m));
        }
    }
}

// Rescoring, the lower-bit-pattern rule and the outputs, once sm holds the shortlist
// (sm.cand_*, sm.n_cand, sm.overflow) and, for the zero rule, sm.win_b / sm.win_flags.
template <int E>
__device__ void finish_group(const SweepArgs& a, int64_t g, SweepSmem<E>& sm) {
    const int tid = threadIdx.x;
    __syncthreads();
    const int n = sm.n_cand;
    if (sm.overflow || n > CAP) {
        queue_fp64(a, g);
        return;
    }
    rescore<E>(sm, n, a.E);
    {
        // wave 0 picks the minimax winner, wave 1 the pooled one
        const int pol = tid >> 6;
        const bool want = pol == 0 ? a.want_minimax : (pol == 1 && a.want_pooled);
        if (want) {
            const uint8_t tag = pol == 0 ? TAG_MINIMAX : TAG_POOLED;
            const uint32_t b = sm.win_b[pol];
            const uint8_t f = sm.win_flags[pol];
            pick_winner<E>(sm, n, tag, pol);
            if (b != 0xFFFFFFFFu && (tid & 63) == 0) {  // zero rule: only the value from rescoring
                sm.win_b[pol] = b;
                sm.win_flags[pol] = f;
            }
        }
    }
    __syncthreads();
    if (a.want_minimax) {
        const uint32_t b = sm.win_b[0];
        if (tid < G && a.codes) a.codes[g * G + tid] = (int8_t)exact_code(sm.w[tid], half_bits_value(b));
        if (tid == 0) {
            a.scales[g] = (uint16_t)b;
            if (a.objective) a.objective[g] = sm.win_F[0];
            if (a.flags)
                a.flags[g] = sm.win_flags[0] | top_tie_flags(b, sm.b_top) | (a.mark_fallback ? FLAG_FALLBACK : 0);
        }
    }
    if (a.want_pooled && tid == 0) {
        if (a.pscales) a.pscales[g] = (uint16_t)sm.win_b[1];
        if (a.pobjective) a.pobjective[g] = sm.win_F[1];
        if (!a.want_minimax && a.flags) a.flags[g] = sm.win_flags[1] | top_tie_flags(sm.win_b[1], sm.b_top);
    }
    if (a.want_pooled && !a.want_minimax && tid < G && a.codes)
        a.codes[g * G + tid] = (int8_t)exact_code(sm.w[tid], half_bits_value(sm.win_b[1]));
}

// One workgroup per group: screen everything, shortlist, finish.
template <int E>
__device__ void sweep_group(const SweepArgs& a, int64_t g, SweepSmem<E>& sm) {
    const int tid = threadIdx.x;
    float pk, wmax;
    const int status = stage_group<E>(a, g, sm, pk, wmax);
    if (status == 1) { write_bad(a, g); return; }
    if (status == 2) { queue_fp64(a, g); return; }
    uint64_t mk[3], qk[3];
    screen_keys<E>(a, sm, pk, 0, 1, mk, qk);
    // both policies' smallest keys in one block reduction
    uint64_t best[2] = {mk[0], qk[0]};
    block_min_u64n<2>(best, sm.redk);
    for (int pol = 0; pol < 2; ++pol) {
        const bool want = pol == 0 ? a.want_minimax : a.want_pooled;
        if (!want) continue;
        const uint64_t* kk = pol == 0 ? mk : qk;
        const uint8_t tag = pol == 0 ? TAG_MINIMAX : TAG_POOLED;
        const uint64_t M1 = best[pol];
        const float m = key_value(M1);
        if (m == 0.0f) {
            // zero binary32 error is exact here: the lowest such pattern wins; the second key
            // tells whether another pattern is zero too
            const uint64_t S2 = block_min_u64(kk[0] == M1 ? kk[1] : kk[0], sm.redk);
            if (tid == 0) {
                append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(M1), tag);
                sm.win_flags[pol] = (S2 != KEY_NONE && key_value(S2) == 0.0f) ? (FLAG_NEAR_TIE | FLAG_EXACT_TIE) : 0;
                sm.win_b[pol] = key_bits(M1);
            }
        } else {
            const float T = m * SCREEN_RATIO;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                if (kk[r] != KEY_NONE && key_value(kk[r]) <= T) {
                    if (r == 2) sm.overflow = 1;
                    else append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(kk[r]), tag);
                }
            }
            if (tid == 0) sm.win_b[pol] = 0xFFFFFFFFu;  // decided by rescoring
        }
    }
    finish_group<E>(a, g, sm);  // starts with a barrier: the appends are in place
}

// Slice `slice` of S of one group: screen its chunks and record, per policy, its best and
// second keys and every key within the screen ratio of its own best (a superset of its share of
// the group's shortlist, since the group's best is no larger).  A lane whose third key is inside
// that bound may have dropped a fourth: its third value is recorded as the smallest value not kept.
template <int E>
__device__ void sweep_slice(const SweepArgs& a, int64_t g, int slice, int S, SlicePart* part, SweepSmem<E>& sm) {
    const int tid = threadIdx.x;
    float pk, wmax;
    const int status = stage_group<E>(a, g, sm, pk, wmax);
    if (status != 0) {
        if (tid == 0) part->status = (uint32_t)status;
        return;
    }
    uint64_t mk[3], qk[3];
    screen_keys<E>(a, sm, pk, slice, S, mk, qk);
    for (int pol = 0; pol < 2; ++pol) {
        const bool want = pol == 0 ? a.want_minimax : a.want_pooled;
        if (!want) continue;
        const uint64_t* kk = pol == 0 ? mk : qk;
        const uint64_t M1 = block_min_u64(kk[0], sm.redk);
        const uint64_t S2 = block_min_u64(kk[0] == M1 ? kk[1] : kk[0], sm.redk);
        if (tid == 0) { sm.n_cand = 0; sm.ovbits = 0xFFFFFFFFu; }
        __syncthreads();
        const float m = key_value(M1);
        const float T = m * SCREEN_RATIO;  // 0 when m == 0: only exact zeros are kept
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            if (kk[r] != KEY_NONE && key_value(kk[r]) <= T) {
                if (r == 2) atomicMin(&sm.ovbits, (uint32_t)(kk[r] >> 32));
                const int j = atomicAdd(&sm.n_cand, 1);
                if (j < SLICE_KEYS) part->keys[pol][j] = kk[r];
                else atomicMin(&sm.ovbits, (uint32_t)(kk[r] >> 32));
            }
        }
        __syncthreads();
        if (tid == 0) {
            part->m1[pol] = M1;
            part->s2[pol] = S2;
            part->n[pol] = (uint32_t)min(sm.n_cand, SLICE_KEYS);
            part->ov[pol] = sm.ovbits;
        }
        __syncthreads();
    }
    if (tid == 0) {
        part->b_top = sm.b_top;
        part->status = 0;
    }
}

// Merge the S parts of one group into its shortlist, then finish it.
template <int E>
__device__ void merge_group(const SweepArgs& a, int64_t g, int S, const SlicePart* parts, SweepSmem<E>& sm) {
    const int tid = threadIdx.x;
    const uint32_t status = parts[0].status;  // identical in every slice
    if (status == 1) { write_bad(a, g); return; }
    if (status == 2) { queue_fp64(a, g); return; }
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);
    if (tid < G) sm.w[tid] = wg[tid];
    for (int j = tid; j < E * G; j += BLOCK) sm.dt[(j % G) * E + j / G] = j / G < a.E ? dg[j] : 0.0f;
    if (tid == 0) { sm.n_cand = 0; sm.overflow = 0; sm.b_top = parts[0].b_top; }
    __syncthreads();
    for (int pol = 0; pol < 2; ++pol) {
        const bool want = pol == 0 ? a.want_minimax : a.want_pooled;
        if (!want) continue;
        const uint8_t tag = pol == 0 ? TAG_MINIMAX : TAG_POOLED;
        if (tid == 0) {
            uint64_t M1 = KEY_NONE, S2 = KEY_NONE;
            uint32_t ov = 0xFFFFFFFFu;
            for (int q = 0; q < S; ++q) {
                const uint64_t x = parts[q].m1[pol], y = parts[q].s2[pol];
                // keep the two smallest of all slices' best and second keys
                if (x < M1) { S2 = M1 < y ? M1 : y; M1 = x; }
                else if (x < S2) S2 = x;
                if (y < S2 && y != M1) S2 = y;
                ov = parts[q].ov[pol] < ov ? parts[q].ov[pol] : ov;
            }
            sm.mrg_m1[pol] = M1;
            const float m = key_value(M1);
            if (m == 0.0f) {
                sm.win_b[pol] = key_bits(M1);
                sm.win_flags[pol] = (S2 != KEY_NONE && key_value(S2) == 0.0f) ? (FLAG_NEAR_TIE | FLAG_EXACT_TIE) : 0;
                append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(M1), tag);
            } else {
                sm.win_b[pol] = 0xFFFFFFFFu;
                if (__uint_as_float(ov) <= m * SCREEN_RATIO) sm.overflow = 1;
            }
        }
        __syncthreads();
        const float m = key_value(sm.mrg_m1[pol]);
        if (m != 0.0f) {
            const float T = m * SCREEN_RATIO;
            for (int j = tid; j < S * SLICE_KEYS; j += BLOCK) {
                const int q = j / SLICE_KEYS, r = j % SLICE_KEYS;
                if (r < (int)parts[q].n[pol]) {
                    const uint64_t k = parts[q].keys[pol][r];
                    if (key_value(k) <= T) append_cand(sm.cand_b, sm.cand_tag, &sm.n_cand, key_bits(k), tag);
                }
            }
        }
        __syncthreads();
    }
    finish_group<E>(a, g, sm);
}

template <int E>
__global__ __launch_bounds__(BLOCK, min_blocks_for(E)) void sweep_f32_kernel(SweepArgs a) {
    __shared__ SweepSmem<E> sm;
    const int S = a.slices;
    if (a.list) {
        // Listed groups (the count is on the device).  Workgroups below list_split serve the
        // entries below LIST_SLICED, each split over S workgroups (entry k, slice j on workgroup
        // (k % lanes) * S + j, lanes = list_split / S); the others serve the entries from
        // LIST_SLICED on, one workgroup each.
        const int cnt = *a.list_count;
        if ((int)blockIdx.x < a.list_split) {
            const int lanes = a.list_split / S;
            const int sl = blockIdx.x % S;
            for (int k = blockIdx.x / S; k < min(cnt, LIST_SLICED); k += lanes) {
                sweep_slice<E>(a, (int64_t)a.list[k], sl, S, a.parts + (int64_t)k * S + sl, sm);
                __syncthreads();
            }
        } else {
            const int nb = gridDim.x - a.list_split;
            for (int k = LIST_SLICED + ((int)blockIdx.x - a.list_split); k < cnt; k += nb) {
                sweep_group<E>(a, (int64_t)a.list[k], sm);
                __syncthreads();
            }
        }
    } else if (S > 1) {
        const int64_t k = blockIdx.x / S;
        sweep_slice<E>(a, k + a.group_offset, blockIdx.x % S, S, a.parts + blockIdx.x, sm);
    } else {
        sweep_group<E>(a, (int64_t)blockIdx.x + a.group_offset, sm);
    }
}

template <int E>
__global__ __launch_bounds__(BLOCK) void sweep_merge_kernel(SweepArgs a, int n_direct) {
    __shared__ SweepSmem<E> sm;
    const int S = a.slices;
    if (a.list) {
        const int end = min(*a.list_count, LIST_SLICED);
        for (int k = blockIdx.x; k < end; k += gridDim.x) {
            merge_group<E>(a, (int64_t)a.list[k], S, a.parts + (int64_t)k * S, sm);
            __syncthreads();
        }
    } else if ((int)blockIdx.x < n_direct) {
        merge_group<E>(a, (int64_t)blockIdx.x + a.group_offset, S, a.parts + (int64_t)blockIdx.x * S, sm);
    }
}

// ------------------------------------------------------------------ binary64 sweep
// Every scale in binary64, each environment summed in the definition's order;
// the lexicographic (value, bits) minimum is the answer with no screen at all.
// Used for groups the binary32 screen could not settle.
template <int E>
struct F64Smem {
    float w[G];
    float dt[G * E];
    double rv[BLOCK];
    uint32_t rb[BLOCK];
    double rv2[BLOCK];
    uint32_t rb2[BLOCK];
};

__device__ __forceinline__ bool lex_less(double v, uint32_t b, double v2, uint32_t b2) {
    return v < v2 || (v == v2 && b < b2);
}

template <int E>
__device__ void f64_reduce(F64Smem<E>& sm, double v1, uint32_t b1, double v2, uint32_t b2,
                           double& outv, uint32_t& outb, double& outv2) {
    const int t = threadIdx.x;
    sm.rv[t] = v1; sm.rb[t] = b1; sm.rv2[t] = v2; sm.rb2[t] = b2;
    __syncthreads();
    for (int s = BLOCK / 2; s > 0; s >>= 1) {
        if (t < s) {
            // merge two (best, second) pairs
            double av = sm.rv[t], av2 = sm.rv2[t], bv = sm.rv[t + s], bv2 = sm.rv2[t + s];
            uint32_t ab = sm.rb[t], ab2 = sm.rb2[t], bb = sm.rb[t + s], bb2 = sm.rb2[t + s];
            if (lex_less(bv, bb, av, ab)) {
                // b is best; second = min(a, b2)
                sm.rv[t] = bv; sm.rb[t] = bb;
                if (lex_less(av, ab, bv2, bb2)) { sm.rv2[t] = av; sm.rb2[t] = ab; }
                else { sm.rv2[t] = bv2; sm.rb2[t] = bb2; }
            } else {
                if (lex_less(bv, bb, av2, ab2)) { sm.rv2[t] = bv; sm.rb2[t] = bb; }
            }
        }
        __syncthreads();
    }
    outv = sm.rv[0]; outb = sm.rb[0]; outv2 = sm.rv2[0];
    __syncthreads();
}

template <int E>
__device__ void f64_sweep_group(const SweepArgs& a, int64_t g, F64Smem<E>& sm) {
    const int tid = threadIdx.x;
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);
    if (tid < G) sm.w[tid] = wg[tid];
    for (int j = tid; j < E * G; j += BLOCK) sm.dt[(j % G) * E + j / G] = j / G < a.E ? dg[j] : 0.0f;
    __syncthreads();
    float wmax = 0.0f;
    for (int i = 0; i < G; ++i) wmax = fmaxf(wmax, fabsf(sm.w[i]));
    const uint32_t b_top = top_pattern(wmax);
    const double INF = __builtin_inf();
    double mv1 = INF, mv2 = INF, pv1 = INF, pv2 = INF;
    uint32_t mb1 = 0xFFFFFFFFu, mb2 = 0xFFFFFFFFu, pb1 = 0xFFFFFFFFu, pb2 = 0xFFFFFFFFu;
    for (uint32_t b = BITS_FIRST + tid; b <= b_top; b += BLOCK) {
        const double s = (double)half_bits_value(b), inv = 1.0 / s;
        double Fe[E];
#pragma unroll
        for (int e = 0; e < E; ++e) Fe[e] = 0.0;
        for (int i = 0; i < G; ++i) {
            const double wi = (double)sm.w[i];
            double r = __builtin_rint(wi * inv);
            r = r < -8.0 ? -8.0 : (r > 7.0 ? 7.0 : r);
            const double sq = s * r;
            const double t = wi - sq;
            const double t2 = t * t;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double term = (double)sm.dt[i * E + e] * t2;
                Fe[e] = Fe[e] + term;
            }
        }
        double F = Fe[0], P = Fe[0];
#pragma unroll
        for (int e = 1; e < E; ++e) { F = Fe[e] > F ? Fe[e] : F; P = P + Fe[e]; }
        P = P / (double)a.E;
        // ascending b within a thread: strict '<' keeps the lower pattern
        if (F < mv1) { mv2 = mv1; mb2 = mb1; mv1 = F; mb1 = b; }
        else if (F < mv2) { mv2 = F; mb2 = b; }
        if (P < pv1) { pv2 = pv1; pb2 = pb1; pv1 = P; pb1 = b; }
        else if (P < pv2) { pv2 = P; pb2 = b; }
    }
    double bestF, secF, bestP, secP;
    uint32_t bm, bp;
    f64_reduce<E>(sm, mv1, mb1, mv2, mb2, bestF, bm, secF);
    f64_reduce<E>(sm, pv1, pb1, pv2, pb2, bestP, bp, secP);
    if (a.want_minimax) {
        if (tid < G && a.codes) a.codes[g * G + tid] = (int8_t)exact_code(sm.w[tid], half_bits_value(bm));
        if (tid == 0) {
            a.scales[g] = (uint16_t)bm;
            if (a.objective) a.objective[g] = bestF;
            if (a.flags)
                a.flags[g] = FLAG_FP64_SWEEP | (secF == bestF ? (FLAG_EXACT_TIE | FLAG_NEAR_TIE) : 0) |
                             top_tie_flags(bm, b_top) | (a.mark_fallback ? FLAG_FALLBACK : 0);
        }
    }
    if (a.want_pooled) {
        if (tid == 0) {
            if (a.pscales) a.pscales[g] = (uint16_t)bp;
            if (a.pobjective) a.pobjective[g] = bestP;
            if (!a.want_minimax && a.flags)
                a.flags[g] = FLAG_FP64_SWEEP | (secP == bestP ? (FLAG_EXACT_TIE | FLAG_NEAR_TIE) : 0) |
                             top_tie_flags(bp, b_top);
        }
        if (!a.want_minimax && tid < G && a.codes)
            a.codes[g * G + tid] = (int8_t)exact_code(sm.w[tid], half_bits_value(bp));
    }
}

template <int E>
__global__ __launch_bounds__(BLOCK) void sweep_f64_kernel(SweepArgs a) {
    __shared__ F64Smem<E> sm;
    const int cnt = *a.fb_count;
    for (int k = blockIdx.x; k < cnt; k += gridDim.x) {
        f64_sweep_group<E>(a, (int64_t)a.fb_list[k], sm);
        __syncthreads();
    }
}

__global__ void zero_counter_kernel(int32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

template <int E>
static hipError_t launch_e(const SweepArgs& a_in, int64_t n_groups, hipStream_t st) {
    constexpr int NCHUNK = (N_SCALES + 64 * ns_for(E) - 1) / (64 * ns_for(E));
    // Slices per group: the screen usually stops near 40% of the grid (the top pattern), so a
    // group has about NCHUNK / 2 chunks; S_MAX gives each wave of each slice about one of them.
    constexpr int S_MAX = NCHUNK / 8 < 15 ? NCHUNK / 8 : 15;
    SweepArgs a = a_in;
    const int fb_blocks = (int)(n_groups < 1024 ? (n_groups > 0 ? n_groups : 1) : 1024);
    if (!a.fb_zeroed) hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(64), 0, st, a.fb_count);
    if (a.list) {
        // listed groups (few, count unknown on the host): one small looping grid, the first
        // LIST_SLICED entries sliced, a long list's rest one workgroup each
        a.slices = LIST_SLICES;
        const int lanes = (int)(n_groups < 32 ? n_groups : 32);
        a.list_split = lanes * LIST_SLICES;
        const int64_t rest = n_groups > LIST_SLICED ? n_groups - LIST_SLICED : 0;
        const int rest_blocks = (int)(rest < 2048 ? rest : 2048);
        hipLaunchKernelGGL(sweep_f32_kernel<E>, dim3(a.list_split + rest_blocks), dim3(BLOCK), 0, st, a);
        hipLaunchKernelGGL(sweep_merge_kernel<E>, dim3(lanes), dim3(BLOCK), 0, st, a, 0);
    } else {
        // few groups: split each over S workgroups so that the whole GPU works on them
        int S = 1;
        if (n_groups < 1024) {
            S = (int)((2048 + n_groups - 1) / n_groups);
            S = S > S_MAX ? S_MAX : S;
            while (S > 1 && n_groups * S > SLICE_PARTS) --S;
        }
        a.slices = S;
        if (S > 1) {
            hipLaunchKernelGGL(sweep_f32_kernel<E>, dim3((unsigned)(n_groups * S)), dim3(BLOCK), 0, st, a);
            hipLaunchKernelGGL(sweep_merge_kernel<E>, dim3((unsigned)n_groups), dim3(BLOCK), 0, st, a,
                               (int)n_groups);
        } else {
            // grid.x is limited to 2^31-1 blocks: split very large batches
            const int64_t step = 1ll << 30;
            for (int64_t off = 0; off < n_groups; off += step) {
                SweepArgs b = a;
                b.group_offset = off;
                const int64_t n = n_groups - off < step ? n_groups - off : step;
                hipLaunchKernelGGL(sweep_f32_kernel<E>, dim3((unsigned)n), dim3(BLOCK), 0, st, b);
            }
        }
    }
    hipLaunchKernelGGL(sweep_f64_kernel<E>, dim3(fb_blocks), dim3(BLOCK), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sweep(const SweepArgs& a_in, int E, int64_t n_groups, hipStream_t st) {
    SweepArgs a = a_in;
    a.E = E;
    switch (pad_envs(E)) {
        case 1: return launch_e<1>(a, n_groups, st);
        case 2: return launch_e<2>(a, n_groups, st);
        case 4: return launch_e<4>(a, n_groups, st);
        case 8: return launch_e<8>(a, n_groups, st);
        case 16: return launch_e<16>(a, n_groups, st);
        case 32: return launch_e<32>(a, n_groups, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cqk
