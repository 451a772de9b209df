// Candidate-set solver for gfx950.
//
// The pages' production solver lists the scales that can be optimal -- those
// where a code changes, the vertices of the quadratic pieces, and the points
// where two environments' errors cross -- and hands a tie between directly
// scored candidates to an exhaustive check of the grid (CliffQuant repository
// README, "What CliffQuant changes" and "Verification"; model card
// "Verification").  The steps here are our own design of that idea on the
// binary16 grid:
//
//  0. Window.  Scales below a bound from the best single clipped weight
//     against F at max|w|/9 (max|w|/(X + 1) for another code range, X its larger
//     end magnitude) cannot be optimal; no transition below it is kept.
//  1. Code transitions.  For w_i != 0 and each c with |q_i| able to fall from
//     c+1 to c, the first grid pattern t where |q_i(s_t)| <= c.  The test
//     |q| <= c  <=>  |w| < (c+1/2) s  or  (|w| == (c+1/2) s and c even)  is
//     exact in binary32 ((c+1/2) s has at most 15 significant bits) and monotone
//     in s; t is the binary16 rounding of |w|/(c+1/2) confirmed by a short walk
//     on that predicate (bisection if the walk does not settle).
//  2. Runs.  The events are sorted by t (a bitonic sort held in registers:
//     lane shuffles; one wave up to 512 events, else four waves with 3 stages
//     through LDS); between two
//     consecutive event patterns every code is constant, so each environment
//     error is the quadratic f_e(s) = A_e - 2 B_e s + C_e s^2 with
//     B_e = sum d w q, C_e = sum d q^2.  A block-wide prefix sum over the
//     sorted events gives (B_e, C_e) of every run in binary64.
//  3. Candidates.  F = max_e f_e is convex on a run, so its grid minimum sits
//     next to the run's continuous minimiser: a run end, the vertex B_e/C_e
//     of an environment on top, or the crossing of two environments on top.
//     Runs whose lower bound max_e min f_e already exceeds the best end-point
//     value are skipped; the rest are compacted into LDS and every vertex and
//     crossing on their upper envelope is mapped to its grid neighbours (+-2
//     patterns of slack).
//  4. Reduction.  Every candidate within the proven error of the quadratic
//     form of the best one is rescored directly in binary64 in the same
//     summation order as the definition's plain sequential sum.  The lowest
//     value wins; if two distinct patterns tie bit for bit, or a list overflows
//     (kept runs, candidates, shortlist), the group is handed to the exhaustive
//     sweep (flag FALLBACK).
//
// Quantizers.  Besides the pages' [-8, 7] on groups of 128, the solver takes any code range
// [qmin, qmax] with -8 <= qmin <= 0 <= qmax <= 8 on groups of up to 128 weights (the quantizer
// specification of the README's "Use the solver"): a weight has at most max(qmax, -qmin)
// transitions, which the 8 event slots per weight hold, and a shorter group is padded in LDS with
// zero weights, which change no code, no sum and no transition.
#include "device.h"
#include "search_args.h"

namespace cqk {
namespace {

constexpr int MAX_EV = 1024;  // 8 slots per weight: at most 7 (w > 0) or 8 (w < 0) transitions
constexpr int QCAP = 512;     // quadratic-form candidates per group
constexpr int CCAP = 256;     // direct-rescoring shortlist per group
constexpr int rcap_for(int E) { return E <= 8 ? 64 : (E == 16 ? 32 : 16); }  // surviving runs
// |error of a quadratic-form value| <= ERR_REL * max_e (A_e + 2 B0_e s + C0_e s^2): the prefix
// sums run over <= 1024 events with partial sums in [0, B0_e] / [0, C0_e], plus the 128-term
// initial sums and the evaluation itself, i.e. < 1200 roundings of 2^-53 each.
constexpr double ERR_REL = 0x1p-40;
constexpr double SEL_SLACK = 1e-12;

template <int E>
struct CandSmem {
    static constexpr int RCAP = rcap_for(E);
    // the rescoring terms of PER_T scales at a time are formed in LDS
    static constexpr int PER_T = E <= 8 ? 8 / E : 1;
    __align__(16) float w[G];
    __align__(16) float d[E * G];  // [e][i]
    union {
        uint32_t ev[MAX_EV];   // transitions: read last by the run folds
        struct {               // quadratic-form candidates: written first after the runs are kept
            double q_lo[QCAP];
            uint32_t q_b[QCAP];
        };
        uint8_t qbuf[RCAP][G];  // the codes of the kept runs' first patterns (read last before
                                // the candidates are listed)
        // rescoring terms d_ei (w_i - s q_i)^2, written first after the shortlist is taken (rows
        // padded by one: the summing lanes read distinct banks)
        double term[PER_T][E][G + 1];
    };
    uint8_t magp[BLOCK];
    double part[2][E];
    double A[E], B0[E], C0[E];
    double mag_c[3];  // max_e A_e, 2 max_e B0_e, max_e C0_e: the magnitude bound's coefficients
    double wtot[BLOCK / 64][8];
    double redd[BLOCK / 64];
    float redf[2 * (BLOCK / 64)];
    int redi[BLOCK / 64];
    uint32_t run_lo[RCAP], run_hi[RCAP];
    double run_B[RCAP][E], run_C[RCAP][E];
    uint32_t cand_b[CCAP];
    double cand_F[CCAP];
    int n_runs, n_q, n_cand, n_ev;
    uint32_t win_b;
    double win_F;
    int win_state, win_count;
};

__device__ __forceinline__ double wave_min_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double u = lane_xor(v, o);
        v = u < v ? u : v;
    }
    return v;
}
__device__ __forceinline__ double block_min_d(double v, double* red) {
    v = wave_min_d(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = red[0];
#pragma unroll
    for (int k = 1; k < BLOCK / 64; ++k) r = red[k] < r ? red[k] : r;
    return r;
}
__device__ __forceinline__ int block_sum_i(int v, int* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += (int)lane_xor((uint32_t)v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int k = 0; k < BLOCK / 64; ++k) r += red[k];
    return r;
}

// |q(w, s_b)| <= c  (exact, see the file comment)
// Inclusive prefix sum over the 64 lanes of a wave through DPP: row_shr 1, 2, 4, 8 within each
// row of 16 lanes (lanes with no source add 0), then row_bcast15 and row_bcast31 carry the
// totals of the earlier rows.  Both 32-bit halves of a double move together.
__device__ __forceinline__ double wave_inclusive_sum_f64(double x) {
#define CQ_SCAN_STEP(ctrl, rmask)                                                                      \
    {                                                                                                  \
        const uint64_t u_ = __builtin_bit_cast(uint64_t, x);                                           \
        const uint32_t lo_ = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u_, ctrl, rmask, 0xF, true); \
        const uint32_t hi_ = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u_ >> 32), ctrl, rmask, 0xF, true); \
        x += __builtin_bit_cast(double, ((uint64_t)hi_ << 32) | lo_);                                  \
    }
    CQ_SCAN_STEP(0x111, 0xF)
    CQ_SCAN_STEP(0x112, 0xF)
    CQ_SCAN_STEP(0x114, 0xF)
    CQ_SCAN_STEP(0x118, 0xF)
    CQ_SCAN_STEP(0x142, 0xA)
    CQ_SCAN_STEP(0x143, 0xC)
#undef CQ_SCAN_STEP
    return x;
}

// Bitonic sort (ascending) of positions 0 .. 2^log_n - 1 of ev by one wave, 64 KPT >= 2^log_n:
// lane l holds positions KPT l .. KPT l + KPT - 1 in registers, so partners closer than KPT are in
// the same lane and the others one lane shuffle away; no barrier is needed.
template <int KPT>
__device__ __forceinline__ void wave_sort(uint32_t* ev, int log_n, int lane) {
    constexpr int LOGMAX = KPT == 4 ? 8 : (KPT == 8 ? 9 : 10);
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = ev[KPT * lane + r];
#pragma unroll
    for (int kk = 1; kk <= LOGMAX; ++kk) {
        const int k = 1 << kk;
#pragma unroll
        for (int jj = kk - 1; jj >= 0; --jj) {
            if (kk > log_n) continue;  // uniform: the phases past the sort's size
            const int j = 1 << jj;
            if (j < KPT) {
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    if ((r & j) == 0) {
                        const bool up = ((KPT * lane + r) & k) == 0;
                        const uint32_t x = key[r], y = key[r + j];
                        if ((x > y) == up) { key[r] = y; key[r + j] = x; }
                    }
                }
            } else {
                const int m = j / KPT;  // partner lane: lane ^ m
                const bool up = ((KPT * lane) & k) == 0, lower = (lane & m) == 0;
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const uint32_t o = lane_xor(key[r], m);
                    const uint32_t lo = key[r] < o ? key[r] : o, hi = key[r] < o ? o : key[r];
                    key[r] = lower == up ? lo : hi;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) ev[KPT * lane + r] = key[r];
}

// The value of a finite binary16 pattern by one hardware conversion (exact: every binary16 value
// is a binary32 value).
__device__ __forceinline__ float half_value_hw(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ bool mag_at_most(float a, int c, uint32_t b) {
    const float hs = (float)(2 * c + 1) * 0.5f * half_value_hw(b);
    return a < hs || (a == hs && (c & 1) == 0);
}

// First pattern b with mag_at_most(a, c, b), given that it is false at the first pattern and
// true at the last.  The boundary a/(c+1/2) rounded to binary16 lands within a pattern of it;
// a short walk confirms the first true pattern and bisection covers anything else.
__device__ __forceinline__ uint32_t first_at_most(float a, int c) {
    // a guess only (the walk and the bisection below decide): a reciprocal, a product and a
    // hardware conversion to binary16 (infinity above the range, clamped below)
    const float tau = a * __builtin_amdgcn_rcpf((float)(2 * c + 1) * 0.5f);
    uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)tau);
    b = b < BITS_FIRST + 1 ? BITS_FIRST + 1 : (b > BITS_LAST ? BITS_LAST : b);
    for (int k = 0; k < 4; ++k) {
        const bool here = mag_at_most(a, c, b), before = mag_at_most(a, c, b - 1);
        if (here && !before) return b;
        if (here) --b;   // b > BITS_FIRST + 0 always: the first pattern is false
        else ++b;        // b < BITS_LAST always: the last pattern is true
    }
    uint32_t lo = BITS_FIRST, hi = BITS_LAST;  // false at lo, true at hi
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (mag_at_most(a, c, mid)) hi = mid;
        else lo = mid;
    }
    return hi;
}

template <int E>
__device__ __forceinline__ double quad_run(const CandSmem<E>& sm, int r, double s, double& err) {
    double F = sm.A[0] + s * (sm.run_C[r][0] * s - 2.0 * sm.run_B[r][0]);
    for (int e = 1; e < E; ++e) {
        const double f = sm.A[e] + s * (sm.run_C[r][e] * s - 2.0 * sm.run_B[r][e]);
        F = f > F ? f : F;
    }
    // the magnitude bound from the maxima of A, B0 and C0 over the environments (never smaller
    // than max_e (A_e + 2 B0_e s + C0_e s^2))
    err = ERR_REL * __builtin_fma(s, __builtin_fma(sm.mag_c[2], s, sm.mag_c[1]), sm.mag_c[0]);
    return F;
}

// Items of the candidate search of a surviving run: k = 0 its two ends, k = 1..E the vertex of
// environment k-1, then one item per pair of environments for their crossings.
template <int E>
constexpr int cand_items() { return 1 + E + E * (E - 1) / 2; }

// Calls fn(b) for every candidate pattern of item k of surviving run r: the run's ends, or the
// grid neighbours (+-2) of a vertex or of a pairwise crossing that lies on the upper envelope.
template <int E, typename Fn>
__device__ void run_candidate_item(const CandSmem<E>& sm, int r, int k, Fn&& fn) {
    const uint32_t blo = sm.run_lo[r], bhi = sm.run_hi[r];
    if (k == 0) {
        fn(blo);
        if (bhi != blo) fn(bhi);
        return;
    }
    if (bhi - blo < 2) return;
    const double slo = (double)half_bits_value(blo), shi = (double)half_bits_value(bhi);
    auto near = [&](double s) {
        const uint32_t b0 = f32_to_half_bits_rne((float)s);
        const uint32_t lo = b0 >= blo + 2 ? b0 - 2 : blo;
        const uint32_t hi = b0 + 2 <= bhi ? b0 + 2 : bhi;
        for (uint32_t b = lo; b <= hi; ++b)
            if (b != blo && b != bhi) fn(b);
    };
    auto on_top = [&](double s, int e1, int e2) {
        double err;
        const double F = quad_run<E>(sm, r, s, err);
        const double tol = 2.0 * err + SEL_SLACK * (F > 0.0 ? F : 0.0);
        const double f1 = sm.A[e1] + s * (sm.run_C[r][e1] * s - 2.0 * sm.run_B[r][e1]);
        const double f2 = sm.A[e2] + s * (sm.run_C[r][e2] * s - 2.0 * sm.run_B[r][e2]);
        return f1 >= F - tol && f2 >= F - tol;
    };
    if (k <= E) {
        const int e = k - 1;
        const double C = sm.run_C[r][e];
        if (C > 0.0) {
            const double v = sm.run_B[r][e] / C;
            if (v >= slo && v <= shi && on_top(v, e, e)) near(v);
        }
        return;
    }
    int p = k - 1 - E, e1 = 0;
    while (p >= E - 1 - e1) { p -= E - 1 - e1; ++e1; }
    const int e2 = e1 + 1 + p;
    const double a = sm.run_C[r][e1] - sm.run_C[r][e2];
    const double hb = sm.run_B[r][e1] - sm.run_B[r][e2];
    const double cc = sm.A[e1] - sm.A[e2];
    double r0 = -1.0, r1 = -1.0;
    if (a == 0.0) {
        if (hb != 0.0) r0 = cc / (2.0 * hb);
    } else {
        const double disc = hb * hb - a * cc;
        if (disc >= 0.0) {
            const double sq = __builtin_sqrt(disc);
            const double qq = hb + (hb >= 0.0 ? sq : -sq);
            if (qq != 0.0) {
                r0 = qq / a;
                r1 = cc / qq;
            } else {
                r0 = hb / a;
            }
        }
    }
    if (r0 >= slo && r0 <= shi && on_top(r0, e1, e2)) near(r0);
    if (r1 >= slo && r1 <= shi && on_top(r1, e1, e2)) near(r1);
}

template <int E>
__device__ void candidate_group(const CandArgs& a, int64_t g, CandSmem<E>& sm) {
    constexpr int RCAP = CandSmem<E>::RCAP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Gn = a.G;  // the group's own length; weights Gn..G-1 are zero padding
    const float qlo = (float)a.qmin, qhi = (float)a.qmax;
    const float* wg = a.w + g * Gn;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * Gn);

    // ---- staging and input checks (environments a.E..E-1 and weights Gn..G-1 are zero padding:
    //      a zero weight has code 0 and residual 0 at every scale, so it adds an exact 0.0 to
    //      every sum and starts no transition)
    if (tid < G) sm.w[tid] = tid < Gn ? wg[tid] : 0.0f;
    for (int j = tid; j < E * G; j += BLOCK) {
        const int e = j / G, i = j - e * G;
        sm.d[j] = (e < a.E && i < Gn) ? dg[e * Gn + i] : 0.0f;
    }
    if (tid == 0) { sm.n_runs = 0; sm.n_q = 0; sm.n_cand = 0; sm.n_ev = 0; }
    __syncthreads();
    float bad = 0.0f;
    if (tid < G && !__builtin_isfinite(sm.w[tid])) bad = 1.0f;
    for (int j = tid; j < E * G; j += BLOCK) {
        const float v = sm.d[j];
        if (!(v >= 0.0f) || !__builtin_isfinite(v)) bad = 1.0f;
    }
    // whether an input is bad, and max|w|, in one reduction
    float red2[2] = {bad, tid < G ? fabsf(sm.w[tid]) : 0.0f};
    block_max_fn<2>(red2, sm.redf);
    if (red2[0] != 0.0f) {
        if (tid < Gn && a.codes) a.codes[g * Gn + tid] = 0;
        if (tid == 0) {
            a.scales[g] = 0;
            if (a.objective) a.objective[g] = __builtin_nan("");
            if (a.flags) a.flags[g] = FLAG_BAD_INPUT;
        }
        return;
    }
    const float wmax = red2[1];

    // ---- 0. where the optimum can lie.  U = F at s_a = binary16(max|w|/(X + 1)) (binary64, X the
    //         larger magnitude of the range ends: max|w|/9 for [-8, 7]) bounds the optimum from
    //         above; the minimax optimum usually lies near there, below the AbsMax scale, so U is
    //         tighter than at max|w|/7.  Below y_i = |w_i|/|q_i| (q_i = qmax for w_i > 0, qmin
    //         otherwise) weight i is clipped and its residual is |w_i| - |q_i| s,
    //         so every scale with s <= (|w_i| - sqrt(1.0001 U / max_e d_ei)) / |q_i| has
    //         max_e F_e(s) > U: it is neither the answer nor a tie with it.  The largest such
    //         bound over the weights (less 2^-40 for the binary64 roundings) gives the first
    //         pattern that can hold the optimum; only transitions above it matter.  Thread i < G
    //         takes weight i: its residual at s_a (waves 0 and 1 sum each environment by a DPP
    //         scan) and then its bound.
    uint32_t win_lo = BITS_FIRST;  // the window of patterns that can hold the optimum
    const uint32_t win_hi = BITS_LAST;
    uint32_t b_a = f32_to_half_bits_rne(wmax * a.start_ratio);
    b_a = b_a < BITS_FIRST ? BITS_FIRST : (b_a > BITS_LAST ? BITS_LAST : b_a);
    {
        const float sa = half_bits_value(b_a);
        double dmax = 0.0;
        if (wave < 2) {
            const double r = __builtin_fma(-(double)sa, (double)exact_code_range(sm.w[tid], sa, qlo, qhi), (double)sm.w[tid]);
            const double r2 = r * r;
            // the environments' wave sums side by side (DPP scans; lane 63 holds each total)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double dv = (double)sm.d[e * G + tid];
                dmax = fmax(dmax, dv);
                const double v = wave_inclusive_sum_f64(dv * r2);
                if (lane == 63) sm.part[wave][e] = v;
            }
        }
        __syncthreads();
        double U = 0.0;
        for (int e = 0; e < E; ++e) U = fmax(U, sm.part[0][e] + sm.part[1][e]);
        double lo = -1.0;
        // (a weight whose side of the range holds only code 0 keeps its residual |w| at every
        // scale and bounds nothing)
        if (wave < 2 && dmax > 0.0 && wmax > 0.0f) {
            const double aw = fabs((double)sm.w[tid]), qa = sm.w[tid] > 0.0f ? (double)a.qmax : -(double)a.qmin;
            if (qa > 0.0) lo = (aw - __builtin_sqrt(1.0001 * U / dmax)) / qa * (1.0 - 0x1p-40);
        }
        lo = -block_min_d(-lo, sm.redd);  // the largest bound over the weights
        // the first pattern above lo (never above b_a: F(s_a) <= U), the same in every thread
        uint32_t b = BITS_FIRST;
        if (lo >= (double)half_bits_value(BITS_FIRST)) {
            b = f32_to_half_bits_rne((float)lo);
            b = b < BITS_FIRST ? BITS_FIRST : (b > b_a ? b_a : b);
            while (b > BITS_FIRST && (double)half_bits_value(b - 1) > lo) --b;
            while (b < b_a && (double)half_bits_value(b) <= lo) ++b;
        }
        win_lo = b;
    }

    // ---- 1. code transitions inside the window: thread t handles weight t/2, thresholds
    //         c = 4(t&1) .. 4(t&1)+3; the events are appended in any order (the sort orders them)
    {
        const int i = tid >> 1, c0 = 4 * (tid & 1);
        const float wi = sm.w[i];
        const float aw = fabsf(wi);
        const int cmax = wi > 0.0f ? a.qmax - 1 : -a.qmin - 1;  // the clip caps |q| at the range end
        int m0 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = c0 + k;
            bool hit = false;
            uint32_t key = 0;
            if (wi != 0.0f && c <= cmax && !mag_at_most(aw, c, win_lo)) {
                ++m0;  // the magnitude at the window's first pattern exceeds c
                if (mag_at_most(aw, c, win_hi)) {
                    hit = true;
                    key = (first_at_most(aw, c) << 11) | ((uint32_t)i << 4) | (uint32_t)c;
                }
            }
            // one LDS atomic per wave: the wave's hits take consecutive slots in lane order
            const uint64_t m = __ballot(hit);
            int base = 0;
            if (lane == 0 && m) base = atomicAdd(&sm.n_ev, (int)__popcll(m));
            base = __builtin_amdgcn_readfirstlane(base);
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit) sm.ev[base + rank] = key;
        }
        sm.magp[tid] = (uint8_t)m0;
    }
    __syncthreads();
    const int n_ev = sm.n_ev;
    // the sort's size: the next power of two >= n_ev (at least 4), padding keys sort last
    const int log_n = n_ev <= 4 ? 2 : 32 - __builtin_clz((uint32_t)(n_ev - 1));
    for (int j = n_ev + tid; j < (1 << log_n); j += BLOCK) sm.ev[j] = 0xFFFFFFFFu;
    __syncthreads();

    // ---- 2a. sort the events (bitonic, ascending): the first log_n merge phases of the network
    //          over 1024 positions sort positions 0 .. 2^log_n - 1.  Thread t holds positions
    //          4t..4t+3 in registers: partners closer than 4 are in the same thread, closer than
    //          256 in the same wave (lane shuffles); only stages with partners in another wave
    //          (2^log_n > 256) go through LDS.  Up to 512 events, wave 0 sorts alone (wave_sort).
    if (log_n <= 8) {
        if (wave == 0) wave_sort<4>(sm.ev, log_n, lane);
    } else if (log_n == 9) {
        if (wave == 0) wave_sort<8>(sm.ev, log_n, lane);
    } else {
        uint32_t key[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) key[r] = sm.ev[4 * tid + r];
#pragma unroll
        for (int kk = 1; kk <= 10; ++kk) {
            const int k = 1 << kk;
#pragma unroll
            for (int jj = kk - 1; jj >= 0; --jj) {
                if (kk > log_n) continue;  // uniform: the phases past the sort's size
                const int j = 1 << jj;
                if (j < 4) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if ((r & j) == 0) {
                            const bool up = ((4 * tid + r) & k) == 0;
                            const uint32_t x = key[r], y = key[r + j];
                            if ((x > y) == up) { key[r] = y; key[r + j] = x; }
                        }
                    }
                } else {
                    const int m = j >> 2;  // partner thread: tid ^ m
                    const bool up = ((4 * tid) & k) == 0, lower = (tid & m) == 0;
                    uint32_t other[4];
                    if (j < 256) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) other[r] = lane_xor(key[r], m);
                    } else {
                        __syncthreads();
#pragma unroll
                        for (int r = 0; r < 4; ++r) sm.ev[4 * tid + r] = key[r];
                        __syncthreads();
#pragma unroll
                        for (int r = 0; r < 4; ++r) other[r] = sm.ev[4 * (tid ^ m) + r];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t lo = key[r] < other[r] ? key[r] : other[r];
                        const uint32_t hi = key[r] < other[r] ? other[r] : key[r];
                        key[r] = lower == up ? lo : hi;
                    }
                }
            }
        }
        if (log_n > 8) __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.ev[4 * tid + r] = key[r];
    }
    __syncthreads();

    // ---- 2b. coefficients at the window's first pattern: A = sum d w^2, B0 = sum d |w| |q|,
    //          C0 = sum d q^2 (wave w takes environments w, w + 4, ...; lane l weights l and
    //          l + 64; a butterfly sums the wave)
    for (int e = wave; e < E; e += BLOCK / 64) {
        double A = 0.0, B = 0.0, C = 0.0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = lane + 64 * h;
            const double dv = (double)sm.d[e * G + i];
            const double wv = (double)sm.w[i];
            const double m = (double)(sm.magp[2 * i] + sm.magp[2 * i + 1]);
            A += dv * (wv * wv);
            B += dv * (fabs(wv) * m);
            C += dv * (m * m);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            A += lane_xor(A, o);
            B += lane_xor(B, o);
            C += lane_xor(C, o);
        }
        if (lane == 0) { sm.A[e] = A; sm.B0[e] = B; sm.C0[e] = C; }
    }
    __syncthreads();

    // ---- 2c/3a. per batch of 4 environments: block prefix sum of the coefficient changes
    //          (thread t owns events 4t..4t+3), then a walk over the thread's runs that folds
    //          the batch into each run's end values, lower bound and magnitude bound.  Run k
    //          starts at event k (after applying it) and ends one pattern before the next event;
    //          thread 0 also owns the run before the first event.  Only 8 coefficients and the
    //          per-run maxima stay in registers, whatever E is.
    const int e0 = 4 * tid;
    // Fixed run slots of this thread: slot 0 is the run before the first event (thread 0 only),
    // slot 1+k the run that starts at event e0+k (empty when the next event has the same pattern).
    uint32_t r_pat[5];  // first pattern | last pattern << 16
    auto r_lo = [&](int j) { return r_pat[j] & 0xFFFFu; };
    auto r_hi = [&](int j) { return r_pat[j] >> 16; };
    bool r_ok[5];
    double r_flo[5], r_fhi[5], r_lb[5];
    r_ok[0] = tid == 0;
    r_pat[0] = win_lo | (((n_ev > 0 ? (sm.ev[0] >> 11) : (win_hi + 1)) - 1) << 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int ev_k = e0 + k;
        const uint32_t t = ev_k < n_ev ? (sm.ev[ev_k] >> 11) : 0u;
        const uint32_t tn = ev_k + 1 < n_ev ? (sm.ev[ev_k + 1] >> 11) : (win_hi + 1);
        r_ok[k + 1] = ev_k < n_ev && tn > t;
        r_pat[k + 1] = t | (((tn - 1) & 0xFFFFu) << 16);
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        r_flo[j] = -__builtin_inf(); r_fhi[j] = -__builtin_inf(); r_lb[j] = -__builtin_inf();
    }
    // Magnitude bound of a run end, max_e (A_e + 2 B0_e s + C0_e s^2), taken from the maxima of
    // A, B0 and C0 over the environments: never smaller, so the allowances only grow.
    // Up to four environments there is one batch: each run's end values are final after its
    // fold and go straight into U (the upper bound from the run ends); beyond, the per-run
    // maxima are held over the batches and the magnitude maxima are read after them.
    constexpr bool ONE_BATCH = E <= 4;
    double am = 0.0, b2m = 0.0, cm = 0.0;
    auto read_mag = [&]() {
        double bm = 0.0;
        for (int e = 0; e < E; ++e) { am = fmax(am, sm.A[e]); bm = fmax(bm, sm.B0[e]); cm = fmax(cm, sm.C0[e]); }
        b2m = 2.0 * bm;
    };
    auto mag = [&](double s) { return __builtin_fma(s, __builtin_fma(cm, s, b2m), am); };
    if constexpr (ONE_BATCH) read_mag();
    if (tid == 0) {  // for the candidates' allowances (read after several barriers)
        double a0 = 0.0, b0 = 0.0, c0 = 0.0;
        for (int e = 0; e < E; ++e) { a0 = fmax(a0, sm.A[e]); b0 = fmax(b0, sm.B0[e]); c0 = fmax(c0, sm.C0[e]); }
        sm.mag_c[0] = a0; sm.mag_c[1] = 2.0 * b0; sm.mag_c[2] = c0;
    }
    double U = __builtin_inf();
#pragma unroll 1
    for (int eb = 0; eb < E; eb += 4) {
        constexpr int NB = E < 4 ? E : 4;  // environments in this batch
        double loc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) loc[v] = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (e0 + k < n_ev) {
                const uint32_t key = sm.ev[e0 + k];
                const int i = (key >> 4) & 127, c = key & 15;
                const double aw = fabs((double)sm.w[i]);
#pragma unroll
                for (int v = 0; v < NB; ++v) {
                    const double dv = (double)sm.d[(eb + v) * G + i];
                    loc[v] = __builtin_fma(-dv, aw, loc[v]);
                    loc[4 + v] = __builtin_fma(-dv, (double)(2 * c + 1), loc[4 + v]);
                }
            }
        }
        double inc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) inc[v] = wave_inclusive_sum_f64(loc[v]);
        __syncthreads();
        if (lane == 63) {
#pragma unroll
            for (int v = 0; v < 8; ++v) sm.wtot[wave][v] = inc[v];
        }
        __syncthreads();
        double cB[4], cC[4];  // coefficients at this thread's first run
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            double exB = lane_prev(inc[v]), exC = lane_prev(inc[4 + v]);
            if (lane == 0) { exB = 0.0; exC = 0.0; }
            for (int w2 = 0; w2 < wave; ++w2) { exB += sm.wtot[w2][v]; exC += sm.wtot[w2][4 + v]; }
            cB[v] = v < NB ? sm.B0[eb + v] + exB : 0.0;
            cC[v] = v < NB ? sm.C0[eb + v] + exC : 0.0;
        }
        // fold this batch into run slot j with the current coefficients
        auto fold = [&](int j) {
            const double slo = (double)half_bits_value(r_lo(j)), shi = (double)half_bits_value(r_hi(j));
#pragma unroll
            for (int v = 0; v < NB; ++v) {
                const double A = sm.A[eb + v], B = cB[v], C = cC[v], B2 = -2.0 * B;
                const double fl = __builtin_fma(slo, __builtin_fma(C, slo, B2), A);
                const double fh = __builtin_fma(shi, __builtin_fma(C, shi, B2), A);
                double sv;
                if (C > 0.0) {
                    // The vertex B/C need not be exact: an error d moves f(sv) by C d^2, and a
                    // relative error of 2^-40 in sv keeps that below 2^-80 of the magnitude bound,
                    // far inside the 2^-40 allowance.  Hardware reciprocal plus one Newton step.
                    const double r0 = __builtin_amdgcn_rcp(C);
                    const double r1 = __builtin_fma(r0, __builtin_fma(-C, r0, 1.0), r0);
                    sv = B * r1;
                    sv = sv < slo ? slo : (sv > shi ? shi : sv);
                } else {
                    sv = B > 0.0 ? shi : slo;  // linear (C = 0): B >= 0 decreases towards shi
                }
                const double fv = __builtin_fma(sv, __builtin_fma(C, sv, B2), A);
                r_flo[j] = fmax(r_flo[j], fl);
                r_fhi[j] = fmax(r_fhi[j], fh);
                r_lb[j] = fmax(r_lb[j], fv);
            }
            if constexpr (ONE_BATCH) {
                U = fmin(U, fmin(r_flo[j] + ERR_REL * mag(slo), r_fhi[j] + ERR_REL * mag(shi)));
                r_flo[j] = -__builtin_inf();  // dead from here on
                r_fhi[j] = -__builtin_inf();
            }
        };
        if (r_ok[0]) fold(0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (e0 + k < n_ev) {
                const uint32_t key = sm.ev[e0 + k];
                const int i = (key >> 4) & 127, c = key & 15;
                const double aw = fabs((double)sm.w[i]);
#pragma unroll
                for (int v = 0; v < NB; ++v) {
                    const double dv = (double)sm.d[(eb + v) * G + i];
                    cB[v] = __builtin_fma(-dv, aw, cB[v]);
                    cC[v] = __builtin_fma(-dv, (double)(2 * c + 1), cC[v]);
                }
            }
            if (r_ok[k + 1]) fold(k + 1);
        }
    }
    // upper bound U from the run ends, and each run's lower bound minus its error allowance
    if constexpr (!ONE_BATCH) {
        read_mag();
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const double slo = (double)half_bits_value(r_lo(j)), shi = (double)half_bits_value(r_hi(j));
            if (r_ok[j]) U = fmin(U, fmin(r_flo[j] + ERR_REL * mag(slo), r_fhi[j] + ERR_REL * mag(shi)));
        }
    }
    U = block_min_d(U, sm.redd);

    // ---- 3b. keep the runs whose lower bound can reach U, and recompute their coefficients
    //          directly from the codes at the run's first pattern
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        if (r_ok[j] && r_lb[j] - 2.0 * ERR_REL * mag((double)half_bits_value(r_hi(j))) <= U) {  // grows with s
            const int r = atomicAdd(&sm.n_runs, 1);
            if (r < RCAP) { sm.run_lo[r] = r_lo(j); sm.run_hi[r] = r_hi(j); }
        }
    }
    __syncthreads();
    const int n_runs = sm.n_runs;
    if (n_runs <= RCAP) {
        for (int j = tid; j < n_runs * G; j += BLOCK) {
            const int r = j / G, i = j % G;
            sm.qbuf[r][i] = (uint8_t)fabsf(exact_code_range(sm.w[i], half_bits_value(sm.run_lo[r]), qlo, qhi));
        }
        __syncthreads();
        // four consecutive threads per (run, environment), 32 weights each
        for (int j0 = 0; j0 < n_runs * E * 4; j0 += BLOCK) {
            const int j = j0 + tid;
            const bool live = j < n_runs * E * 4;
            const int r = j / (4 * E), e = (j / 4) % E, part = j % 4;
            double B = 0.0, C = 0.0;
            if (live) {
                for (int i = 32 * part; i < 32 * part + 32; ++i) {
                    const double dv = (double)sm.d[e * G + i];
                    const double q = (double)sm.qbuf[r][i];
                    B = __builtin_fma(dv, fabs((double)sm.w[i]) * q, B);
                    C = __builtin_fma(dv, q * q, C);
                }
            }
            B += lane_xor(B, 1);
            C += lane_xor(C, 1);
            B += lane_xor(B, 2);
            C += lane_xor(C, 2);
            if (live && part == 0) {
                sm.run_B[r][e] = B;
                sm.run_C[r][e] = C;
            }
        }
    }
    __syncthreads();

    // ---- 3c. candidates of the kept runs: ends, vertices and crossings on the upper envelope
    double M = __builtin_inf();
    if (n_runs <= RCAP) {
        constexpr int K = cand_items<E>();
        for (int j = tid; j < n_runs * K; j += BLOCK) {
            const int r = j / K;
            run_candidate_item<E>(sm, r, j % K, [&](uint32_t b) {
                double err;
                const double f = quad_run<E>(sm, r, (double)half_bits_value(b), err);
                M = fmin(M, f + err);
                const int j = atomicAdd(&sm.n_q, 1);
                if (j < QCAP) { sm.q_b[j] = b; sm.q_lo[j] = f - err; }
            });
        }
    }
    M = block_min_d(M, sm.redd);
    const int n_q = sm.n_q;
    const double Msel = M * (1.0 + SEL_SLACK);

    // ---- 3d. shortlist: every candidate whose lower bound reaches the best upper bound
    if (n_runs <= RCAP && n_q <= QCAP) {
        for (int j = tid; j < n_q; j += BLOCK) {
            if (sm.q_lo[j] <= Msel) {
                const int k = atomicAdd(&sm.n_cand, 1);
                if (k < CCAP) sm.cand_b[k] = sm.q_b[j];
            }
        }
    }
    __syncthreads();
    const int n = sm.n_cand;
    if (n_runs > RCAP || n_q > QCAP || n > CCAP || n == 0) {
        if (tid == 0) {
            const int j = atomicAdd(a.tie_count, 1);
            a.tie_list[j] = (int32_t)g;
        }
        return;
    }

    // ---- 4. direct binary64 rescoring (definition order) and the reduction
    // All threads form the terms of a batch of scales in LDS (free by now; the code, residual,
    // square and weighting as in the definition); one lane per (scale, environment) then adds
    // them in the definition's order, and lane butterflies take the maximum over the environments.
    constexpr int PT = CandSmem<E>::PER_T;
    for (int base = 0; base < n; base += PT) {
        const int nb = min(PT, n - base);
        for (int j = tid; j < nb * G; j += BLOCK) {
            const int c = j / G, i = j % G;
            const float sf = half_bits_value(sm.cand_b[base + c]);
            const double sq = (double)sf * (double)exact_code_range(sm.w[i], sf, qlo, qhi);
            const double t = (double)sm.w[i] - sq;
            const double t2 = t * t;
#pragma unroll
            for (int e = 0; e < E; ++e) sm.term[c][e][i] = (double)sm.d[e * G + i] * t2;
        }
        __syncthreads();
        if (wave == 0) {
            const int c = lane / E, e = lane % E;
            double F = 0.0;
            if (lane < nb * E) {
                const double* tr = sm.term[c][e];
#pragma unroll 16
                for (int i = 0; i < G; ++i) F = F + tr[i];
            }
#pragma unroll
            for (int o = 1; o < E; o <<= 1) {
                const double u = lane_xor(F, o);
                F = u > F ? u : F;
            }
            if (lane < nb * E && e == 0) sm.cand_F[base + c] = F;
        }
        __syncthreads();
    }
    if (tid < 64) {
        // wave 0: the lexicographic (value, bits) minimum, each lane over every 64th entry and
        // then a DPP reduction under the same order; the other patterns counted once each, and
        // whether one of them has the same value
        uint32_t bb = 0xFFFFFFFFu;
        double bF = __builtin_inf();
        for (int j = tid; j < n; j += 64) {
            const double v = sm.cand_F[j];
            const uint32_t b = sm.cand_b[j];
            if (v < bF || (v == bF && b < bb)) { bF = v; bb = b; }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double v = lane_xor(bF, o);
            const uint32_t b = lane_xor(bb, o);
            if (v < bF || (v == bF && b < bb)) { bF = v; bb = b; }
        }
        int distinct = 0;
        bool tie = false;
        for (int j0 = 0; j0 < n; j0 += 64) {
            const int j = j0 + tid;
            bool first = false, same = false;
            if (j < n) {
                const uint32_t bj = sm.cand_b[j];
                if (bj != bb) {
                    first = true;  // the first entry with this pattern
                    for (int k = 0; k < j; ++k)
                        if (sm.cand_b[k] == bj) { first = false; break; }
                    same = sm.cand_F[j] == bF;
                }
            }
            distinct += (int)__popcll(__ballot(first));
            tie = tie || __ballot(same) != 0;
        }
        if (tid == 0) {
            sm.win_b = bb;
            sm.win_F = bF;
            sm.win_state = tie ? 1 : 0;
            sm.win_count = distinct + 1;
        }
    }
    __syncthreads();
    if (sm.win_state) {
        if (tid == 0) {
            const int j = atomicAdd(a.tie_count, 1);
            a.tie_list[j] = (int32_t)g;
        }
        return;
    }
    const uint32_t b = sm.win_b;
    if (tid < Gn && a.codes) a.codes[g * Gn + tid] = (int8_t)exact_code_range(sm.w[tid], half_bits_value(b), qlo, qhi);
    if (tid == 0) {
        a.scales[g] = (uint16_t)b;
        if (a.objective) a.objective[g] = sm.win_F;
        if (a.flags) a.flags[g] = sm.win_count > 1 ? FLAG_NEAR_TIE : 0;
    }
}

// Workgroups per CU.  Up to E = 4 five (94 registers, no spills; five beat four by 11% on
// gfx950).  Six fit the LDS too (25.7 KB each at E = 4, with the unions in CandSmem) and ran 2%
// faster, but only by spilling 24 registers to scratch, about 370 MB of write traffic per
// 28,672-group launch.  At E = 16 three (with some spills) beat two by 13%.
constexpr int cand_min_blocks(int E) { return E <= 4 ? 6 : (E == 8 ? 3 : (E == 16 ? 3 : 1)); }

template <int E>
__global__ __launch_bounds__(BLOCK, cand_min_blocks(E)) void candidate_kernel(CandArgs a, int64_t group_offset) {
    __shared__ CandSmem<E> sm;
    candidate_group<E>(a, (int64_t)blockIdx.x + group_offset, sm);
}

__global__ void zero_tie_counter(int32_t* p, int32_t* q) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        *p = 0;
        if (q) *q = 0;
    }
}

template <int E>
hipError_t launch_e(const CandArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(zero_tie_counter, dim3(1), dim3(64), 0, st, a.tie_count, a.zero_also);
    const int64_t step = 1ll << 30;
    for (int64_t off = 0; off < a.n_groups; off += step) {
        const int64_t n = a.n_groups - off < step ? a.n_groups - off : step;
        hipLaunchKernelGGL(candidate_kernel<E>, dim3((unsigned)n), dim3(BLOCK), 0, st, a, off);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_candidate(const CandArgs& a_in, int E, hipStream_t st) {
    CandArgs a = a_in;
    a.E = E;
    switch (pad_envs(E)) {
        case 1: return launch_e<1>(a, st);
        case 2: return launch_e<2>(a, st);
        case 4: return launch_e<4>(a, st);
        case 8: return launch_e<8>(a, st);
        case 16: return launch_e<16>(a, st);
        case 32: return launch_e<32>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cqk
