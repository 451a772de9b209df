// Candidate-set solver for gfx950.
//
// The pages' production solver "enumerates the analytically sufficient
// candidates induced by code transitions, quadratic vertices, and environment
// intersections" and sends a tie between direct-candidate objectives to an
// exhaustive-grid check (CliffQuant repository README, "What CliffQuant
// changes" and "Verification"; model card "Verification").  The steps here
// are our own design of that idea on the binary16 grid:
//
//  1. Code transitions.  For w_i != 0 and each c with |q_i| able to fall from
//     c+1 to c, the first grid pattern t where |q_i(s_t)| <= c.  The test
//     |q| <= c  <=>  |w| < (c+1/2) s  or  (|w| == (c+1/2) s and c even)  is
//     exact in binary32 ((c+1/2) s has at most 15 significant bits), and it is
//     monotone in s, so t is found by bisection over the 31,743 patterns.
//  2. Runs.  The events are sorted by t (bitonic sort in LDS); between two
//     consecutive event patterns every code is constant, so each environment
//     error is the quadratic f_e(s) = A_e - 2 B_e s + C_e s^2 with
//     B_e = sum d w q, C_e = sum d q^2.  A block-wide prefix sum over the
//     sorted events gives (B_e, C_e) of every run in binary64.
//  3. Candidates.  F = max_e f_e is convex on a run, so its grid minimum sits
//     next to the run's continuous minimiser: a run end, the vertex B_e/C_e
//     of an environment on top, or the crossing of two environments on top.
//     Runs whose lower bound max_e min f_e already exceeds the best end-point
//     value are skipped; in the rest every vertex and crossing on the upper
//     envelope is mapped to its grid neighbours (+-2 patterns of slack).
//  4. Reduction.  Every candidate within the proven error of the quadratic
//     form of the best one is rescored directly in binary64 in the same
//     summation order as the definition's plain sequential sum.  The lowest
//     value wins; if two distinct patterns tie bit for bit, or the shortlist
//     overflows, the group is handed to the exhaustive sweep (flag FALLBACK).
#include "device.h"
#include "launch.h"

namespace cqk {
namespace {

constexpr int MAX_EV = 1024;  // at most 7 (w > 0) or 8 (w < 0) transitions per weight
constexpr int CCAP = 256;
// |error of a quadratic-form value| <= ERR_REL * max_e (A_e + 2 B0_e s + C0_e s^2): the prefix
// sums run over <= 1024 events with partial sums in [0, B0_e] / [0, C0_e], plus the 128-term
// initial sums and the evaluation itself, i.e. < 1200 roundings of 2^-53 each.
constexpr double ERR_REL = 0x1p-40;
constexpr double SEL_SLACK = 1e-12;

template <int E>
struct CandSmem {
    float w[G];
    float d[E * G];  // [e][i]
    uint32_t ev[MAX_EV];
    uint8_t mag0[G];
    double A[E], B0[E], C0[E];
    double wtot[BLOCK / 64][8];
    double redd[BLOCK / 64];
    float redf[BLOCK / 64];
    uint32_t cand_b[CCAP];
    double cand_F[CCAP];
    double pairF[BLOCK];
    int n_ev;
    int n_cand;
    int overflow;
    uint32_t win_b;
    double win_F;
    int win_state;  // 0 ok, 1 tie or overflow -> exhaustive
    int win_count;
};

__device__ __forceinline__ double wave_min_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double u = __shfl_xor(v, o, 64);
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

// |q(w, s_b)| <= c  (exact, see the file comment)
__device__ __forceinline__ bool mag_at_most(float a, int c, uint32_t b) {
    const float hs = (float)(2 * c + 1) * 0.5f * half_bits_value(b);
    return a < hs || (a == hs && (c & 1) == 0);
}

template <int E>
struct Run {
    double B[E], C[E];
};

template <int E>
__device__ __forceinline__ double quad_at(const CandSmem<E>& sm, const double (&B)[E], const double (&C)[E],
                                          double s, double& err) {
    double F = sm.A[0] + s * (C[0] * s - 2.0 * B[0]), mag = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const double f = sm.A[e] + s * (C[e] * s - 2.0 * B[e]);
        F = f > F ? f : F;
        const double m = sm.A[e] + s * (sm.C0[e] * s + 2.0 * sm.B0[e]);
        mag = m > mag ? m : mag;
    }
    err = ERR_REL * mag;
    return F;
}

// lower bound of F over the continuous run [slo, shi] (before the error allowance)
template <int E>
__device__ __forceinline__ double run_lower_bound(const CandSmem<E>& sm, const double (&B)[E], const double (&C)[E],
                                                  double slo, double shi) {
    double lb = -__builtin_inf();
#pragma unroll
    for (int e = 0; e < E; ++e) {
        double s;
        if (C[e] > 0.0) {
            s = B[e] / C[e];
            s = s < slo ? slo : (s > shi ? shi : s);
        } else {
            s = B[e] > 0.0 ? shi : slo;  // linear (C = 0): B >= 0 decreases towards shi
        }
        const double f = sm.A[e] + s * (C[e] * s - 2.0 * B[e]);
        lb = f > lb ? f : lb;
    }
    return lb;
}

// Calls fn(b) for every candidate pattern of the run [blo, bhi]: the two ends, and the grid
// neighbours (+-2) of each vertex and each pairwise crossing that lies on the upper envelope.
template <int E, typename Fn>
__device__ __forceinline__ void run_candidates(const CandSmem<E>& sm, const double (&B)[E], const double (&C)[E],
                                               uint32_t blo, uint32_t bhi, Fn&& fn) {
    fn(blo);
    if (bhi != blo) fn(bhi);
    if (bhi - blo < 2) return;
    const double slo = (double)half_bits_value(blo), shi = (double)half_bits_value(bhi);
    auto near = [&](double s) {
        if (!(s >= slo && s <= shi)) return;
        const uint32_t b0 = f32_to_half_bits_rne((float)s);
        const uint32_t lo = b0 >= blo + 2 ? b0 - 2 : blo;
        const uint32_t hi = b0 + 2 <= bhi ? b0 + 2 : bhi;
        for (uint32_t b = lo; b <= hi; ++b)
            if (b != blo && b != bhi) fn(b);
    };
    auto on_top = [&](double s, int e1, int e2) {
        double err;
        const double F = quad_at<E>(sm, B, C, s, err);
        const double tol = 2.0 * err + SEL_SLACK * (F > 0.0 ? F : 0.0);
        const double f1 = sm.A[e1] + s * (C[e1] * s - 2.0 * B[e1]);
        const double f2 = sm.A[e2] + s * (C[e2] * s - 2.0 * B[e2]);
        return f1 >= F - tol && f2 >= F - tol;
    };
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (C[e] > 0.0) {
            const double v = B[e] / C[e];
            if (v >= slo && v <= shi && on_top(v, e, e)) near(v);
        }
    }
    for (int e1 = 0; e1 < E; ++e1) {
        for (int e2 = e1 + 1; e2 < E; ++e2) {
            const double a = C[e1] - C[e2], hb = B[e1] - B[e2], cc = sm.A[e1] - sm.A[e2];
            double r[2];
            int nr = 0;
            if (a == 0.0) {
                if (hb != 0.0) r[nr++] = cc / (2.0 * hb);
            } else {
                const double disc = hb * hb - a * cc;
                if (disc >= 0.0) {
                    const double sq = __builtin_sqrt(disc);
                    const double qq = hb + (hb >= 0.0 ? sq : -sq);
                    if (qq != 0.0) {
                        r[nr++] = qq / a;
                        r[nr++] = cc / qq;
                    } else {
                        r[nr++] = hb / a;
                    }
                }
            }
            for (int k = 0; k < nr; ++k)
                if (r[k] >= slo && r[k] <= shi && on_top(r[k], e1, e2)) near(r[k]);
        }
    }
}

template <int E>
__device__ void candidate_group(const CandArgs& a, int64_t g, CandSmem<E>& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* wg = a.w + g * G;
    const float* dg = a.d + (g % a.d_period) * (int64_t)(a.E * G);

    // ---- staging and input checks (environments a.E..E-1 are zero padding)
    if (tid < G) sm.w[tid] = wg[tid];
    for (int j = tid; j < E * G; j += BLOCK) sm.d[j] = j / G < a.E ? dg[j] : 0.0f;
    if (tid == 0) { sm.n_ev = 0; sm.n_cand = 0; sm.overflow = 0; }
    __syncthreads();
    float bad = 0.0f;
    if (tid < G && !__builtin_isfinite(sm.w[tid])) bad = 1.0f;
    for (int j = tid; j < E * G; j += BLOCK) {
        const float v = sm.d[j];
        if (!(v >= 0.0f) || !__builtin_isfinite(v)) bad = 1.0f;
    }
    if (block_max_f(bad, sm.redf) != 0.0f) {
        if (tid < G && a.codes) a.codes[g * G + tid] = 0;
        if (tid == 0) {
            a.scales[g] = 0;
            if (a.objective) a.objective[g] = __builtin_nan("");
            if (a.flags) a.flags[g] = FLAG_BAD_INPUT;
        }
        return;
    }

    // ---- 1. code transitions
    for (int j = tid; j < MAX_EV; j += BLOCK) sm.ev[j] = 0xFFFFFFFFu;
    __syncthreads();
    if (tid < G) {
        const float wi = sm.w[tid];
        const float aw = fabsf(wi);
        uint32_t keys[8];
        int nk = 0, m0 = 0;
        if (wi != 0.0f) {
            const int cmax = wi > 0.0f ? 6 : 7;
            for (int c = 0; c <= cmax; ++c) {
                if (mag_at_most(aw, c, BITS_FIRST)) continue;
                ++m0;  // the magnitude at the first pattern exceeds c
                if (!mag_at_most(aw, c, BITS_LAST)) continue;
                uint32_t lo = BITS_FIRST, hi = BITS_LAST;  // false at lo, true at hi
                while (hi - lo > 1) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (mag_at_most(aw, c, mid)) hi = mid;
                    else lo = mid;
                }
                keys[nk++] = (hi << 11) | ((uint32_t)tid << 4) | (uint32_t)c;
            }
        }
        sm.mag0[tid] = (uint8_t)m0;
        if (nk) {
            const int base = atomicAdd(&sm.n_ev, nk);
            for (int k = 0; k < nk; ++k) sm.ev[base + k] = keys[k];
        }
    }
    __syncthreads();
    const int n_ev = sm.n_ev;

    // ---- 2a. sort the events (bitonic, ascending; padding sorts last)
    int N = 2;
    while (N < n_ev) N <<= 1;
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int idx = tid; idx < N / 2; idx += BLOCK) {
                const int p = 2 * idx - (idx & (j - 1));
                const int q = p + j;
                const uint32_t x = sm.ev[p], y = sm.ev[q];
                const bool up = (p & k) == 0;
                if ((x > y) == up) { sm.ev[p] = y; sm.ev[q] = x; }
            }
            __syncthreads();
        }
    }

    // ---- 2b. initial coefficients at the first pattern
    if (tid < E) {
        double A = 0.0, B = 0.0, C = 0.0;
        for (int i = 0; i < G; ++i) {
            const double dv = (double)sm.d[tid * G + i];
            const double wv = (double)sm.w[i];
            const double m = (double)sm.mag0[i];
            A += dv * (wv * wv);
            B += dv * (fabs(wv) * m);
            C += dv * (m * m);
        }
        sm.A[tid] = A; sm.B0[tid] = B; sm.C0[tid] = C;
    }
    __syncthreads();

    // ---- 2c. block prefix sum of the coefficient changes; thread t owns events 4t..4t+3
    double curB[E], curC[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { curB[e] = sm.B0[e]; curC[e] = sm.C0[e]; }
    const int e0 = 4 * tid;
    for (int eb = 0; eb < E; eb += 4) {
        double loc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) loc[v] = 0.0;
        for (int k = e0; k < e0 + 4 && k < n_ev; ++k) {
            const uint32_t key = sm.ev[k];
            const int i = (key >> 4) & 127, c = key & 15;
            const double aw = fabs((double)sm.w[i]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (eb + v < E) {
                    const double dv = (double)sm.d[(eb + v) * G + i];
                    loc[v] -= dv * aw;
                    loc[4 + v] -= dv * (double)(2 * c + 1);
                }
            }
        }
        double inc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            double x = loc[v];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            inc[v] = x;
        }
        __syncthreads();
        if (lane == 63) {
#pragma unroll
            for (int v = 0; v < 8; ++v) sm.wtot[wave][v] = inc[v];
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            double ex = __shfl_up(inc[v], 1, 64);
            if (lane == 0) ex = 0.0;
            for (int w2 = 0; w2 < wave; ++w2) ex += sm.wtot[w2][v];
            inc[v] = ex;  // exclusive prefix at this thread's first event
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (eb + v < E) {
                curB[eb + v] += inc[v];
                curC[eb + v] += inc[4 + v];
            }
        }
    }

    // Walk this thread's runs: run k starts at event k (after applying it) and ends one pattern
    // before the next event; thread 0 also owns the run before the first event.
    auto walk = [&](auto&& on_run) {
        double B[E], C[E];
#pragma unroll
        for (int e = 0; e < E; ++e) { B[e] = curB[e]; C[e] = curC[e]; }
        if (tid == 0) {
            const uint32_t t0 = n_ev > 0 ? (sm.ev[0] >> 11) : (BITS_LAST + 1);
            on_run(B, C, BITS_FIRST, t0 - 1);
        }
        for (int k = e0; k < e0 + 4 && k < n_ev; ++k) {
            const uint32_t key = sm.ev[k];
            const int i = (key >> 4) & 127, c = key & 15;
            const double aw = fabs((double)sm.w[i]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double dv = (double)sm.d[e * G + i];
                B[e] -= dv * aw;
                C[e] -= dv * (double)(2 * c + 1);
            }
            const uint32_t t = key >> 11;
            const uint32_t tn = k + 1 < n_ev ? (sm.ev[k + 1] >> 11) : (BITS_LAST + 1);
            if (tn > t) on_run(B, C, t, tn - 1);
        }
    };

    // ---- 3a. upper bound U from the run ends
    double U = __builtin_inf();
    walk([&](const double (&B)[E], const double (&C)[E], uint32_t blo, uint32_t bhi) {
        double err;
        const double f0 = quad_at<E>(sm, B, C, (double)half_bits_value(blo), err);
        U = fmin(U, f0 + err);
        const double f1 = quad_at<E>(sm, B, C, (double)half_bits_value(bhi), err);
        U = fmin(U, f1 + err);
    });
    U = block_min_d(U, sm.redd);

    // ---- 3b. candidates of the runs that can hold the minimum: their best upper bound
    auto survives = [&](const double (&B)[E], const double (&C)[E], uint32_t blo, uint32_t bhi) {
        const double slo = (double)half_bits_value(blo), shi = (double)half_bits_value(bhi);
        double err;
        quad_at<E>(sm, B, C, shi, err);  // the magnitude bound grows with s
        return run_lower_bound<E>(sm, B, C, slo, shi) - 2.0 * err <= U;
    };
    double M = __builtin_inf();
    walk([&](const double (&B)[E], const double (&C)[E], uint32_t blo, uint32_t bhi) {
        if (!survives(B, C, blo, bhi)) return;
        run_candidates<E>(sm, B, C, blo, bhi, [&](uint32_t b) {
            double err;
            const double f = quad_at<E>(sm, B, C, (double)half_bits_value(b), err);
            M = fmin(M, f + err);
        });
    });
    M = block_min_d(M, sm.redd);
    const double Msel = M * (1.0 + SEL_SLACK);

    // ---- 3c. shortlist: every candidate whose lower bound reaches the best upper bound
    walk([&](const double (&B)[E], const double (&C)[E], uint32_t blo, uint32_t bhi) {
        if (!survives(B, C, blo, bhi)) return;
        run_candidates<E>(sm, B, C, blo, bhi, [&](uint32_t b) {
            double err;
            const double f = quad_at<E>(sm, B, C, (double)half_bits_value(b), err);
            if (f - err <= Msel) {
                const int j = atomicAdd(&sm.n_cand, 1);
                if (j < CCAP) sm.cand_b[j] = b;
            }
        });
    });
    __syncthreads();
    const int n = sm.n_cand;
    if (n > CCAP || n == 0) {
        if (tid == 0) {
            const int j = atomicAdd(a.tie_count, 1);
            a.tie_list[j] = (int32_t)g;
        }
        return;
    }

    // ---- 4. direct binary64 rescoring (definition order) and the reduction
    constexpr int PER = BLOCK / E;
    for (int base = 0; base < n; base += PER) {
        const int nb = min(PER, n - base);
        if (tid < nb * E) {
            const int j = base + tid / E, e = tid % E;
            const double s = (double)half_bits_value(sm.cand_b[j]);
            sm.pairF[tid] = env_error_f64(sm.w, sm.d + e * G, 1, s, 1.0 / s);
        }
        __syncthreads();
        if (tid < nb) {
            double F = sm.pairF[tid * E];
#pragma unroll
            for (int e = 1; e < E; ++e) F = sm.pairF[tid * E + e] > F ? sm.pairF[tid * E + e] : F;
            sm.cand_F[base + tid] = F;
        }
        __syncthreads();
    }
    if (tid == 0) {
        uint32_t bb = 0xFFFFFFFFu;
        double bF = __builtin_inf();
        for (int j = 0; j < n; ++j) {
            const double v = sm.cand_F[j];
            const uint32_t b = sm.cand_b[j];
            if (v < bF || (v == bF && b < bb)) { bF = v; bb = b; }
        }
        int tie = 0, distinct = 0;
        for (int j = 0; j < n; ++j) {
            if (sm.cand_b[j] == bb) continue;
            bool first = true;  // count each other pattern once
            for (int k = 0; k < j; ++k) if (sm.cand_b[k] == sm.cand_b[j]) { first = false; break; }
            if (first) ++distinct;
            if (sm.cand_F[j] == bF) tie = 1;
        }
        sm.win_b = bb;
        sm.win_F = bF;
        sm.win_state = tie;
        sm.win_count = distinct + 1;
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
    if (tid < G && a.codes) a.codes[g * G + tid] = (int8_t)exact_code(sm.w[tid], half_bits_value(b));
    if (tid == 0) {
        a.scales[g] = (uint16_t)b;
        if (a.objective) a.objective[g] = sm.win_F;
        if (a.flags) a.flags[g] = sm.win_count > 1 ? FLAG_NEAR_TIE : 0;
    }
}

template <int E>
__global__ __launch_bounds__(BLOCK) void candidate_kernel(CandArgs a, int64_t group_offset) {
    __shared__ CandSmem<E> sm;
    candidate_group<E>(a, (int64_t)blockIdx.x + group_offset, sm);
}

__global__ void zero_tie_counter(int32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

template <int E>
hipError_t launch_e(const CandArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(zero_tie_counter, dim3(1), dim3(64), 0, st, a.tie_count);
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
