/*
 * CPU oracle for exact minimax FP16 group-scale selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * It is a plain brute force written for a reader to check by eye against the
 * definition on the pages (CliffQuant repository README, "What CliffQuant
 * changes", displayed objective and the paragraph after it):
 *
 *   minimise over every positive finite IEEE binary16 scale s
 *       F(s) = max_e  sum_i d[e][i] * (w[i] - s*q_i(s))^2
 *   q_i(s) = clip(round-half-even(w[i]/s), qmin, qmax)   (rounding first, then clipping)
 *   an exact objective tie goes to the lower FP16 bit pattern.
 *
 * The quantizer is a parameter, as in the README's "Use the solver" call
 * (a QuantizerSpec with qmin and qmax, and a group of any length; the
 * configuration the pages run is qmin = -8, qmax = 7, groups of 128).
 * Every function below takes the group length G and the code range.
 *
 * The pooled policy (README, the opening question and the proxy table:
 * average the environments first, then choose the scale) minimises
 *       P(s) = (sum_e F_e(s)) / E
 * over the same grid with the same tie rule.
 *
 * Precision (the pages fix none): w/s is one IEEE binary32 division rounded to
 * nearest-even; rintf() then rounds half to even (default rounding mode);
 * the objective is summed in binary64, i = 0..G-1 in order, every operation
 * rounded separately (build with -ffp-contract=off, never -ffast-math).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC cq_oracle.c -o libcq_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MAX_G 1024         /* longest group the oracle takes */
#define MAX_E 64           /* most environments the oracle takes */
#define FIRST_BITS 0x0001u /* smallest positive subnormal binary16, 2^-24 */
#define LAST_BITS  0x7BFFu /* largest finite binary16, 65504 */

/* Value of a positive binary16 bit pattern, exactly, as a double
 * (IEEE 754 binary16: 5 exponent bits, bias 15, 10 fraction bits). */
double oracle_fp16_value(uint32_t bits)
{
    uint32_t ex = (bits >> 10) & 0x1Fu, man = bits & 0x3FFu;
    if (ex == 0)
        return ldexp((double)man, -24);               /* subnormal: man * 2^-24 */
    return ldexp((double)(1024u + man), (int)ex - 25); /* (1 + man/1024) * 2^(ex-15) */
}

/* q(w, s) = clip(round-half-even(fl32(w / s)), qmin, qmax). */
static int code_of(float w, float s, int qmin, int qmax)
{
    float x = w / s;
    float r = rintf(x);
    if (r < (float)qmin) r = (float)qmin;
    if (r > (float)qmax) r = (float)qmax;
    return (int)r;
}

/* sum_i d[i] * (w[i] - s*q[i])^2 in binary64, sequential in i = 0..G-1. */
static double env_error(const float *w, const float *d, int G, double s, const int *q)
{
    double F = 0.0;
    for (int i = 0; i < G; i++) {
        double t = (double)w[i] - s * (double)q[i];
        double t2 = t * t;
        F = F + (double)d[i] * t2;
    }
    return F;
}

/* Per-environment errors at one scale: out[e] for e < E; d is [E][G]. */
static void all_env_errors(const float *w, const float *d, int E, int G, int qmin, int qmax,
                           uint32_t bits, int *q, double *out)
{
    double s = oracle_fp16_value(bits);
    float sf = (float)s; /* exact: every binary16 value is a binary32 value */
    for (int i = 0; i < G; i++)
        q[i] = code_of(w[i], sf, qmin, qmax);
    for (int e = 0; e < E; e++)
        out[e] = env_error(w, d + (size_t)e * G, G, s, q);
}

/* 1 when every input of the group is finite and every diagonal entry is >= 0. */
static int group_ok(const float *w, const float *d, int E, int G)
{
    for (int i = 0; i < G; i++)
        if (!isfinite(w[i])) return 0;
    for (int j = 0; j < E * G; j++)
        if (!isfinite(d[j]) || d[j] < 0.0f) return 0;
    return 1;
}

/* 1 when the quantizer is one the oracle takes: 1 <= G <= MAX_G, 1 <= E <= MAX_E,
 * qmin <= 0 <= qmax, qmin < qmax, codes within int8. */
static int spec_ok(int E, int G, int qmin, int qmax)
{
    return E >= 1 && E <= MAX_E && G >= 1 && G <= MAX_G && qmin <= 0 && qmax >= 0 && qmin < qmax &&
           qmin >= -128 && qmax <= 127;
}

/*
 * Brute force over all 31,743 scales for n_groups groups of G weights.
 *   w: [n_groups][G]; d: [n_d][E][G], group g uses slice g % d_period.
 * Per group (nullable outputs skipped):
 *   mm_bits, mm_F1, mm_F2  -- minimax argmin bits, its objective, the smallest
 *                             objective over every other scale (runner-up);
 *   pl_bits, pl_P1, pl_P2  -- the same for the pooled objective
 *                             P(s) = (sum_e F_e(s)) / E, summed e = 0..E-1;
 *   codes [n_groups][G]    -- q at the minimax scale;
 *   ok                     -- 0 when the group has a non-finite or negative input
 *                             (then nothing else is written for it).
 * n_threads <= 0 leaves the OpenMP default.  Returns -1 (and writes nothing) for
 * a quantizer spec_ok() rejects, else 0.
 */
int oracle_solve(const float *w, const float *d, int64_t d_period, int E, int64_t n_groups,
                 int G, int qmin, int qmax,
                 uint16_t *mm_bits, double *mm_F1, double *mm_F2,
                 uint16_t *pl_bits, double *pl_P1, double *pl_P2,
                 int8_t *codes, uint8_t *ok, int n_threads)
{
    if (!spec_ok(E, G, qmin, qmax)) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t g = 0; g < n_groups; g++) {
        const float *wg = w + (size_t)g * G;
        const float *dg = d + (size_t)(g % d_period) * (size_t)E * G;
        int q[MAX_G];
        double Fe[MAX_E];
        if (ok) ok[g] = (uint8_t)group_ok(wg, dg, E, G);
        if (!group_ok(wg, dg, E, G)) continue;

        uint32_t best_b = 0, bestp_b = 0;
        double best = INFINITY, second = INFINITY, bestp = INFINITY, secondp = INFINITY;
        for (uint32_t b = FIRST_BITS; b <= LAST_BITS; b++) {
            all_env_errors(wg, dg, E, G, qmin, qmax, b, q, Fe);
            double F = Fe[0], P = Fe[0];
            for (int e = 1; e < E; e++) {
                if (Fe[e] > F) F = Fe[e];
                P = P + Fe[e];
            }
            P = P / (double)E;
            /* ascending b, strict '<': an exact tie keeps the lower bit pattern */
            if (F < best) { second = best; best = F; best_b = b; }
            else if (F < second) second = F;
            if (P < bestp) { secondp = bestp; bestp = P; bestp_b = b; }
            else if (P < secondp) secondp = P;
        }
        if (mm_bits) mm_bits[g] = (uint16_t)best_b;
        if (mm_F1) mm_F1[g] = best;
        if (mm_F2) mm_F2[g] = second;
        if (pl_bits) pl_bits[g] = (uint16_t)bestp_b;
        if (pl_P1) pl_P1[g] = bestp;
        if (pl_P2) pl_P2[g] = secondp;
        if (codes) {
            float sf = (float)oracle_fp16_value(best_b);
            for (int i = 0; i < G; i++)
                codes[(size_t)g * G + i] = (int8_t)code_of(wg[i], sf, qmin, qmax);
        }
    }
    return 0;
}

/* Codes of n weights at one scale: out[i] = q(w[i], s(bits)) in [qmin, qmax]. */
void oracle_codes(const float *w, int64_t n, uint32_t bits, int qmin, int qmax, int8_t *out)
{
    float sf = (float)oracle_fp16_value(bits);
    for (int64_t i = 0; i < n; i++)
        out[i] = (int8_t)code_of(w[i], sf, qmin, qmax);
}

/* Per-environment errors of each group at a given scale:
 * F_env[g][e] = sum_i d[e][i] (w[i] - s_g q_i(s_g))^2, s_g = bits[g].  Returns -1 for a
 * quantizer spec_ok() rejects. */
int oracle_env_errors(const float *w, const float *d, int64_t d_period, int E, int64_t n_groups,
                      int G, int qmin, int qmax, const uint16_t *bits, double *F_env, int n_threads)
{
    if (!spec_ok(E, G, qmin, qmax)) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t g = 0; g < n_groups; g++) {
        int q[MAX_G];
        all_env_errors(w + (size_t)g * G, d + (size_t)(g % d_period) * (size_t)E * G,
                       E, G, qmin, qmax, bits[g], q, F_env + (size_t)g * E);
    }
    return 0;
}

/* Objective curve of one group over every scale: F[b-1] = max_e F_e(b),
 * P[b-1] = pooled objective, for b = 1..0x7BFF (either output nullable). */
int oracle_curve(const float *w, const float *d, int E, int G, int qmin, int qmax, double *F, double *P)
{
    if (!spec_ok(E, G, qmin, qmax)) return -1;
    int q[MAX_G];
    double Fe[MAX_E];
    for (uint32_t b = FIRST_BITS; b <= LAST_BITS; b++) {
        all_env_errors(w, d, E, G, qmin, qmax, b, q, Fe);
        double m = Fe[0], p = Fe[0];
        for (int e = 1; e < E; e++) {
            if (Fe[e] > m) m = Fe[e];
            p = p + Fe[e];
        }
        if (F) F[b - 1] = m;
        if (P) P[b - 1] = p / (double)E;
    }
    return 0;
}

/* Round a non-negative float to binary16, nearest with ties to the even bit
 * pattern, by searching the grid for the nearest value (0 and +inf included).
 * Returns 0x7C00 (+inf) when x is at or beyond the overflow threshold
 * 65504 + 16 (half the last spacing, a tie that goes to the even pattern, inf). */
uint32_t oracle_fp16_round(float x)
{
    double xv = (double)x;
    if (xv >= 65520.0) return 0x7C00u;
    uint32_t best = 0;
    double best_dist = xv; /* distance to +0 */
    for (uint32_t b = FIRST_BITS; b <= LAST_BITS; b++) {
        double dist = fabs(xv - oracle_fp16_value(b));
        if (dist < best_dist || (dist == best_dist && (b & 1u) == 0u && (best & 1u) != 0u)) {
            best = b;
            best_dist = dist;
        }
    }
    return best;
}

/* AbsMax scale policy for groups of G weights and largest positive code qmax:
 * bits of fp16(fl32(max_i |w_i| / qmax)); a result of 0 becomes the smallest positive
 * scale and an overflow the largest finite one. */
void oracle_absmax(const float *w, int64_t n_groups, int G, int qmax, uint16_t *bits)
{
    for (int64_t g = 0; g < n_groups; g++) {
        float m = 0.0f;
        for (int i = 0; i < G; i++) {
            float a = fabsf(w[(size_t)g * G + i]);
            if (a > m) m = a;
        }
        uint32_t h = oracle_fp16_round(m / (float)qmax);
        if (h == 0) h = FIRST_BITS;
        if (h >= 0x7C00u) h = LAST_BITS;
        bits[g] = (uint16_t)h;
    }
}
