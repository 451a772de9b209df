/*
 * cq.h -- C ABI of the MI355X (gfx950) library for exact minimax FP16
 * group-scale selection in symmetric 4-bit, group-size-128 weight
 * quantization, and GPTQ-v1 packing of the result.
 *
 * The operation (CliffQuant repository README, "What CliffQuant changes",
 * displayed objective and the paragraph after it): for one group of 128
 * weights w_i and E environment diagonals d_{e,i} >= 0, choose the positive
 * finite IEEE binary16 scale s (bit patterns 0x0001..0x7BFF, 31,743 values)
 * that minimises
 *        F(s) = max_e sum_i d_{e,i} (w_i - s q_i(s))^2,
 *        q_i(s) = clip(round-half-even(w_i / s), -8, 7)   (round, then clip),
 * an exact objective tie going to the lower binary16 bit pattern.  The
 * quotient w_i/s is taken as one correctly rounded binary32 division and the
 * reported objective is summed in binary64, i = 0..127 in order, each
 * operation rounded on its own.
 *
 * Conventions for every entry point:
 *  - Array arguments are DEVICE pointers (HIP global memory on the current
 *    device) owned by the caller; the library never frees or keeps them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on that stream and return after enqueueing; the
 *    outputs are valid once the stream has reached that point.
 *  - No entry point allocates device memory: scratch space comes from the
 *    caller's `workspace` (device memory, 256-byte aligned, at least
 *    cq_workspace_size(...) bytes, not shared between calls that may overlap).
 *  - Pointers to float32 inputs (w, d) and to int8 codes must be 16-byte
 *    aligned, other arrays naturally aligned (torch allocations are).
 *  - Argument errors are reported before anything is enqueued; data errors
 *    (non-finite weights or diagonals, negative diagonals) are reported per
 *    group through CQ_FLAG_BAD_INPUT, never through the status.
 *  - The library keeps no state between calls; distinct streams may be used
 *    from distinct host threads at once.
 *
 * Layouts:
 *   w      float32 [n_groups][128]   group g: 128 consecutive input channels
 *                                    of one output row (row-major [out][in]
 *                                    matrices give g = row*(in/128) + chunk).
 *   d      float32 [n_d][E][128]     group g uses slice (g % d_period); a
 *                                    matrix has d_period = in/128 (groups
 *                                    inherit the diagonals of their input
 *                                    channels), per-group diagonals have
 *                                    d_period = n_groups.
 *   scales uint16  [n_groups]        binary16 bit patterns (0x0001..0x7BFF).
 *   codes  int8    [n_groups][128]   q_i in [-8, 7] at the chosen scale.
 */
#ifndef CQ_H
#define CQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CQ_ABI_VERSION 2
#define CQ_GROUP 128
#define CQ_MAX_GROUP 256 /* longest group cq_quantize_groups_spec takes */
#define CQ_MAX_ENVS 32
#define CQ_MAX_POLICIES 64
#define CQ_MAX_BOOT (1 << 20)

/* Status codes. */
#define CQ_OK 0
#define CQ_EINVAL (-1)       /* null required pointer, bad size or enum */
#define CQ_EWORKSPACE (-2)   /* workspace missing, misaligned or too small */
#define CQ_EHIP (-3)         /* a HIP launch failed (hipGetLastError) */
#define CQ_EUNSUPPORTED (-4) /* valid arguments this entry point does not serve */
#define CQ_ELIMIT (-5)       /* more groups than cq_quantize_groups_noalloc's fixed scratch holds */

/* Solvers (cq_quantize_groups `method`); all three return the same result.
 *  CQ_EXHAUSTIVE  the independent full-grid enumerator (README, "What CliffQuant changes": a
 *                 separate reference evaluates every one of the 31,743 binary16 values): the
 *                 binary32 objective of every weight at every scale, then binary64 rescoring of
 *                 every scale its error bound cannot rule out.  No scale is skipped.
 *  CQ_CANDIDATE   the production solver's idea (same section): candidates from code transitions,
 *                 quadratic vertices and environment intersections; groups whose direct
 *                 candidates tie exactly go to CQ_BOUNDED (CQ_EXHAUSTIVE for another quantizer;
 *                 README and model card, "Verification").
 *  CQ_BOUNDED     branch and bound over the grid: stops at the first scale >= 2 max|w| (every
 *                 larger one ties with it exactly and loses to it), takes chunk-constant codes in
 *                 closed form and skips chunks of scales whose proven lower bound exceeds the
 *                 best value screened; the outputs are those of the full grid. */
#define CQ_EXHAUSTIVE 0
#define CQ_CANDIDATE 1
#define CQ_BOUNDED 2

/* Baseline policies (cq_baseline_scales `which`), the two the pages compare the minimax
 * scales with (CliffQuant README, the opening question and the "Held-out reconstruction
 * proxy" table; model card, "Held-out reconstruction proxy"):
 *  CQ_ABSMAX       the matched AbsMax checkpoint's scale, s = fp16(fl32(max_i |w_i| / 7));
 *                  0 -> 0x0001, overflow -> 0x7BFF.
 *  CQ_POOLED_WMSE  the environments averaged before the scale is chosen: minimise
 *                  P(s) = (1/E) sum_e F_e(s) over the same grid with the same tie rule. */
#define CQ_ABSMAX 0
#define CQ_POOLED_WMSE 1

/* Per-group flag bits (cq_quantize_groups `flags`). */
#define CQ_FLAG_BAD_INPUT 1u  /* non-finite w or d, or d < 0: scale 0, codes 0, objective NaN */
#define CQ_FLAG_NEAR_TIE 2u   /* more than one scale survived the binary32 screen */
#define CQ_FLAG_EXACT_TIE 4u  /* the winner's binary64 objective equals another scale's */
#define CQ_FLAG_FALLBACK 8u   /* the candidate solver handed the group to the exhaustive one */
#define CQ_FLAG_FP64_SWEEP 16u /* decided by a full binary64 sweep (screen inconclusive) */

/* ABI version of the loaded library (CQ_ABI_VERSION). */
int32_t cq_abi_version(void);

/* Static description of a status code. */
const char *cq_status_string(int32_t status);

/* Bytes of workspace cq_quantize_groups (and cq_quantize_groups_spec) needs for
 * `method`, E and n_groups (any group length); CQ_EXHAUSTIVE and CQ_BOUNDED
 * return the same size, which is also what cq_baseline_scales with
 * CQ_POOLED_WMSE needs.  Returns 0 for invalid arguments. */
size_t cq_workspace_size(int32_t method, int32_t E, int64_t n_groups);

/*
 * Minimax scale, codes and objective for n_groups groups.
 *   method       CQ_EXHAUSTIVE, CQ_CANDIDATE or CQ_BOUNDED; all return the same result.
 *   scales       out, required.
 *   codes        out, nullable.
 *   objective    out, nullable: F(s) at the chosen scale, binary64.
 *   flags        out, nullable: CQ_FLAG_* bits.
 *   pooled_scales / pooled_objective
 *                out, nullable, CQ_EXHAUSTIVE only (else CQ_EUNSUPPORTED):
 *                the pooled-WMSE policy decided in the same sweep.
 * E in 1..32, n_groups >= 0 (0 enqueues nothing), 1 <= d_period.
 * The binary32 screen is followed by binary64 rescoring of every scale the
 * screen's error bound cannot rule out, so the pick equals the binary64
 * argmin over all scales with the lower-bit-pattern tie rule.
 */
int32_t cq_quantize_groups(const float *w, const float *d, int64_t d_period, int32_t E,
                           int64_t n_groups, int32_t method,
                           uint16_t *scales, int8_t *codes, double *objective, uint8_t *flags,
                           uint16_t *pooled_scales, double *pooled_objective,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * cq_quantize_groups for another quantizer (CliffQuant README, "Use the solver": the
 * solver takes a quantizer specification with qmin and qmax and a group of any length,
 * its example four weights): codes q_i = clip(round-half-even(w_i / s), qmin, qmax),
 * groups of group_len weights.
 *   w      float32 [n_groups][group_len], 4-byte aligned.
 *   d      float32 [n_d][E][group_len], 4-byte aligned; group g uses slice g % d_period.
 *   codes  out, nullable, int8 [n_groups][group_len].
 * 1 <= group_len <= CQ_MAX_GROUP, -128 <= qmin <= 0 <= qmax <= 127, qmin < qmax (else
 * CQ_EINVAL).  (128, -8, 7) is cq_quantize_groups itself, with its alignment rules.  Any
 * other quantizer is served by CQ_EXHAUSTIVE, and by CQ_CANDIDATE when group_len <= 128 and
 * -8 <= qmin, qmax <= 8 (its tied groups then go to CQ_EXHAUSTIVE, flag CQ_FLAG_FALLBACK;
 * pooled outputs CQ_EUNSUPPORTED); other methods and quantizers return CQ_EUNSUPPORTED.
 * Other outputs, workspace and errors as for cq_quantize_groups.
 */
int32_t cq_quantize_groups_spec(const float *w, const float *d, int32_t group_len, int32_t qmin, int32_t qmax,
                                int64_t d_period, int32_t E, int64_t n_groups, int32_t method,
                                uint16_t *scales, int8_t *codes, double *objective, uint8_t *flags,
                                uint16_t *pooled_scales, double *pooled_objective,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * cq_quantize_groups for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments without
 * the workspace, and the same results.  The scratch space lives in a fixed array of the library
 * on each GPU (about 12.6 MB, held until the process ends), found at the first call on that
 * device; the call itself allocates nothing.
 *   n_groups  0..CQ_NOALLOC_MAX_GROUPS, else CQ_ELIMIT before anything is enqueued.
 * Every call on one GPU uses that GPU's one array; the kernels clear what must start at zero,
 * but calls that overlap on one GPU (other streams, other host threads) race.
 */
#define CQ_NOALLOC_MAX_GROUPS (1 << 20)
int32_t cq_quantize_groups_noalloc(const float *w, const float *d, int64_t d_period, int32_t E,
                                   int64_t n_groups, int32_t method,
                                   uint16_t *scales, int8_t *codes, double *objective, uint8_t *flags,
                                   uint16_t *pooled_scales, double *pooled_objective, void *stream);

/*
 * Baseline scale policies.
 *   CQ_ABSMAX       d may be NULL when objective is NULL; no workspace needed.
 *   CQ_POOLED_WMSE  the argmin of P(s) over every scale (the CQ_BOUNDED search of P);
 *                   workspace as for cq_workspace_size(CQ_EXHAUSTIVE, E, n_groups).
 *   objective  nullable: for CQ_ABSMAX the worst-environment objective F at
 *              the AbsMax scale; for CQ_POOLED_WMSE the pooled objective P.
 */
int32_t cq_baseline_scales(const float *w, const float *d, int64_t d_period, int32_t E,
                           int64_t n_groups, int32_t which,
                           uint16_t *scales, int8_t *codes, double *objective,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * cq_baseline_scales for another quantizer (CliffQuant README, "Use the solver": the solver takes
 * a quantizer specification; the baselines as in cq_baseline_scales).  w is [n_groups][group_len],
 * d [n_d][E][group_len]; codes in [qmin, qmax] as for cq_quantize_groups_spec.
 *   CQ_ABSMAX       s = fp16(fl32(max_i |w_i| / qmax)), 0 -> 0x0001, overflow -> 0x7BFF (the
 *                   largest magnitude maps to the largest positive code, as max|w| / 7 does for
 *                   [-8, 7]); needs qmax >= 1, else CQ_EINVAL.  workspace unused.
 *   CQ_POOLED_WMSE  the pooled policy of the full-grid search (cq_quantize_groups_spec's pooled
 *                   outputs alone); workspace as cq_workspace_size(CQ_EXHAUSTIVE, E, n_groups).
 * codes (nullable) are those of the chosen scale; objective (nullable) max_e F_e (AbsMax) or
 * (1/E) sum_e F_e (pooled), binary64.  Limits as for cq_quantize_groups_spec; w and d 4-byte
 * aligned.  The pages' quantizer (group_len 128, [-8, 7]) is cq_baseline_scales itself, with its
 * alignment rules.
 */
int32_t cq_baseline_scales_spec(const float *w, const float *d, int32_t group_len, int32_t qmin, int32_t qmax,
                                int64_t d_period, int32_t E, int64_t n_groups, int32_t which, uint16_t *scales,
                                int8_t *codes, double *objective, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * GPTQ-v1 packing of one [out][in] matrix (Qwen3.5-0.8B-Base-CliffQuant-
 * W4A16-G128 model card, "Quantization configuration": GPTQ v1, 4-bit,
 * group size 128, symmetric).
 *   codes       int8 [out][in], values in [-8, 7] (the cq_quantize_groups
 *               codes of the matrix's groups, in group order).
 *   grp_scales  uint16 [out][in/128] (the matrix's per-group scales).
 *   qweight     out, int32 [in/8][out]: nibble j (bits 4j..4j+3) of
 *               qweight[r][o] is codes[o][8r+j] + 8.
 *   scales      out, uint16 [in/128][out]: scales[c][o] = grp_scales[o][c].
 * out >= 0, in >= 0, in % 128 == 0.  Codes outside [-8, 7] are packed
 * modulo 16 (the caller guarantees the range).
 */
int32_t cq_pack_gptq_v1(const int8_t *codes, const uint16_t *grp_scales, int64_t out, int64_t in,
                        int32_t *qweight, uint16_t *scales, void *stream);

/*
 * GPTQ-v1 packing of one [out][in] matrix for another quantizer (CliffQuant README, "Use the
 * solver": the solver takes a quantizer specification; the model card's format, "Quantization
 * configuration", with the field width and the group length as parameters).
 *   codes       int8 [out][in], values in [-2^(bits-1), 2^(bits-1) - 1].
 *   grp_scales  uint16 [out][in/group_len] (binary16 bit patterns).
 *   qweight     out, int32 [in*bits/32][out]: field j (bits j*bits .. j*bits + bits - 1, low
 *               field first) of qweight[r][o] is codes[o][(32/bits) r + j] + 2^(bits-1).
 *   scales      out, uint16 [in/group_len][out]: scales[c][o] = grp_scales[o][c].
 * bits in {2, 4, 8}; 1 <= group_len <= CQ_MAX_GROUP; out >= 0, in >= 0, in a multiple of
 * group_len and of 32/bits; else CQ_EINVAL (bits = 4 with group_len = 128 gives what
 * cq_pack_gptq_v1 gives).  Codes outside the range are packed modulo 2^bits (the caller
 * guarantees the range).  codes and qweight 4-byte aligned, grp_scales and scales 2-byte.
 * Two launches on `stream`.
 */
int32_t cq_pack_gptq_v1_spec(const int8_t *codes, const uint16_t *grp_scales, int64_t out, int64_t in,
                             int32_t bits, int32_t group_len, int32_t *qweight, uint16_t *scales, void *stream);

/*
 * GPTQ-v1 packing of n_mats matrices in one launch (model card, "Verification": the packed
 * checkpoint holds 150 module-buffer sets, each unpacked again; "Quantization configuration":
 * GPTQ v1, 4-bit, group size 128, symmetric).  Matrix k has shape outs[k] x ins[k]; every array
 * holds the matrices back to back in order, each block exactly what cq_pack_gptq_v1 takes or
 * writes for that matrix alone:
 *   codes       int8 [sum_k outs[k] * ins[k]], matrix k from offset sum_{j<k} outs[j] * ins[j].
 *   grp_scales  uint16, matrix k from offset sum_{j<k} outs[j] * ins[j] / 128.
 *   qweight     out, int32, matrix k's [ins[k]/8][outs[k]] from offset sum_{j<k} outs[j] * ins[j] / 8.
 *   scales      out, uint16, matrix k's [ins[k]/128][outs[k]] from offset sum_{j<k} outs[j] * ins[j] / 128.
 *   outs, ins   HOST int64 arrays [n_mats], read before the call returns.
 * 0 <= n_mats <= CQ_MAX_PACK_MATRICES; every ins[k] a multiple of 128 (ins[k] / 128 <= 65535);
 * shapes below 2^31 each and 2^46 elements in all; else CQ_EINVAL.  Alignment as for
 * cq_pack_gptq_v1.
 */
#define CQ_MAX_PACK_MATRICES 256
int32_t cq_pack_gptq_v1_multi(const int8_t *codes, const uint16_t *grp_scales, int32_t n_mats,
                              const int64_t *outs, const int64_t *ins, int32_t *qweight, uint16_t *scales,
                              void *stream);

/*
 * Module-macro worst-environment weighted MSE (Qwen3.5-0.8B-Base-CliffQuant-
 * W4A16-G128 model card, "Held-out reconstruction proxy"; CliffQuant README,
 * "Held-out reconstruction proxy").
 *   per group  p_g = max_e (1/128) sum_i d_eval_{e,i} (w_i - s_g q_i(s_g))^2
 *   per module mean of p_g over groups [module_offsets[m], module_offsets[m+1])
 *   macro      mean over the n_modules module means.
 *   scales          device uint16 [n_groups] binary16 patterns (0x0001..0x7BFF).
 *   module_offsets  device int64 [n_modules+1], non-decreasing, first 0, last
 *                   n_groups; a module whose range is empty or out of bounds
 *                   gets NaN.
 *   module_mean     out, double [n_modules].   macro  out, double [1].
 *   per_group       out, nullable, double [n_groups].
 * workspace: cq_proxy_workspace_size(n_groups) bytes.
 */
size_t cq_proxy_workspace_size(int64_t n_groups);
int32_t cq_proxy_worst_env_wmse(const float *w, const float *d_eval, int64_t d_period, int32_t E,
                                int64_t n_groups, const uint16_t *scales,
                                const int64_t *module_offsets, int32_t n_modules,
                                double *module_mean, double *macro, double *per_group,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same proxy for n_policies scale policies of the same groups in one call
 * (the model card compares the minimax scales with the AbsMax baseline on this
 * proxy: Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Held-out
 * reconstruction proxy"); w and d_eval are read once for all of them, and each
 * policy's results equal those of a cq_proxy_worst_env_wmse call on its own
 * scales bit for bit.
 *   scales       device uint16 [n_policies][n_groups].
 *   module_mean  out, double [n_policies][n_modules].
 *   macro        out, double [n_policies].
 *   per_group    out, nullable, double [n_policies][n_groups].
 * 1 <= n_policies <= CQ_MAX_POLICIES.  workspace (only when per_group is
 * NULL): cq_proxy_workspace_size(n_policies * n_groups) bytes.
 */
int32_t cq_proxy_worst_env_wmse_multi(const float *w, const float *d_eval, int64_t d_period, int32_t E,
                                      int64_t n_groups, int32_t n_policies, const uint16_t *scales,
                                      const int64_t *module_offsets, int32_t n_modules,
                                      double *module_mean, double *macro, double *per_group,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * cq_proxy_worst_env_wmse_multi for another quantizer (CliffQuant README, "Use the solver": a
 * quantizer specification; the proxy as in cq_proxy_worst_env_wmse, with 1/group_len for the
 * pages' 1/128: the mean over the group's weights).  w is [n_groups][group_len], d_eval
 * [n_d][E][group_len]; codes in [qmin, qmax].  Arguments, limits and workspace as for
 * cq_proxy_worst_env_wmse_multi (w and d_eval 4-byte aligned); the pages' quantizer is
 * cq_proxy_worst_env_wmse_multi itself, with its alignment rules.  Per-group sums run over the group's 16 lanes (each lane's weights in index order, then a
 * fixed butterfly): within rounding of the sequential definition, bit-identical across runs.
 */
int32_t cq_proxy_worst_env_wmse_multi_spec(const float *w, const float *d_eval, int32_t group_len, int32_t qmin,
                                           int32_t qmax, int64_t d_period, int32_t E, int64_t n_groups,
                                           int32_t n_policies, const uint16_t *scales,
                                           const int64_t *module_offsets, int32_t n_modules, double *module_mean,
                                           double *macro, double *per_group, void *workspace,
                                           size_t workspace_bytes, void *stream);

/*
 * W4A16 matmul over the GPTQ-v1 tensors, the consumer check of the packed
 * output (Qwen3.5-0.8B-Base-CliffQuant-W4A16-G128 model card, "Quantization
 * configuration": GPTQ v1, 4 bits, group 128, symmetric, 16-bit activations).
 *   x        device uint16 [M][in]: bfloat16 bit patterns, 16-byte aligned.
 *   qweight  device int32 [in/8][out], scales device uint16 [in/128][out]
 *            (binary16 bit patterns): the cq_pack_gptq_v1 outputs.
 *   y        out, float [M][out]: y[m][o] = sum_g s[g][o] sum_{k in g}
 *            x[m][k] (u[k][o] - 8), each group's sum in fp32 on the matrix
 *            cores (exact products), then one fp32 fma with its scale.
 * in a multiple of 128; M up to 64 * 65535; M == 0 or out == 0 enqueues nothing.
 */
int32_t cq_w4a16_matmul(const uint16_t *x, const int32_t *qweight, const uint16_t *scales, int64_t M,
                        int64_t out, int64_t in, float *y, void *stream);

/*
 * Separately normalized environment diagonals from calibration activations
 * (CliffQuant README, "What CliffQuant changes": each channel's sensitivity
 * weighted by its activations, per calibration environment, each environment
 * normalized on its own; model
 * card, "Calibration and evaluation data": environments of 256-token windows,
 * a 16-bit model runtime).
 *   x   device uint16 [E][T][in]: bfloat16 bit patterns of the activations
 *       entering one matrix, T tokens per environment, row-major.
 *   d   out, float [in/128][E][128]: d_{e,i} = mean_t x_{t,i}^2 divided by its
 *       mean over the channels i (binary64, rounded once), the layout
 *       cq_quantize_groups takes with d_period = in/128.  An environment whose
 *       activations are all zero gives NaN (the solver flags it).
 * 1 <= E <= CQ_MAX_ENVS, T >= 1, in a multiple of 128 up to 2^24; x 16-byte
 * aligned.  workspace: cq_diagonals_workspace_size(E, T, in) bytes.
 */
size_t cq_diagonals_workspace_size(int32_t E, int64_t T, int64_t in);
int32_t cq_environment_diagonals(const uint16_t *x, int32_t E, int64_t T, int64_t in, float *d,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Held-out comparison of two scale policies on the proxy's per-group values
 * (CliffQuant README, "Held-out reconstruction proxy": the minimax policy's
 * wins, ties and losses against Pooled-WMSE by group, and a 95% interval for
 * the effect from a bootstrap resampling within modules, paired across the
 * policies).
 *   pa, pb          device double [n_groups]: per-group proxy values p_g of
 *                   policies A and B (e.g. two rows of the per_group output of
 *                   cq_proxy_worst_env_wmse_multi on held-out diagonals).
 *   module_offsets  device int64 [n_modules+1] as for the proxy; a module whose
 *                   range is empty or out of bounds makes the effect NaN.
 *   boot_idx        device int32 [n_boot][n_groups], drawn by the caller:
 *                   replicate r takes, at position j of module m's range, group
 *                   boot_idx[r][j], which must lie in m's range (else that
 *                   replicate is NaN).  The same draw serves both policies.
 *   alpha           0 < alpha < 1: the interval runs from the 100 alpha/2 to
 *                   the 100 (1 - alpha/2) percentile.
 *   counts          out, device int64 [3]: groups with p_A < p_B, ==, >.
 *   effect          out, device double [1]: the mean over modules of each
 *                   module's mean of (p_B - p_A), every sum left to right.
 *   boot            out, device double [n_boot]: the replicate effects (the same
 *                   formula on each draw), sorted ascending, NaN last.
 *   ci              out, device double [2]: the percentiles of boot by linear
 *                   interpolation at position q (n_boot - 1); NaN when n_boot is
 *                   0 or a replicate is NaN.
 * 0 <= n_boot <= CQ_MAX_BOOT; (n_boot + 1) * n_modules <= 2^31 - 1.
 * workspace: cq_heldout_workspace_size(n_boot, n_modules) bytes.
 */
size_t cq_heldout_workspace_size(int32_t n_boot, int32_t n_modules);
int32_t cq_heldout_compare(const double *pa, const double *pb, int64_t n_groups,
                           const int64_t *module_offsets, int32_t n_modules,
                           const int32_t *boot_idx, int32_t n_boot, double alpha,
                           int64_t *counts, double *effect, double *boot, double *ci,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Measurement aid, not part of the method: the fp32 fma issue rate the vector units reach, the
 * ceiling against which the full-grid search's issue rate (and its fraction of the published
 * 157.3 TFLOP/s fp32 peak: 256 CUs x 128 fma lanes x 2 flop x 2.4 GHz) is read.
 *   iters          >= 1: fmas per chain; each thread of `blocks` workgroups of 256 threads runs
 *                  8 independent chains, so the launch issues blocks x 4 waves x 8 x iters
 *                  fma wave instructions (2 flop per lane each).
 *   mode           0: the chains as x = fma(x, c, y) with c, y in vector registers (the
 *                  three-operand encoding, v_fma_f32); 1: as x = fma(y, c, x) (the accumulate
 *                  encoding, v_fmac_f32, which the full-grid search's environment sums use);
 *                  2: as x = fma(x, a, b) with a, b scalar kernel arguments (v_fma_f32 with a
 *                  scalar-register operand).  The forms issue at different rates.
 *   out            device float [blocks * 256]: the chains' sums (kept so nothing is dead code).
 *   clocks         device uint64 [2 * blocks]: per workgroup, the shader clock cycles and the
 *                  constant-rate wall clock ticks between its thread 0's start and end.
 *   wall_clock_hz  HOST double, out: the wall clock's rate (cycles / ticks x this = the clock).
 * Returns CQ_EINVAL for iters < 1, blocks < 1, another mode or a null pointer.
 */
int32_t cq_probe_valu_fma(int32_t iters, int32_t blocks, int32_t mode, float *out, uint64_t *clocks,
                          double *wall_clock_hz, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CQ_H */
