/*
 * awq.h -- C ABI of libawq, the MI355X (gfx950) library for the per-layer hot
 * path of activation-aware weight quantization (AWQ):
 *
 *   calibration activations X --(awq_act_stats)--> per-input-channel mean |x|
 *   --(awq_candidate_scales / awq_search_scales)--> grid search over alpha in
 *   s = x_mean^alpha (normalised), each candidate scored by group-wise
 *   symmetric INT4 fake quantization of W*s --(awq_quantize_pack)--> AutoAWQ
 *   GEMM layout (qweight / scales / qzeros) --(awq_unpack_dequant)--> check;
 *   for export, awq_norm_group_fold shares one scale per norm group and folds
 *   it into the norm.
 *
 * Sources (page title, section):
 *   [konic]     "From-Scratch AWQ INT4 Quantization on Qwen3-8B": "AWQ scaling",
 *               "Group-wise symmetric INT4", "AutoAWQ / HF-AWQ GEMM on-disk
 *               format", exporter steps 1-4.
 *   [cassindra] "AWQ architecture, in depth": "The pipeline end to end",
 *               "The scale search as code", "Quantization, storage and packing".
 *   [lm]        "Weight-Only Quantization: GPTQ and AWQ": "5. Technical
 *               explanation / AWQ", "6-9. Under the hood: the packed format".
 *
 * Conventions (all entry points):
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *     buffer; the library never allocates or frees device memory and keeps no
 *     pointer after a call returns.  Scratch memory is caller-supplied (`ws`),
 *     sized by the matching *_workspace query.
 *   - Matrices are row-major.  Weights are fp16 [rows, d_in]; activations are
 *     fp16 or bf16 [T, d_in] with a leading dimension `ld_x` >= d_in (elements).
 *   - `stream` is a hipStream_t (NULL = the null stream); the header declares
 *     the handle type itself, identically to HIP's own declaration, so that it
 *     needs no HIP header.  Every call validates its arguments synchronously on
 *     the host, then enqueues its kernels asynchronously on `stream`; results
 *     are ready when the stream is.
 *   - Inputs are never modified.  On any argument error nothing is launched and
 *     outputs are untouched; the call returns a nonzero status and
 *     awq_last_error() describes it.  A launch failure returns AWQ_EHIP.
 *   - No global mutable device state, except the scratch array of
 *     awq_search_scales_noalloc (see there): other calls on distinct streams may
 *     run concurrently if their buffers are distinct.  Results are
 *     deterministic (fixed-order reductions, no floating-point atomics).  The
 *     only host-side state is per host thread: the last error message and the
 *     benchmark hook awq_set_timing_events.
 */
#ifndef AWQ_H
#define AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;   /* identical to HIP's declaration */

typedef int32_t awq_status;
#define AWQ_OK 0
#define AWQ_EINVAL 1     /* null pointer, negative size, unsupported value */
#define AWQ_ESHAPE 2     /* d_in % group_size, d_out % 8, ld_x < d_in, ... */
#define AWQ_EDTYPE 3     /* unknown dtype enum */
#define AWQ_EWORKSPACE 4 /* ws too small or missing */
#define AWQ_EALIGN 5     /* pointer or leading dimension not 16-byte aligned */
#define AWQ_EHIP 6       /* HIP launch / runtime error */

#define AWQ_F16 0
#define AWQ_BF16 1
#define AWQ_F32 2

#define AWQ_SCORE_WEIGHT 0 /* [konic] AWQ scaling: ||(W - Q(W s)/s) diag(x_mean)||^2 */
#define AWQ_SCORE_OUTPUT 1 /* [cassindra] mean((X W_hat^T - X W^T)^2) over the group */

#define AWQ_ABI_VERSION 1

/* Search configuration ([cassindra] search_scale(x, linears, ..., n_grid=20)). */
typedef struct {
  int32_t group_size; /* quantization group along d_in: 32, 64 or 128           */
  int32_t n_grid;     /* number of alpha points, alpha_k = k / n_grid; 1..64      */
  int32_t score;      /* AWQ_SCORE_WEIGHT or AWQ_SCORE_OUTPUT                     */
  int32_t n_clip;     /* 0 = no clip search; else >= 2 ratios (output score only) */
  double s_min;       /* lower clamp of x_mean^alpha before normalising (1e-4)    */
  float clip_lo;      /* smallest clip ratio, in (0, 1]; ratios 1.0 .. clip_lo     */
  int32_t flags;      /* AWQ_FLAG_DUO | AWQ_FLAG_ASYM | AWQ_FLAG_OUT_*; others 0   */
} awq_search_cfg;

/* [cassindra] The scale search as code, duo_scaling=True: the candidates are
 * s = x_mean^r / (w_mean^(1-r) + 1e-4) (then the same clamp and
 * normalisation), w_mean the row-normalised mean |w| of the group's rows per
 * input channel (awq_weight_channel_mean). */
#define AWQ_FLAG_DUO 1

/* [cassindra] Why it works (worked example: step about range / 15) and
 * Quantization, storage and packing (one 16-bit scale and one 4-bit zero point
 * per group and output channel; the recipe's W4A16_ASYM): score the
 * asymmetric grid of awq_quantize_pack_asym instead of the symmetric one. */
#define AWQ_FLAG_ASYM 2

/* Output score only: how the sum of squares of X (W_hat - W)^T is formed.
 * Both give the same quantity ([cassindra] The scale search as code); by
 * default the library takes the one with less matrix-core work.
 *   direct:        each candidate contracts X with dW = W_hat - W
 *                  (2 T d_in d_out flops per candidate);
 *   second moment: per row o, sum_t (X dW^T)[t,o]^2 = dW_o H dW_o^T with
 *                  H = X^T X formed once (2 T d_in^2 flops), then
 *                  2 d_in^2 d_out flops per candidate: the lighter form when
 *                  the calibration set has more tokens than d_in.
 * Setting both is AWQ_EINVAL; with neither the library chooses each search's
 * form by its matrix-core work.  The alpha search compares sums over rows,
 * which the well-measured rows carry, and takes H (normalised) in fp16; the
 * clip search decides per row, and the error of a single row's form over H
 * grows with the conditioning of X^T X, so it takes H as two fp16 parts
 * (hi + lo, twice the products).  AWQ_FLAG_OUT_GRAM puts both searches in the
 * second-moment form. */
#define AWQ_FLAG_OUT_DIRECT 4
#define AWQ_FLAG_OUT_GRAM 8

/* One group of linears sharing an input ([cassindra] torch.cat of the group's
 * weights): part p is an fp16 device matrix [rows[p], d_in], 16-byte aligned.
 * The rows of all parts are scored as one concatenated matrix. */
typedef struct {
  int32_t n_parts;       /* 1..8                                  */
  const void* const* w;  /* [host] array of n_parts device ptrs   */
  const int64_t* rows;   /* [host] array of n_parts row counts    */
} awq_wgroup;

/* ---------------------------------------------------------------------------
 * awq_act_stats -- per-input-channel mean absolute activation.
 * [konic] AWQ scaling (x = |X|.mean(0)); [cassindra] search_scale, first line.
 *
 *   x_mean[i] = (accumulate ? x_mean[i] : 0) + inv_count * sum_t |X[t, i]|
 *
 * X: fp16/bf16 [T, ld_x] (x_dtype = AWQ_F16 | AWQ_BF16); T >= 0, d_in >= 1.
 * Sums: per channel, |x| of four consecutive rows added in fp32 (in row
 * order; all terms non-negative, so within 3 * 2^-24 of their exact sum),
 * those sums added in fp64 over token splits, each partial covering a fixed
 * set of splits in a fixed order, the partials added in a fixed order,
 * rounded once to fp32: deterministic.
 * Pass inv_count = 1/T for one chunk; to stream tokens in chunks, call with
 * accumulate = 1 and inv_count = 1/T_total for every chunk after the first.
 * ws: awq_act_stats_workspace(T, d_in) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
awq_status awq_act_stats_workspace(int64_t T, int64_t d_in, size_t* bytes /* [host] */);
awq_status awq_act_stats(const void* X, int32_t x_dtype, int64_t T, int64_t d_in, int64_t ld_x,
                         float inv_count, int32_t accumulate, float* x_mean,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_candidate_scales -- the candidate scale table of the grid search.
 * [cassindra] The scale search as code (non-duo branch); [lm] 5. AWQ: s = |X|^alpha.
 *
 *   t_k,i  = max(x_mean_i ^ (k / n_grid), s_min)     (x^0 = 1 for every x)
 *   S[k,i] = fp32( t_k,i / sqrt(max_i t_k,i * min_i t_k,i) )   evaluated in fp64
 *
 * x_mean: fp32 [d_in] (non-negative, finite); S: fp32 [n_grid, d_in].
 * Row 0 is exactly 1.0 (alpha = 0 is plain round-to-nearest).
 * ws: awq_candidate_scales_workspace(d_in, n_grid) bytes; that is 0 in this
 * version, so ws may be NULL (the argument is kept for later versions).
 * ------------------------------------------------------------------------- */
awq_status awq_candidate_scales_workspace(int64_t d_in, int32_t n_grid, size_t* bytes /* [host] */);
awq_status awq_candidate_scales(const float* x_mean, int64_t d_in, int32_t n_grid, double s_min,
                                float* S, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_weight_channel_mean -- duo scaling's weight statistic.
 * [cassindra] The scale search as code:
 *   w_mean = (w_cat.abs() / w_cat.abs().amax(dim=1)).mean(dim=0)
 *
 *   w_mean[i] = (1/d_out) sum_o |W[o, i]| / max_j |W[o, j]|
 *
 * over the concatenated rows of W (each quotient an IEEE fp32 division, an
 * all-zero row contributing 0; sums in fp64 in a fixed order, rounded once to
 * fp32).  W: as awq_search_scales, d_in a positive multiple of 8.
 * w_mean: fp32 [d_in].  ws: awq_weight_channel_mean_workspace(d_out_total,
 * d_in) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
awq_status awq_weight_channel_mean_workspace(int64_t d_out_total, int64_t d_in, size_t* bytes /* [host] */);
awq_status awq_weight_channel_mean(const awq_wgroup* W /* [host] */, int64_t d_in, float* w_mean, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_candidate_scales_duo -- the duo-scaling candidate table.
 * [cassindra] The scale search as code (duo_scaling=True):
 *
 *   t_k[i] = max(x_mean[i]^r / (w_mean[i]^(1-r) + 1e-4), s_min),  r = k / n_grid
 *   S[k, i] = RN_fp32(t_k[i] / sqrt(max_i t_k[i] * min_i t_k[i]))
 *
 * evaluated in fp64 (pow(v, 0) = 1; r = 0 gives 1 / (w_mean + 1e-4), which is
 * not plain RTN).  x_mean, w_mean: fp32 [d_in], finite, >= 0.  S: fp32
 * [n_grid, d_in].  ws: awq_candidate_scales_duo_workspace(d_in, n_grid) bytes,
 * 256-byte aligned (the fp64 table and per-block extrema).
 * ------------------------------------------------------------------------- */
awq_status awq_candidate_scales_duo_workspace(int64_t d_in, int32_t n_grid, size_t* bytes /* [host] */);
awq_status awq_candidate_scales_duo(const float* x_mean, const float* w_mean, int64_t d_in, int32_t n_grid,
                                    double s_min, float* S, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_search_scales -- grid search of alpha for one input-sharing group.
 * [konic] AWQ scaling (grid search, activation-weighted error, alpha = 0 is
 * RTN so the search never worsens it -- for the plain candidates; with
 * cfg->flags & AWQ_FLAG_DUO the table is awq_candidate_scales_duo's over
 * awq_weight_channel_mean of the group, and alpha = 0 is not RTN); [konic]
 * Group-wise symmetric INT4
 * (step = max|group| / 7, q = round(w / step).clamp(-7, 7), round half to
 * even); [cassindra] The scale search as code (keep the first strict minimum,
 * weights restored: W is read-only here) and pipeline step 5 (clip search).
 *
 * S is the awq_candidate_scales table (or, duo, awq_candidate_scales_duo's).
 * For k = 0..n_grid-1, with s = S[k] and v = W*s (fp32), per row o and group g:
 *   a = max|v|, step = RN(a / 7), q = clamp(rint(v / step), -7, 7), w_hat = q*step/s
 *   AWQ_SCORE_WEIGHT: err[k] = sum_{o,i} ((W[o,i] - w_hat[o,i]) * x_mean[i])^2
 *   AWQ_SCORE_OUTPUT: err[k] = mean_{t,o} (sum_i X[t,i] (w_hat[o,i] - W[o,i]))^2
 * best_idx = first k attaining the minimum of err; best_s = S[best_idx].
 * With cfg->flags & AWQ_FLAG_ASYM the quantizer is awq_quantize_pack_asym's:
 *   lo = min(0, min v), hi = max(0, max v), step = RN(RN(hi - lo) / 15),
 *   z = clamp(rint(RN(-lo / step)), 0, 15), w_hat = (clamp(rint(v / step) + z,
 *   0, 15) - z) * step / s; the clip ratio multiplies both lo and hi.
 * With n_clip >= 2 (output score only), afterwards per output row o and ratio
 * c_j = fp32(1 - j (1 - clip_lo) / (n_clip - 1)), j = 0..n_clip-1, the step of
 * every group of that row becomes RN(RN(c_j * a) / 7) with s = best_s, the row's
 * output error sum_t (sum_i X[t,i] (w_hat - W)[o,i])^2 is evaluated, and
 * clip[o] = c_j of the first strict minimum (ties keep the larger ratio).
 *
 * W: group of fp16 parts (rows concatenated), d_out_total = sum rows,
 *    d_out_total >= 1, d_in % group_size == 0.
 * x_mean: fp32 [d_in].  X: activations [T, ld_x] (x_dtype), required for the
 *    output score and for the clip search, else may be NULL; T >= 1 then.
 * err: fp32 [n_grid]; best_idx: int32 [1]; best_s: fp32 [d_in];
 * clip: fp32 [d_out_total], required iff n_clip >= 2, else may be NULL;
 * clip_err: fp32 [d_out_total, n_clip] per-row clip errors or NULL.
 * Arithmetic: weight score decides codes in fp32 with a reciprocal of the step
 * (codes can differ from an IEEE division only where v/step lies within a few
 * ulp of a half-integer); partial sums in fp32, final sums in fp64.  Output
 * score uses the bit-exact codes of awq_quantize_pack and contracts X with
 * (w_hat - W) on the matrix cores in fp16, each operand scaled by a power of
 * two chosen from its maximum (X) or from a bound on it (dW: the column
 * maxima of |W| and the step, never below the true maximum), so the scaling
 * is exact and overflow-free, fp32 accumulation, fp64
 * final sums; the fp16 rounding of (w_hat - W) bounds the relative error of
 * err[k] near 1e-4 on small inputs and far below it at calibration sizes.
 * In the second-moment form (AWQ_FLAG_OUT_GRAM, or chosen by the library)
 * H = X^T X is accumulated in fp32 from the same fp16 X, normalised to unit
 * diagonal (R H R, R = diag(H_ii^-1/2)) and rounded to fp16, and the columns
 * of dW carry sqrt(H_ii) instead: the extra rounding of H perturbs each
 * row's quadratic form by random-signed terms far below 1e-4 of it.
 * ws: awq_search_workspace(...) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
awq_status awq_search_workspace(const awq_search_cfg* cfg /* [host] */, int64_t d_out_total,
                                int64_t d_in, int64_t T, size_t* bytes /* [host] */);
/* Which forms awq_search_scales takes for the output score with these
 * arguments (see AWQ_FLAG_OUT_*): *form = AWQ_OUT_FORM_GRAM if the alpha
 * search is in the second-moment form (else AWQ_OUT_FORM_DIRECT), plus
 * AWQ_OUT_FORM_CLIP_GRAM if the clip search (n_clip >= 2) is.  Host only,
 * enqueues nothing; AWQ_EINVAL unless cfg->score = AWQ_SCORE_OUTPUT, shape
 * errors as awq_search_workspace. */
#define AWQ_OUT_FORM_DIRECT 0
#define AWQ_OUT_FORM_GRAM 1
#define AWQ_OUT_FORM_CLIP_GRAM 2
awq_status awq_search_output_form(const awq_search_cfg* cfg /* [host] */, int64_t d_out_total, int64_t d_in,
                                  int64_t T, int32_t* form /* [host] */);
awq_status awq_search_scales(const awq_search_cfg* cfg /* [host] */, const awq_wgroup* W /* [host] */,
                             int64_t d_in, const float* x_mean,
                             const void* X, int32_t x_dtype, int64_t T, int64_t ld_x,
                             float* err, int32_t* best_idx, float* best_s,
                             float* clip, float* clip_err,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_search_scales_noalloc -- awq_search_scales (weight score) for callers
 * that cannot allocate device memory: code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc.
 *
 * Same computation, arguments and results as awq_search_scales with
 * cfg->score = AWQ_SCORE_WEIGHT, cfg->n_clip = 0 (X, clip, clip_err absent),
 * duo and asymmetric flags allowed.  The scratch (candidate table, (x/s)^2,
 * per-block partial errors, and the duo statistic) is a 16 MiB array inside
 * the library, one per GPU, held until the process ends; the call uses the
 * copy of the current device (hipGetDevice), which must be the device of
 * `stream` and of every pointer.  The first call on a device looks up that
 * copy's address; no call allocates or frees memory.  Searches that need more
 * than 16 MiB of scratch (d_in x n_grid x 8 bytes of tables plus 4 bytes per
 * block and candidate: every Qwen3-8B-shaped group fits at n_grid = 20) are
 * rejected with AWQ_EWORKSPACE before anything is enqueued; the output score
 * and the clip search are rejected with AWQ_EINVAL (they need gigabytes).
 * Every kernel writes the scratch it reads before reading it, so nothing in it
 * needs clearing, but all calls on one GPU share it: calls that overlap on one
 * GPU (two streams, two host threads) race and must be serialized by the caller.
 * ------------------------------------------------------------------------- */
awq_status awq_search_scales_noalloc(const awq_search_cfg* cfg /* [host] */, const awq_wgroup* W /* [host] */,
                                     int64_t d_in, const float* x_mean, float* err, int32_t* best_idx,
                                     float* best_s, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_quantize_pack -- quantize W*s and pack into the AutoAWQ GEMM layout.
 * [konic] Group-wise symmetric INT4; AutoAWQ / HF-AWQ GEMM on-disk format
 * (unsigned codes, 8 per int32, pack order [0,2,4,6,1,3,5,7]); exporter step 4
 * (zero = 7, u = q + 7); [lm] 6-9 (scales [in/G, out] fp16, zeros [in/G, out/8]).
 *
 * v = RN(W*s) (s = NULL: v = W), a = max|v| over the group,
 * step = RN(RN(clip[o]*a) / 7) (clip = NULL: RN(a / 7)),
 * q = clamp(rint(RN(v / step)), -7, 7) with IEEE division and round half to
 * even (bit-exact), step = 0 gives q = 0;  u = q + 7 in [0, 14].
 *   qweight[i, m]: int32 [d_in, d_out/8]; nibble j (bits 4j..4j+3) holds u of
 *                  output row 8m + order[j], order = {0,2,4,6,1,3,5,7}
 *   scales[g, o]:  fp16 bits [d_in/G, d_out], fp16 round-to-nearest-even of step
 *   qzeros[g, m]:  int32 [d_in/G, d_out/8], every nibble 7 (may be NULL)
 * W: fp16 [d_out, d_in] 16-byte aligned; d_out % 8 == 0, d_in % group_size == 0,
 * group_size in {32, 64, 128}; s: fp32 [d_in] or NULL; clip: fp32 [d_out] or NULL.
 * W, s and clip are expected to be finite (s > 0, clip in (0, 1]); codes of
 * non-finite weights are unspecified (nothing faults).
 * ------------------------------------------------------------------------- */
awq_status awq_quantize_pack(const void* W, int64_t d_out, int64_t d_in, int32_t group_size,
                             const float* s, const float* clip,
                             int32_t* qweight, uint16_t* scales, int32_t* qzeros, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_quantize_pack_asym -- asymmetric INT4 codes in the same layout.
 * [cassindra] Why it works (range / 15 steps) and Quantization, storage and
 * packing (16-bit scale and 4-bit zero point per group and output channel,
 * about 4.16 bits per weight); [konic] AutoAWQ / HF-AWQ GEMM on-disk format
 * for the nibble order.
 *
 * v = RN(W*s), per row o and group g: lo = min(0, min v), hi = max(0, max v),
 * with clip: lo = RN(clip[o]*lo), hi = RN(clip[o]*hi);
 * step = RN(RN(hi - lo) / 15); z = clamp(rint(RN(-lo / step)), 0, 15);
 * u = clamp(rint(RN(v / step)) + z, 0, 15) (IEEE division, round half to
 * even, bit-exact); step = 0 (all-zero group) gives z = 0, u = 0.
 *   qweight[i, m]: as awq_quantize_pack, nibbles hold u
 *   scales[g, o]:  fp16 round-to-nearest-even of step
 *   qzeros[g, m]:  int32 [d_in/G, d_out/8], nibble j holds z of row 8m + order[j]
 *                  (required, 4-byte aligned)
 * awq_unpack_dequant with these qzeros gives (u - z) * fp16(step).
 * Shapes, alignment and errors as awq_quantize_pack; qzeros NULL is AWQ_EINVAL.
 * ------------------------------------------------------------------------- */
awq_status awq_quantize_pack_asym(const void* W, int64_t d_out, int64_t d_in, int32_t group_size,
                                  const float* s, const float* clip,
                                  int32_t* qweight, uint16_t* scales, int32_t* qzeros, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_norm_group_fold -- shared scale of a norm group and the folded norm.
 * [konic] exporter steps 1-3: q/k/v share input_layernorm and gate/up share
 * post_attention_layernorm; the member linears' scales become one shared
 * scale (their per-channel geometric mean) folded into the norm
 * (norm.weight /= s_shared); the members are then packed with s = s_shared
 * (awq_quantize_pack) and o_proj / down_proj with s = NULL (plain RTN).
 *
 *   s_shared[i] = RN_fp32(exp((1/M) sum_m ln s[m][i]))   fp64 logarithms, summed
 *                                                         in member order
 *   norm_out[i] = RN_dtype(norm[i] / s_shared[i])         IEEE fp32 quotient
 *
 * s: [host] array of n_members (1..8) device pointers, each fp32 [d_in] with
 * finite positive entries (the s_k rows awq_search_scales returns).
 * norm: [d_in] of norm_dtype (AWQ_F16, AWQ_BF16 or AWQ_F32), aligned to its
 * element size, or NULL (then norm_out must be NULL and only s_shared is
 * produced).  norm_out: [d_in] of the same dtype; it may equal norm (in
 * place: each element is read before it is written).
 * s_shared: fp32 [d_in], 4-byte aligned.  d_in = 0 returns AWQ_OK at once.
 * No workspace.
 * ------------------------------------------------------------------------- */
awq_status awq_norm_group_fold(const float* const* s /* [host] */, int32_t n_members, int64_t d_in,
                               const void* norm, int32_t norm_dtype, void* norm_out, float* s_shared,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_unpack_dequant -- inverse of awq_quantize_pack, for verification.
 * [konic] exporter step 4: (u - zero) * scale reproduces q * step exactly.
 *
 * out[o, i] = (u[o,i] - zero[g,o]) * float(scales[g,o])   (fp32, exact)
 *             divided by s[i] (IEEE) when s != NULL (back to W's domain).
 * qzeros NULL means zero = 7.  out: [d_out, d_in] of out_dtype (AWQ_F32 or
 * AWQ_F16, the latter rounded to nearest even).
 * ------------------------------------------------------------------------- */
awq_status awq_unpack_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                              int64_t d_out, int64_t d_in, int32_t group_size, const float* s,
                              void* out, int32_t out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_w4a16_matmul -- the W4A16 product on the packed layout (decode and prefill).
 * [cassindra] Kernels: why W4A16 is fast at decode (packed 4-bit weights
 * dequantized in registers with the group's scale and zero point, multiplied
 * with 16-bit activations; bound by reading the weights at a few tokens);
 * [lm] The kernels, 6-9 (layout).
 *
 *   Y[t, o] = sum_i X[t, i] * (u[o, i] - z[g, o]) * scales[g, o],  g = i / G
 *
 * with u, z the nibbles of qweight / qzeros as written by awq_quantize_pack or
 * awq_quantize_pack_asym (qzeros NULL means z = 7), i.e. the weights in the
 * stored (scaled) domain: X must already carry the folded 1/s.
 * X: fp16 [M, ld_x], ld_x >= d_in, 2-byte aligned.  qweight int32 [d_in, d_out/8]
 * and qzeros int32 [d_in/G, d_out/8] 4-byte aligned; scales fp16 [d_in/G, d_out]
 * 16-byte aligned.  Y: [M, ld_y] of y_dtype (AWQ_F16, rounded to nearest even
 * once, or AWQ_F32), ld_y >= d_out and a multiple of 4, 8-byte (fp16) or
 * 16-byte (fp32) aligned.  d_out % 8 == 0, d_in % group_size == 0.
 * Arithmetic, by token count M (X rows 16-byte aligned and ld_x a multiple
 * of 8 unless said otherwise):
 *   M = 1, or X rows not so aligned: the decode GEMV -- u * x exact in fp32,
 *     fp32 sums over 32 input rows, then the zero point and scale, then
 *     fixed-order fp32 sums over 256-row slices; tokens 4 at a time (the
 *     weights are read once per 4 tokens).
 *   2 <= M <= 64, d_out a multiple of 16 and qweight 8-byte aligned: the
 *     few-token matrix-core kernel -- every packed word read once for all
 *     tokens, exact fp16 (u - z) times X accumulated in fp32 per
 *     quantization group, times the fp32 scale, groups and the 4 waves of a
 *     512-row range added in order, the ranges' fp32 results added in range
 *     order.
 *   M >= 17 otherwise: the matrix-core GEMM -- exact fp16 (u - z) times X
 *     accumulated in fp32 per group, times the fp32 scale, groups added in
 *     order; when the output tiles (256 tokens x 128 outputs, or 128 x 128
 *     for at most 128 tokens) are fewer than the compute units, K is cut at
 *     multiples of 128 inputs into up to 8 ranges whose fp32 results are
 *     added in range order.
 *   All are deterministic.
 * ws: awq_w4a16_workspace(M, d_out, d_in) bytes, 256-byte aligned.  M = 0 or
 * d_out = 0 returns AWQ_OK at once.
 * ------------------------------------------------------------------------- */
awq_status awq_w4a16_workspace(int64_t M, int64_t d_out, int64_t d_in, size_t* bytes /* [host] */);
awq_status awq_w4a16_matmul(const void* X, int64_t M, int64_t ld_x, const int32_t* qweight, const uint16_t* scales,
                            const int32_t* qzeros, int64_t d_out, int64_t d_in, int32_t group_size, void* Y,
                            int64_t ld_y, int32_t y_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * awq_set_timing_events -- benchmark hook.  While set, every later call on
 * this host thread records `before` and `after` (hipEvent_t handles passed as
 * void*, created by the caller) on the call's stream immediately around its
 * main kernel launches: the partial-sum kernel of awq_act_stats; the search
 * kernel (weight score) or the chunked dW-build + GEMM launches (output score)
 * of awq_search_scales; the pack kernel of awq_quantize_pack; every launch of
 * awq_w4a16_matmul (GEMV or GEMM and, where used, the reduction).  Pass NULL,
 * NULL to clear.  The library records the events and nothing else.
 * ------------------------------------------------------------------------- */
awq_status awq_set_timing_events(void* before, void* after);

/* Message of the last failing call on this host thread ("" if none). */
const char* awq_last_error(void);
/* AWQ_ABI_VERSION of the loaded library. */
int32_t awq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_H */
