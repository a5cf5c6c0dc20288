// Host-side launch wrappers of the libawq kernels (internal; the public ABI is
// include/awq.h).  Each wrapper enqueues on `stream` and returns
// hipGetLastError() after its launches; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "awq_device.h"

namespace awq {

// activation statistics
void act_stats_plan(int64_t T, int64_t d_in, int64_t* n_split, int64_t* rows_per_split);
hipError_t launch_act_stats(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld,
                            float inv_count, int accumulate, float* x_mean, void* ws,
                            hipStream_t stream);

// candidate scale table S [n_grid, d_in] and, if C2 != nullptr, (x/s)^2 [n_grid, d_in]
hipError_t launch_candidates(const float* x_mean, int64_t d_in, int n_grid, double s_min, float* S,
                             float* C2, hipStream_t stream);

// weight-score search: per-block partial errors, candidate-major [n_grid, n_blocks]
int64_t search_weight_blocks(int group_size, int64_t d_out, int64_t d_in);
// asym: the asymmetric grid (zero point per group row)
hipError_t launch_search_weight(int group_size, bool asym, const WParts& parts, int64_t d_out, int64_t d_in,
                                int n_grid, const float* S, const float* C2, float* partials,
                                hipStream_t stream);

// reduce partials p[c * n_blocks + b] over b (fixed order, fp64), times `scale`
// and cand_scale[c] when given -> tot [n_cand] (fp64) and err [n_cand] (fp32);
// smallest index attaining the minimum -> best_idx; if S is given,
// best_s = S[best] [d_in].  One launch (ceil(d_in / 1024) blocks).
hipError_t launch_select(const float* partials, int64_t n_blocks, int n_cand, double scale,
                         const double* cand_scale, double* tot, float* err, int32_t* best_idx, const float* S,
                         int64_t d_in, float* best_s, hipStream_t stream);
hipError_t launch_select(const double* partials, int64_t n_blocks, int n_cand, double scale,
                         const double* cand_scale, double* tot, float* err, int32_t* best_idx, const float* S,
                         int64_t d_in, float* best_s, hipStream_t stream);

// output-score search
// X -> per-block max |X| [absmax_blocks(T)]
int64_t absmax_blocks(int64_t rows);
hipError_t launch_prepare_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, float* xmax_part,
                            hipStream_t stream);
// scales: xs from the X partial maxima, ds[c] and inv[c] from the dW bounds dmax [n_cand, n_d]
hipError_t launch_out_scales(const float* xmax_part, int64_t n_x, const float* dmax, int64_t n_d, int n_cand,
                             OutScales* sc, hipStream_t stream);
// padded GEMM shapes: T_pad a multiple of the token tile, d_out_pad of 256, K_pad of 64
int64_t gemm_sq_tile_rows();
void gemm_sq_pad(int64_t T, int64_t d_out, int64_t d_in, int64_t* T_pad, int64_t* d_out_pad, int64_t* K_pad);
// X16 [T_pad, K_pad] = fp16(X * xs), zero padded
hipError_t launch_convert_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, int64_t T_pad,
                            int64_t K_pad, const OutScales* sc, uint16_t* X16, hipStream_t stream);
// dW of candidates c = cand0 .. cand0+n_cand-1 (mode 0: s = S[c]; mode 1: s = s_best, clip ratio c):
//   dw[c - cand0] = fp16(dW_c * sc->ds[c]), [d_out_pad, K_pad] each, zero padded;
//   cs != nullptr: column i of every dW_c is multiplied by cs[i] first (second-moment form)
int64_t build_dw_blocks(int group_size, int64_t d_out, int64_t d_in);
hipError_t launch_build_dw(int group_size, bool asym, const WParts& parts, int64_t d_out, int64_t d_in,
                           int64_t d_out_pad, int64_t K_pad, int n_cand, int mode, const float* S, const float* s_best,
                           int n_clip, float clip_lo, int cand0, const OutScales* sc, const float* cs, uint16_t* dw,
                           hipStream_t stream);
// colmax[i] = max_o |W[o, i]| (part: colmax_part_floats(d_in) floats of scratch)
int64_t colmax_part_floats(int64_t d_in);
hipError_t launch_colmax(const WParts& parts, int64_t d_out, int64_t d_in, float* part, float* colmax,
                         hipStream_t stream);
// bound[c] >= max |dW_c| (times cs) for c = 0 .. n_cand-1, from the column maxima (same modes as build_dw)
hipError_t launch_dw_bound(bool asym, const float* colmax, int64_t d_in, int n_cand, int mode, const float* S,
                           const float* s_best, int n_clip, float clip_lo, const float* cs, float* bound,
                           hipStream_t stream);
// gemm of squares on fp16 operands: Y = X16 [T_pad, K_pad] dw^T (dw: [n_cols, K_pad]);
// colpart[mt * ldc + n] = sum over the 384 tokens of tile mt of Y[t, n]^2
hipError_t launch_gemm_sq(const uint16_t* X16, int64_t T_pad, int64_t K_pad, const uint16_t* dw, int64_t n_cols,
                          float* colpart, int64_t ldc, hipStream_t stream);
// second-moment form: Xt [xt_rows, T_pad] = fp16(X^T xs); H32 = Xt Xt^T [K_pad, K_pad];
// c = sqrt(diag H), r = 1 / c; H16 = r_i H_ij r_j as fp16 hi then lo matrices [h_rows, K_pad];
// colpart[mt * ldc + n] = tile mt's share of dw_n H16 dw_n^T (dw built with cs = c)
void gram_pad(int64_t T, int64_t K_pad, int64_t* T_pad, int64_t* xt_rows, int64_t* h_rows);
hipError_t launch_transpose_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, int64_t T_pad,
                              int64_t rows_pad, const OutScales* sc, uint16_t* Xt, hipStream_t stream);
// H is formed in n_slices partial copies over token slices (summed in order by gram_scale)
void gram_slices(int64_t T_pad, int64_t K_pad, int* n_slices, int64_t* slice);
hipError_t launch_gemm_gram_h(const uint16_t* Xt, int64_t T_pad, int64_t K_pad, float* H32, hipStream_t stream);
hipError_t launch_gram_scale(const float* H32, int64_t T_pad, int64_t K_pad, int64_t h_rows, float* c, float* r,
                             uint16_t* H16, hipStream_t stream);
// rows of colpart written by launch_gemm_gram (pairs of 384-row tiles of H16)
int64_t gram_units(int64_t h_rows);
hipError_t launch_gemm_gram(const uint16_t* H16, int64_t h_rows, int64_t K_pad, const uint16_t* dw, int64_t n_cols,
                            float* colpart, int64_t ldc, bool split, hipStream_t stream);
// scales: with dmax == nullptr only sc->xs is set
// chunk_sum[c, ch] = sum_mt sum_{o in chunk ch, o < d_out} colpart[mt * ldc + c * d_out_pad + o]
// (fp64, fixed order), [n_cand, reduce_cols_chunks(d_out)]
int64_t reduce_cols_chunks(int64_t d_out);
hipError_t launch_reduce_cols(const float* colpart, int64_t n_mt, int64_t ldc, int64_t d_out, int64_t d_out_pad,
                              int n_cand, double* chunk_sum, hipStream_t stream);
// per-row argmin over clip ratios: E[o, j] = sc->inv[j] * sum_mt colpart[mt * ldc + j * d_out_pad + o]
hipError_t launch_clip_select(const float* colpart, int64_t n_mt, int64_t ldc, int64_t d_out, int64_t d_out_pad,
                              int n_clip, float clip_lo, const OutScales* sc, float* clip, float* clip_err,
                              hipStream_t stream);

// quantize + pack, unpack + dequant
// asym: unsigned codes with per-(group, row) zero points written to qzeros (required)
hipError_t launch_quantize_pack(const uint16_t* W, int64_t d_out, int64_t d_in, int group_size, bool asym,
                                const float* s, const float* clip, int32_t* qweight,
                                uint16_t* scales, int32_t* qzeros, hipStream_t stream);
hipError_t launch_unpack_dequant(const int32_t* qweight, const uint16_t* scales,
                                 const int32_t* qzeros, int64_t d_out, int64_t d_in, int group_size,
                                 const float* s, void* out, bool out_f16, hipStream_t stream);

// W4A16 product on the packed layout: Y [M, d_out] (fp16 or fp32, row stride
// ld_y) = X [M, d_in] (fp16, row stride ld_x) W_hat^T; part: fp32 scratch of
// w4a16_slices(d_in) * min(4, M rounded up to 1, 2, 4) * d_out floats
int64_t w4a16_slices(int64_t d_in);
// floats of the prefill GEMM's K-split partials (0 when it runs unsplit or M is below the GEMM's range)
int64_t w4a16_gemm_part_floats(int64_t M, int64_t d_out, int64_t d_in);
// the few-token (2..16) matrix-core path: fp32 partials of its input ranges, and whether it runs
int64_t w4a16_skinny_part_floats(int64_t M, int64_t d_out, int64_t d_in);
bool w4a16_uses_skinny(const void* X, int64_t M, int64_t ld_x, const void* qweight, int64_t d_out);
int64_t w4a16_cols(int64_t d_out);
hipError_t launch_w4a16(const uint16_t* X, int64_t M, int64_t ld_x, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, int64_t d_out, int64_t d_in, int group_size, void* Y, int64_t ld_y,
                        bool y_f16, float* part, hipStream_t stream);

// s_shared = fp32 geometric mean of the n member scales (fp64 logs), and
// norm_out = norm / s_shared in the norm's dtype (0 fp16, 1 bf16, 2 fp32);
// norm may be null (then only s_shared).
hipError_t launch_norm_group_fold(const ScaleSet& S, int64_t d_in, const void* norm, int norm_dtype, void* norm_out,
                                  float* s_shared, hipStream_t stream);

// out[i] = inv_count * (sum over the n_split rows of part[split][i], in
// split order, fp64) rounded to fp32 (the statistics' final combine)
hipError_t launch_split_mean(const double* part, int64_t n_split, int64_t d_in, double inv_count, float* out,
                             hipStream_t stream);

// Duo scaling ([cassindra] The scale search as code, duo_scaling=True).
// w_mean of the group's rows: rmax [d_out] and part [wmean_splits(d_out)][d_in]
// are scratch.
int64_t wmean_splits(int64_t d_out);
hipError_t launch_weight_channel_mean(const WParts& parts, int64_t d_out, int64_t d_in, float* rmax, double* part,
                                      float* w_mean, hipStream_t stream);
// duo candidate table: T [n_grid][d_in] fp64 and ext [n_grid][duo_cand_blocks][2]
// fp64 are scratch; S [n_grid][d_in], C2 (optional) as launch_candidates
int64_t duo_cand_blocks(int64_t d_in);
hipError_t launch_candidates_duo(const float* x_mean, const float* w_mean, int64_t d_in, int n_grid, double s_min,
                                 double* T, double* ext, float* S, float* C2, hipStream_t stream);

}  // namespace awq
