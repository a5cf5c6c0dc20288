// Output-score scale search and per-output-channel clip search on the matrix
// cores.  "AWQ architecture, in depth": section "The scale search as code" (the
// candidate is scored by the group's output error against the full-precision
// output, mean of the squared difference) and "The pipeline end to end", step 5
// (search a clipping range per output channel); "Weight-Only Quantization: GPTQ
// and AWQ", section 2 (the layer's output error is X (W - W_hat)).
//
// The difference of the two outputs is one dense contraction,
//   X W_hat^T - X W^T = X (W_hat - W)^T,
// so each candidate c costs one GEMM of X [T, d_in] with dW_c = W_hat_c - W
// [d_out, d_in], and only the sum of squares of the product is kept:
//   1. absmax + convert_x: X is copied once to fp16 scaled by a power of two
//      (exact for bf16 inputs in range, overflow-free), padded with zeros to
//      whole GEMM tiles;
//   2. colmax + dw_bound, then build_dw: dW_c with the same bit-exact codes
//      as the pack kernel, scaled by a power of two from a bound on its
//      largest element (column maxima of |W|, see the bound below) and
//      rounded to fp16 -- 3 more mantissa bits than bf16 at the same
//      matrix-core rate, which keeps the relative error of the errors near
//      1e-4 even for a few tokens and rows (one pass over W per candidate
//      slice, small next to the GEMM);
//   3. gemm_sq (direct form; section 2b holds the second-moment form):
//      fp16 MFMA 32x32x16 GEMM over all candidates of a chunk at once
//      (their dW stacked along N), fp32 accumulation; the epilogue squares the
//      tile and sums each column over the tile's tokens, so the T x d_out
//      product never reaches memory;
//   4. reduce_cols / clip_select: fixed-order fp64 sums of the column partials
//      (per candidate, or per row and clip ratio), times the exact inverse of
//      the squared operand scales.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

// ---------------------------------------------------------------------------
// 1. dW builder
// ---------------------------------------------------------------------------
constexpr int kDwThreads = 256;

__device__ __forceinline__ float clip_ratio(int j, int n_clip, float clip_lo) {
  return (float)(1.0 - (double)j * (1.0 - (double)clip_lo) / (double)(n_clip - 1));
}

// dW16[c - cand0] = fp16(dW_c * ds[c]), ds[c] a power of two from a bound on
// max |dW_c| (dw_bound_kernel below)
// ASYM: codes of the asymmetric grid (range [min(0, min v), max(0, max v)],
//   both ends times the clip ratio in mode 1, step RN(range / 15), exact zero
//   point and codes; the signed code clamp(n, -z, 15 - z) times the step)
//   dW16 rows are d_out_pad apart per candidate and K_pad elements long; rows
//   d_out .. d_out_pad-1 and columns d_in .. K_pad-1 are written as zeros.
// A block loads its tile of W once and takes the launch's candidates
// cand0 + blockIdx.y, + gridDim.y, ... in turn, so W is read once per
// candidate slice instead of once per candidate.
// COLS: every column i of dW_c is multiplied by cs[i] before the fp16
//   rounding (the second-moment form's sqrt(H_ii), see section 2b).
template <int G, bool ASYM, bool COLS>
__global__ __launch_bounds__(kDwThreads) void build_dw_kernel(
    const WParts P, int64_t d_out, int64_t d_in, int64_t d_out_pad, int64_t K_pad, int mode,
    const float* __restrict__ S, const float* __restrict__ s_best, int n_clip, float clip_lo, int cand0, int n_cand,
    const OutScales* __restrict__ sc, const float* __restrict__ cs, uint16_t* __restrict__ dw) {
  constexpr int LPG = G / 16;
  constexpr int RS = kDwThreads / LPG;
  const int64_t n_gcol = d_in / G;
  const int64_t gcol = blockIdx.x % n_gcol;
  const int64_t rblk = blockIdx.x / n_gcol;
  const int tid = threadIdx.x;
  const int lg = tid % LPG, slot = tid / LPG;
  const int64_t row = rblk * RS + slot;
  // rows past d_out run the same code on zeros (dW = 0) so that every lane
  // takes part in the cross-lane group maxima; only the loads are skipped
  const bool valid = row < d_out;
  const int64_t col = gcol * G + lg * 16;

  float w[16];
  if (valid) {
    const uint4* p = (const uint4*)(row_ptr(P, row, d_in) + col);
    unpack8_f16(p[0], w);
    unpack8_f16(p[1], w + 8);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = 0.0f;
  }
  float cv[16];
  if constexpr (COLS) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 t = ((const float4*)(cs + col))[j];
      cv[4 * j] = t.x; cv[4 * j + 1] = t.y; cv[4 * j + 2] = t.z; cv[4 * j + 3] = t.w;
    }
  }
  for (int ci = blockIdx.y; ci < n_cand; ci += gridDim.y) {
    const int c = cand0 + ci;
    const float* s = (mode == 0) ? S + (int64_t)c * d_in : s_best;
    float sv[16], v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 t = ((const float4*)(s + col))[j];
      sv[4 * j] = t.x; sv[4 * j + 1] = t.y; sv[4 * j + 2] = t.z; sv[4 * j + 3] = t.w;
    }
    float m = 0.0f, mn = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[j] = w[j] * sv[j];
      if constexpr (ASYM) {
        m = __builtin_fmaxf(m, v[j]);
        mn = __builtin_fmaxf(mn, -v[j]);
      } else {
        m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
      }
    }
    m = group_max<LPG>(m);
    float a = m, an = 0.0f;
    if constexpr (ASYM) an = group_max<LPG>(mn);
    if (mode == 1) {
      const float cr = clip_ratio(c, n_clip, clip_lo);
      a = cr * a;
      an = cr * an;
    }
    const float step = ASYM ? div15(a + an) : div7(a);
    const float inv = __builtin_amdgcn_rcpf(step);
    float qlo = -7.0f, qhi = 7.0f;
    if constexpr (ASYM) {
      const float z = step > 0.0f ? __builtin_amdgcn_fmed3f(code_exact(an, step, inv), 0.0f, (float)kUMax) : 0.0f;
      qlo = -z;
      qhi = (float)kUMax - z;
    }
    const float dsc = sc->ds[c];
    uint32_t outw[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float n = step > 0.0f ? code_exact(v[j], step, inv) : 0.0f;
      n = __builtin_fminf(__builtin_fmaxf(n, qlo), qhi);
      // w_hat - w = (q * step - w * s) / s, formed in the scaled domain with one
      // fma and the hardware reciprocal of s: within a few fp32 ulp of
      // RN(RN(q * step) / s) - w, far below the fp16 rounding of the operand
      // (the codes q themselves are exact)
      float d = __builtin_fmaf(n, step, -v[j]) * __builtin_amdgcn_rcpf(sv[j]);
      if constexpr (COLS) d *= cv[j];
      const uint32_t b = f2h_bits(d * dsc);       // exact scaling by 2^e, one rounding
      if (j & 1) outw[j >> 1] |= b << 16;
      else outw[j >> 1] = b;
    }
    {
      if (row < d_out_pad) {
        uint16_t* rowp = dw + (int64_t)ci * d_out_pad * K_pad + row * K_pad;
        uint4* dst = (uint4*)(rowp + col);
        if (!valid) {
          for (int j = 0; j < 8; ++j) outw[j] = 0u;
        }
        dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
        if (K_pad > d_in && gcol == n_gcol - 1) {  // zero K padding (at most one group wide)
          uint4* pad = (uint4*)(rowp + col + G);
          if (col + G < K_pad) {
            pad[0] = make_uint4(0u, 0u, 0u, 0u);
            pad[1] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
      }
    }
  }
}

int64_t build_dw_blocks(int group_size, int64_t d_out, int64_t d_in) {
  const int rs = kDwThreads / (group_size / 16);
  return (d_in / group_size) * ((d_out + rs - 1) / rs);
}

hipError_t launch_build_dw(int group_size, bool asym, const WParts& parts, int64_t d_out, int64_t d_in,
                           int64_t d_out_pad, int64_t K_pad, int n_cand, int mode, const float* S, const float* s_best,
                           int n_clip, float clip_lo, int cand0, const OutScales* sc, const float* cs, uint16_t* dw,
                           hipStream_t stream) {
  // d_out_pad rows (zeros past d_out).  One block per W tile takes all of the
  // launch's candidates: measured 1.2% faster on the fused-QKV output-score
  // step than one block per tile and candidate (W read once instead of
  // n_cand times), 0.9% than four slices
  dim3 grid((unsigned)build_dw_blocks(group_size, d_out_pad, d_in), 1u);
#define AWQ_DW3(G, A, C)                                                     \
  build_dw_kernel<G, A, C><<<grid, kDwThreads, 0, stream>>>(parts, d_out, d_in, d_out_pad, K_pad, mode, S, \
                                                            s_best, n_clip, clip_lo, cand0, n_cand, sc, cs, dw);
#define AWQ_DW2(G, A) \
  if (cs != nullptr) { AWQ_DW3(G, A, true) } else { AWQ_DW3(G, A, false) }
#define AWQ_DW(G) \
  if (asym) { AWQ_DW2(G, true) } else { AWQ_DW2(G, false) }
  switch (group_size) {
    case 32: AWQ_DW(32) break;
    case 64: AWQ_DW(64) break;
    default: AWQ_DW(128) break;
  }
#undef AWQ_DW
#undef AWQ_DW2
#undef AWQ_DW3
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bound on max |dW_c| (times cs) for the power-of-two operand scale ds[c].
// With v = w s and the chosen grid point q step, |q step - v| <= |v| (0 is on
// every grid, and the code is the nearest grid point, clamped toward 0's side
// of the range), and |q step - v| <= F a with a the group's max |v|:
//   symmetric:  step = rho a / 7, unclamped error <= step / 2, a clamped value
//               exceeds 7 step by at most (1 - rho) a:  F = (1 - rho) + rho / 14
//   asymmetric: step <= 2 rho a / 15, error <= step unclamped and
//               (1 - rho) a + step clamped:             F = (1 - rho) + 2 rho / 15
// (rho the clip ratio, 1 in the alpha search).  So
//   |dW_c[o, i]| cs_i <= cs_i min(F A_c / s_i, colmax_i),  A_c = max_i colmax_i s_i,
// which needs only the column maxima of |W|, not the codes of every candidate.
// Scaled by the power of two of this bound the largest element lands at most
// a few octaves below 2^14, far from fp16's subnormals.
// ---------------------------------------------------------------------------
constexpr int kColSplits = 256;  // row slices of the column-max pass (enough blocks to fill the chip)

// part[r][i] = max |W[o, i]| over the rows o of slice r, 8 columns per thread,
// four rows' loads in flight at a time
__global__ __launch_bounds__(256) void colmax_part_kernel(const WParts P, int64_t d_out, int64_t d_in,
                                                         float* __restrict__ part) {
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= d_in) return;
  const int64_t per = (d_out + kColSplits - 1) / kColSplits;
  const int64_t r0 = blockIdx.y * per, r1 = r0 + per < d_out ? r0 + per : d_out;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t row = r0;
  for (; row + 4 <= r1; row += 4) {
    uint4 u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = *(const uint4*)(row_ptr(P, row + q, d_in) + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float w[8];
      unpack8_f16(u[q], w);
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = __builtin_fmaxf(m[j], __builtin_fabsf(w[j]));
    }
  }
  for (; row < r1; ++row) {
    float w[8];
    unpack8_f16(*(const uint4*)(row_ptr(P, row, d_in) + c), w);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = __builtin_fmaxf(m[j], __builtin_fabsf(w[j]));
  }
  float* o = part + (int64_t)blockIdx.y * d_in + c;
  *(float4*)o = make_float4(m[0], m[1], m[2], m[3]);
  *(float4*)(o + 4) = make_float4(m[4], m[5], m[6], m[7]);
}

__global__ __launch_bounds__(256) void colmax_final_kernel(const float* __restrict__ part, int64_t d_in,
                                                          float* __restrict__ colmax) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= d_in) return;
  float m = 0.0f;
  for (int r = 0; r < kColSplits; ++r) m = __builtin_fmaxf(m, part[(int64_t)r * d_in + i]);
  colmax[i] = m;
}

__device__ float block_max256_v(float m, float* red) {
  const int tid = threadIdx.x;
  red[tid] = m;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = __builtin_fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// bound[blockIdx.x] for candidate c = cand0 + blockIdx.x (mode 0: s = S[c];
// mode 1: s = s_best and clip ratio c); 1% above the bound for the roundings
// of v, the step, the reciprocal of s and the bound's own arithmetic
__global__ __launch_bounds__(256) void dw_bound_kernel(const float* __restrict__ colmax, int64_t d_in, int mode,
                                                      const float* __restrict__ S, const float* __restrict__ s_best,
                                                      int n_clip, float clip_lo, int cand0, int asym,
                                                      const float* __restrict__ cs, float* __restrict__ bound) {
  __shared__ float red[256];
  const int c = cand0 + blockIdx.x;
  const float* s = mode == 0 ? S + (int64_t)c * d_in : s_best;
  float a = 0.0f;
  for (int64_t i = threadIdx.x; i < d_in; i += 256) a = __builtin_fmaxf(a, colmax[i] * s[i]);
  const float A = block_max256_v(a, red);
  const float rho = mode == 1 ? clip_ratio(c, n_clip, clip_lo) : 1.0f;
  const float F = (1.0f - rho) + rho * (asym ? 2.0f / 15.0f : 1.0f / 14.0f);
  float u = 0.0f;
  for (int64_t i = threadIdx.x; i < d_in; i += 256) {
    float t = __builtin_fminf(F * A / s[i], colmax[i]);
    if (cs != nullptr) t *= cs[i];
    u = __builtin_fmaxf(u, t);
  }
  const float U = block_max256_v(u, red);
  if (threadIdx.x == 0) bound[blockIdx.x] = 1.01f * U;
}

hipError_t launch_colmax(const WParts& parts, int64_t d_out, int64_t d_in, float* part, float* colmax,
                         hipStream_t stream) {
  colmax_part_kernel<<<dim3((unsigned)((d_in + 2047) / 2048), kColSplits), 256, 0, stream>>>(parts, d_out, d_in,
                                                                                               part);
  colmax_final_kernel<<<(unsigned)((d_in + 255) / 256), 256, 0, stream>>>(part, d_in, colmax);
  return hipGetLastError();
}

int64_t colmax_part_floats(int64_t d_in) { return (int64_t)kColSplits * d_in; }

hipError_t launch_dw_bound(bool asym, const float* colmax, int64_t d_in, int n_cand, int mode, const float* S,
                           const float* s_best, int n_clip, float clip_lo, const float* cs, float* bound,
                           hipStream_t stream) {
  dw_bound_kernel<<<(unsigned)n_cand, 256, 0, stream>>>(colmax, d_in, mode, S, s_best, n_clip, clip_lo, 0,
                                                        asym ? 1 : 0, cs, bound);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// X to scaled fp16: per-block max |X| (deterministic: max is order-free),
// scale selection, then the conversion.
// ---------------------------------------------------------------------------
constexpr int kAbsBlocks = 1024;

template <bool BF16>
__global__ __launch_bounds__(256) void absmax_rows_kernel(const uint16_t* __restrict__ X, int64_t rows,
                                                         int64_t cols, int64_t ld, float* __restrict__ out) {
  float m = 0.0f;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* p = X + r * ld;
    for (int64_t c = (int64_t)threadIdx.x * 8; c < cols; c += 256 * 8) {
      const uint4 u = ld_nt(p + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
        const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
      }
    }
  }
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    out[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

__device__ float block_max256(const float* __restrict__ a, int64_t n, float* red) {
  const int tid = threadIdx.x;
  float m = 0.0f;
  for (int64_t i = tid; i < n; i += 256) m = __builtin_fmaxf(m, a[i]);
  red[tid] = m;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = __builtin_fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// xmax: [n_x] partial maxima of |X|; dmax: [n_cand, n_d].  Block c (one per
// candidate) sets ds[c] and inv[c] (every block derives the same xs from the X partials).
__global__ __launch_bounds__(256) void out_scales_kernel(const float* __restrict__ xmax, int64_t n_x,
                                                        const float* __restrict__ dmax, int64_t n_d,
                                                        OutScales* __restrict__ sc) {
  __shared__ float red[256];
  const int c = blockIdx.x;
  const float xs = pow2_scale_for(block_max256(xmax, n_x, red));
  if (dmax == nullptr) {  // xs alone (one block)
    if (threadIdx.x == 0) sc->xs = xs;
    return;
  }
  const float ds = pow2_scale_for(block_max256(dmax + (int64_t)c * n_d, n_d, red));
  if (threadIdx.x == 0) {
    if (c == 0) sc->xs = xs;
    sc->ds[c] = ds;
    const double p = (double)xs * (double)ds;
    sc->inv[c] = 1.0 / (p * p);
  }
}

// X16 [T_pad, K_pad] = fp16(X * xs), zeros in rows >= T and columns >= d_in
template <bool BF16>
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t* __restrict__ X, int64_t rows, int64_t cols,
                                                       int64_t ld, int64_t rows_pad, int64_t cols_pad,
                                                       const OutScales* __restrict__ sc, uint16_t* __restrict__ X16) {
  const float xs = sc->xs;
  const int64_t chunks = cols_pad / 8;
  const int64_t n = rows_pad * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / chunks, c = (idx % chunks) * 8;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) {
      const uint4 u = ld_nt(X + r * ld + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
        const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
        o[j] = (uint32_t)f2h_bits(lo * xs) | ((uint32_t)f2h_bits(hi * xs) << 16);
      }
    }
    *(uint4*)(X16 + r * cols_pad + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

int64_t absmax_blocks(int64_t rows) { return rows < kAbsBlocks ? rows : kAbsBlocks; }

hipError_t launch_prepare_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, float* xmax_part,
                            hipStream_t stream) {
  const unsigned nb = (unsigned)absmax_blocks(T);
  if (bf16) absmax_rows_kernel<true><<<nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, xmax_part);
  else absmax_rows_kernel<false><<<nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, xmax_part);
  return hipGetLastError();
}

hipError_t launch_out_scales(const float* xmax_part, int64_t n_x, const float* dmax, int64_t n_d, int n_cand,
                             OutScales* sc, hipStream_t stream) {
  out_scales_kernel<<<dmax == nullptr ? 1 : n_cand, 256, 0, stream>>>(xmax_part, n_x, dmax, n_d, sc);
  return hipGetLastError();
}

hipError_t launch_convert_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, int64_t T_pad,
                            int64_t K_pad, const OutScales* sc, uint16_t* X16, hipStream_t stream) {
  const int64_t n = T_pad * (K_pad / 8);
  int64_t nb = (n + 255) / 256;
  if (nb > 8192) nb = 8192;
  if (bf16) convert_x_kernel<true><<<(unsigned)nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, T_pad, K_pad, sc, X16);
  else convert_x_kernel<false><<<(unsigned)nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, T_pad, K_pad, sc, X16);
  return hipGetLastError();
}

// Xt [rows_pad, T_pad] = fp16(X^T * xs), zeros in rows >= cols (channels) and
// columns >= rows (tokens): the token axis becomes the contraction axis of
// H = X^T X.  64 x 64 tiles through LDS: coalesced 16-byte reads along the
// channels, coalesced 16-byte writes along the tokens.
template <bool BF16>
__global__ __launch_bounds__(256) void transpose_x_kernel(const uint16_t* __restrict__ X, int64_t rows, int64_t cols,
                                                         int64_t ld, int64_t T_pad, const OutScales* __restrict__ sc,
                                                         uint16_t* __restrict__ Xt) {
  __shared__ uint16_t tile[64][64 + 2];  // [token][channel]; odd word stride spreads the column reads
  const float xs = sc->xs;
  const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int rr = tid >> 3, cc = (tid & 7) * 8;  // 32 rows x 8 chunks of 8 per pass
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t t = t0 + rr + 32 * h, c = c0 + cc;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (t < rows && c < cols) {  // cols is a multiple of 8
      const uint4 u = ld_nt(X + t * ld + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
        const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
        o[j] = (uint32_t)f2h_bits(lo * xs) | ((uint32_t)f2h_bits(hi * xs) << 16);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[rr + 32 * h][cc + 2 * j] = (uint16_t)(o[j] & 0xFFFFu);
      tile[rr + 32 * h][cc + 2 * j + 1] = (uint16_t)(o[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = rr + 32 * h, tt = cc;  // output row = channel, 8 tokens from tt
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (uint32_t)tile[tt + 2 * j][ch] | ((uint32_t)tile[tt + 2 * j + 1][ch] << 16);
    *(uint4*)(Xt + (c0 + ch) * T_pad + t0 + tt) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_transpose_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, int64_t T_pad,
                              int64_t rows_pad, const OutScales* sc, uint16_t* Xt, hipStream_t stream) {
  const dim3 grid((unsigned)(T_pad / 64), (unsigned)(rows_pad / 64));
  if (bf16) transpose_x_kernel<true><<<grid, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, T_pad, sc, Xt);
  else transpose_x_kernel<false><<<grid, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, T_pad, sc, Xt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2. GEMM of squares: Y = X16 dW^T over the concatenated candidates
//    (N_total = n_cand * d_out_pad columns, each candidate padded to a multiple
//    of the tile with zero rows; M and K padded likewise with zeros), and per
//    column the sum over the block's 384 tokens of Y^2 -> colpart[mt][n].
//
//    Block tile 384 x 256, 8 waves (4 x 2), wave tile 96 x 128 = 3 x 4 MFMA
//    32x32x16 f16 tiles: 192 fp32 accumulators per lane, 240 registers in
//    all, so two waves still share a SIMD and one issues MFMAs while the
//    other waits.  Per 16-deep K step a wave reads 7 fragments (7 KiB of LDS)
//    for 12 MFMAs, and the block writes 20 KiB of operands per 96 MFMAs; LDS
//    bandwidth co-limits the matrix cores, so the larger wave tile is what
//    pays (4% over 8 waves of 128 x 64 at K = 4096).  K advances in stages
//    of 32 through a ring of 3 LDS slots of 40 KiB, one distinct array per
//    slot and operand: the operands go from global memory straight into LDS
//    (buffer loads with the LDS bit, 16 bytes per lane, no staging registers
//    and no LDS store instructions), two stages ahead of the MFMAs.  At the
//    end of a stage each wave waits until its loads of the next stage have
//    landed (the younger stage stays in flight) and the block meets at a
//    barrier without a memory fence, which would wait for every load.  The
//    separate slot arrays let the compiler see that fragment reads never
//    alias the loads in flight.  16-byte K-chunks are XOR-swizzled by row so
//    that fragment reads are free of bank conflicts; since a direct load
//    places lane i at byte 16 i of its 1 KiB, the swizzle is applied on the
//    global side (each lane fetches the chunk its LDS slot holds).
//    The block order is remapped so that each XCD owns a contiguous range of
//    tiles, walked in groups of up to 8 M-tiles: concurrent blocks of one XCD
//    share A and B tiles in its L2.
// ---------------------------------------------------------------------------
constexpr int kBM = 384, kBN = 256, kBK = 32;
constexpr int kGemmThreads = 512;
constexpr int kXcds = 8;

// 16-byte K-chunk kc (0..3) of tile row `row` sits at slot kc ^ swz(row): the
// 16 rows read by a quarter-wave fill the 16 16-byte positions of a 256-byte
// bank window
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ uint4 frag(const uint16_t* t, int row, int kc) {
  return *(const uint4*)(t + row * kBK + ((kc ^ swz(row)) << 3));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x16 mfma_f16(const uint4 a, const uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__shared__ __attribute__((aligned(1024))) uint16_t sA0[kBM * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sA1[kBM * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sA2[kBM * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB0[kBN * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB1[kBN * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB2[kBN * kBK];

// NL loads of 16 rows x 32 K straight into LDS rows row0 .. row0 + 16 NL - 1;
// lane i lands in row row0 + 16 n + i/4, slot i%4, and fetches chunk
// (i%4) ^ swz(row) = (i%4) ^ ((i/16) & 3) (row0 is a multiple of 16)
template <int NL>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, uint16_t* dst, int row0, uint32_t vo,
                                         uint32_t soff, uint32_t row16_bytes) {
#pragma unroll
  for (int n = 0; n < NL; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + (row0 + 16 * n) * kBK), 16, vo,
                                             soff + (uint32_t)n * row16_bytes, 0, 0);
}

__device__ __forceinline__ void mfma_stage(const uint16_t* As, const uint16_t* Bs, int wm, int wn, int lane,
                                           f32x16 (&acc)[3][4]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    const int kc = 2 * ks + (lane >> 5);
    uint4 a[3], b[4];
#pragma unroll
    for (int i = 0; i < 3; ++i) a[i] = frag(As, wm * 96 + i * 32 + (lane & 31), kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag(Bs, wn * 128 + j * 32 + (lane & 31), kc);
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f16(a[i], b[j], acc[i][j]);
  }
}

// Epilogues of the block's 384 x 256 product C (rows m of A, columns n of B):
//   kEpiSq:    colpart[mt * ldc + n] = sum over the tile's rows of C[m, n]^2
//   kEpiGram:  colpart[u * ldc + n] = sum over the rows m < lim of the
//              unit's two tiles of C[m, n] * B[n, m]  (A = H'', B = dW': one
//              unit's share of the row's quadratic form dW'_n H' dW'_n^T).  H' is symmetric,
//              so with 384-wide blocks I, J the form is
//              sum_I a_I H'_II a_I + 2 sum_{J > I} a_I H'_IJ a_J: A holds
//              H'' (diagonal blocks as they are, blocks right of the diagonal
//              doubled) and the K loop of row tile mt starts at its diagonal
//              block, column 384 mt.
//   kEpiStore: out[m * ldc + n] = C[m, n] for m, n < lim (H = Xt Xt^T in
//              fp32); tiles wholly left of their rows' diagonal block
//              (n0 + 256 <= m0) are not needed and not launched.
//   kEpiGram2: kEpiGram with H'' in two fp16 parts, hi + lo (the lo matrix
//              follows the hi one, kslice * 384 rows further): the stages
//              alternate hi and lo over the same dW' chunk, so the product is
//              exact to about 2^-22 of H'' instead of 2^-11 -- the accuracy
//              of single rows' forms, which the per-row clip search needs.
//              kEpiGram reads the hi matrix only.
constexpr int kEpiSq = 0, kEpiGram = 1, kEpiStore = 2, kEpiGram2 = 3;

// kEpiStore splits K over blockIdx.y: slice y takes K columns [y kslice,
// (y + 1) kslice) and stores its partial product at out + y lim ldc.
template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_sq_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                              uint32_t a_bytes, const uint16_t* __restrict__ B,
                                                              int64_t ldb, uint32_t b_bytes, int64_t K, int64_t n_mt,
                                                              int64_t n_nt, float* __restrict__ colpart, int64_t ldc,
                                                              int group_m, int64_t lim, int64_t kslice) {
  __shared__ float red[4][kBN];
  const int64_t nblk = (int64_t)gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % kXcds, pos = bid / kXcds;
  const int64_t q = nblk / kXcds, r = nblk % kXcds;
  const int64_t id = xcd * q + (xcd < r ? xcd : r) + pos;
  const int64_t per_group = (int64_t)group_m * n_nt;
  const int64_t first_m = (id / per_group) * group_m;
  const int64_t gsz = (n_mt - first_m) < group_m ? (n_mt - first_m) : group_m;
  const int64_t mu = first_m + (id % per_group) % gsz;  // row unit: a tile, or a pair of tiles
  const int64_t nt = (id % per_group) / gsz;
  int64_t n0 = nt * kBN;
  // kEpiGram: unit mu holds row tiles mu and kslice - 1 - mu (kslice = the
  // number of row tiles, n_mt = ceil(kslice / 2) units): their K ranges from
  // the diagonal block on sum to the same length for every unit, so all
  // blocks carry the same work; the middle tile of an odd count is alone
  constexpr bool kGram = EPI == kEpiGram || EPI == kEpiGram2;
  int64_t mts[2] = {mu, mu};
  int ntile = 1;
  if constexpr (kGram) {
    mts[1] = kslice - 1 - mu;
    ntile = mts[1] != mu ? 2 : 1;
  }
  if constexpr (EPI == kEpiStore) {
    // blockIdx.x enumerates only the tiles on or right of their rows'
    // diagonal block (n0 + 256 > m0, i.e. nt >= m0 / 256), row by row: equal
    // work per block, spread over the XCDs by the dispatch order itself
    int64_t rem = bid, m = 0;
    for (; m < n_mt; ++m) {
      const int64_t cnt = n_nt - m * kBM / kBN;
      if (rem < cnt) break;
      rem -= cnt;
    }
    mts[0] = mts[1] = m;
    n0 = (m * kBM / kBN + rem) * kBN;
    colpart += (int64_t)blockIdx.y * lim * ldc;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves of 96 x 128
  // per-lane byte offset and 16-row stride of the DMA loads, for A and for B
  // (each with its own row stride)
  const uint32_t ld2 = (uint32_t)(lda * 2), ldb2 = (uint32_t)(ldb * 2);
  const uint32_t swz_off = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  const uint32_t vo = (uint32_t)(lane >> 2) * ld2 + swz_off, voB = (uint32_t)(lane >> 2) * ldb2 + swz_off;
  const uint32_t row16 = 16 * ld2, row16B = 16 * ldb2;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(B, b_bytes);
  float csum[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // this lane's column sums over the unit's tiles

  for (int ti = 0; ti < ntile; ++ti) {
    const int64_t m0 = mts[ti] * kBM;
    // K range: from the diagonal block on for the triangular quadratic form,
    // the block's slice for the split product
    int64_t kbeg = kGram ? m0 : 0, kend = K;
    if constexpr (EPI == kEpiStore) {
      kbeg = (int64_t)blockIdx.y * kslice;
      kend = kbeg + kslice < K ? kbeg + kslice : K;
    }

    f32x16 acc[3][4];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = (int)((kend - kbeg) / kBK);         // K chunks
    const int nks = (EPI == kEpiGram2 ? 2 : 1) * nk;     // stages (hi and lo per chunk)
    // wave w fetches A rows 48 w .. 48 w + 47 (3 loads) and B rows 32 w .. 32 w + 31 (2 loads)
    const uint32_t sA = (uint32_t)(((m0 + 48 * wave) * lda + kbeg) * 2),
                   sB = (uint32_t)(((n0 + 32 * wave) * ldb + kbeg) * 2);
    // kEpiGram: a unit's first (long) tile runs K downwards from K_pad, its
    // second (short) tile upwards to K_pad.  At step t every unit of an N-tile
    // then reads B at K_pad - 32 t (first tiles) or at 32 t + 384 (n - 1) - K_pad
    // (second tiles), whatever u is, so the units sharing a B panel fetch the
    // same few chunks at the same time
    const bool desc = kGram && ti == 0;
    // stage t (clamped: past the end the ring re-fetches the last stage into
    // a free slot): its K chunk, the same for A and B, and for kEpiGram2 the
    // part of A (hi on even stages, lo on odd ones, K columns further)
    auto koffB = [&](int t) {
      const int tc = t < nks ? t : nks - 1;
      const int c = EPI == kEpiGram2 ? (tc >> 1) : tc;
      return (uint32_t)((desc ? nk - 1 - c : c) * kBK * 2);
    };
    auto koffA = [&](int t) {
      const int tc = t < nks ? t : nks - 1;
      return koffB(t) + ((EPI == kEpiGram2 && (tc & 1)) ? (uint32_t)(kslice * kBM * lda * 2) : 0u);
    };

    // prologue: stages 0 and 1 in flight; wait for stage 0 (5 loads per stage
    // and wave).  On a unit's second tile every wave has passed the last
    // stage's barrier, so no fragment read of the ring is outstanding.
    dma_rows<3>(rsA, sA0, 48 * wave, vo, sA + koffA(0), row16);
    dma_rows<2>(rsB, sB0, 32 * wave, voB, sB + koffB(0), row16B);
    dma_rows<3>(rsA, sA1, 48 * wave, vo, sA + koffA(1), row16);
    dma_rows<2>(rsB, sB1, 32 * wave, voB, sB + koffB(1), row16B);
    __builtin_amdgcn_s_waitcnt(0x0075);  // vmcnt(5) lgkmcnt(0): this wave's stage-0 loads are in LDS
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // stage kt on ring slot S: fetch stage kt + 2 into slot SN (freed by the
    // previous barrier), MFMAs on slot S, then wait until stage kt + 1 is in
    // LDS (stage kt + 2 may still be in flight) and all reads of slot S are
    // done, barrier
#define AWQ_STAGE3(S, SN)                                                       \
  {                                                                             \
    dma_rows<3>(rsA, sA##SN, 48 * wave, vo, sA + koffA(kt + 2), row16);         \
    dma_rows<2>(rsB, sB##SN, 32 * wave, voB, sB + koffB(kt + 2), row16B);       \
    mfma_stage(sA##S, sB##S, wm, wn, lane, acc);                                \
    __builtin_amdgcn_s_waitcnt(0x0075);                                         \
    asm volatile("" ::: "memory");                                              \
    __builtin_amdgcn_s_barrier();                                               \
    asm volatile("" ::: "memory");                                              \
    ++kt;                                                                       \
  }
    int kt = 0;
    for (; kt + 3 <= nks;) {
      AWQ_STAGE3(0, 2)
      AWQ_STAGE3(1, 0)
      AWQ_STAGE3(2, 1)
    }
    if (kt < nks) AWQ_STAGE3(0, 2)
    if (kt < nks) AWQ_STAGE3(1, 0)
#undef AWQ_STAGE3
    __builtin_amdgcn_s_waitcnt(0x0070);  // no load in flight past this point

    // accumulator element e of MFMA tile (i, j) holds C[m, n] with
    // n = n0 + 128 wn + 32 j + lane % 32 and m = mrow(i) + 8 (e / 4) + e % 4
    const int64_t mlane = m0 + wm * 96 + 4 * (lane >> 5);
    if constexpr (EPI == kEpiStore) {
      // 32-bit element offsets (the launcher keeps lim * ldc below 2^31)
      const uint32_t ldo = (uint32_t)ldc;
      const uint32_t nl = (uint32_t)(n0 + wn * 128 + (lane & 31));
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t mb = (uint32_t)(mlane + i * 32 + 8 * g);  // a multiple of 4, lim a multiple of 64
          if (mb >= (uint32_t)lim) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (nl + 32 * j >= (uint32_t)lim) continue;
            float* p = colpart + (mb * ldo + nl + 32 * j);
            p[0] = acc[i][j][4 * g];
            p[ldo] = acc[i][j][4 * g + 1];
            p[2 * ldo] = acc[i][j][4 * g + 2];
            p[3 * ldo] = acc[i][j][4 * g + 3];
          }
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float cs = 0.0f;
        if constexpr (EPI == kEpiSq) {
#pragma unroll
          for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) cs = __builtin_fmaf(acc[i][j][e], acc[i][j][e], cs);
        } else {
          // the 12 four-element pieces of dW'[n, m] this lane needs, loads
          // issued in two batches of six before their use (rows m >= lim
          // read a valid clamped address and are masked out; m is a multiple
          // of 4, lim of 64)
          const uint16_t* brow = B + (n0 + wn * 128 + j * 32 + (lane & 31)) * ldb;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint2 u[3][2];
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                const int64_t m = mlane + i * 32 + 8 * (2 * h + g);
                u[i][g] = *(const uint2*)(brow + (m < lim ? m : lim - 4));
              }
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                const int e = 4 * (2 * h + g);
                float t = acc[i][j][e] * h2f((uint16_t)(u[i][g].x & 0xFFFFu));
                t = __builtin_fmaf(acc[i][j][e + 1], h2f((uint16_t)(u[i][g].x >> 16)), t);
                t = __builtin_fmaf(acc[i][j][e + 2], h2f((uint16_t)(u[i][g].y & 0xFFFFu)), t);
                t = __builtin_fmaf(acc[i][j][e + 3], h2f((uint16_t)(u[i][g].y >> 16)), t);
                cs += mlane + i * 32 + 8 * (2 * h + g) < lim ? t : 0.0f;
              }
          }
        }
        csum[j] += cs;
      }
    }
  }
  if constexpr (EPI != kEpiStore) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cs = csum[j] + __shfl_xor(csum[j], 32, kWave);
      if (lane < 32) red[wm][wn * 128 + j * 32 + lane] = cs;
    }
    __syncthreads();
    if (tid < kBN) colpart[mu * ldc + n0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  }
}

int64_t gemm_sq_tile_rows() { return kBM; }

// M padded to the block's 384 rows, N to 256, K to a multiple of 64
void gemm_sq_pad(int64_t T, int64_t d_out, int64_t d_in, int64_t* T_pad, int64_t* d_out_pad, int64_t* K_pad) {
  *T_pad = (T + kBM - 1) / kBM * kBM;
  *d_out_pad = (d_out + kBN - 1) / kBN * kBN;
  *K_pad = (d_in + 2 * kBK - 1) / (2 * kBK) * (2 * kBK);
}

// M-tiles per tile group: each XCD walks its tiles in groups of group_m
// M-tiles, so the 8 XCDs keep 8 * group_m A panels (384 rows x K each) in
// use.  The largest group (up to 8) whose panels stay within 320 MiB is
// taken: 8 at K = 4096 (2% faster than 4), 4 at K = 12288 (5% faster than 2,
// 18% than 1), where A re-reads across rounds of tiles mostly hit the 256 MB
// MALL.
static int gemm_group_m(int64_t K_pad) {
  const double budget = 320.0 * 1024 * 1024;
  int g = 8;
  while (g > 1 && 8.0 * g * kBM * (double)K_pad * 2.0 > budget) g /= 2;
  return g;
}

hipError_t launch_gemm_sq(const uint16_t* X16, int64_t T_pad, int64_t K_pad, const uint16_t* dw, int64_t n_cols,
                          float* colpart, int64_t ldc, hipStream_t stream) {
  const int64_t n_mt = T_pad / kBM, n_nt = n_cols / kBN;
  const uint32_t a_bytes = (uint32_t)(T_pad * K_pad * 2), b_bytes = (uint32_t)(n_cols * K_pad * 2);
  gemm_sq_kernel<kEpiSq><<<(unsigned)(n_mt * n_nt), kGemmThreads, 0, stream>>>(
      X16, K_pad, a_bytes, dw, K_pad, b_bytes, K_pad, n_mt, n_nt, colpart, ldc, gemm_group_m(K_pad), 0, 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2b. Second-moment form of the output score.  For one row o of the group,
//   sum_t (X (W_hat - W)^T)[t, o]^2 = dW_o H dW_o^T,  H = X^T X  [d_in, d_in],
// so H is formed once (2 T d_in^2 flops) and each candidate costs
// 2 d_in^2 d_out instead of 2 T d_in d_out: fewer flops whenever
// d_in (T + n d_out) < T n d_out for n scored candidates.  In fp16 on the
// matrix cores H is taken as H' = R H R, R = diag(1 / sqrt(H_ii)) (entries in
// [-1, 1], unit diagonal), and dW as dW' = ds dW diag(sqrt(H_ii)), so that
// dW' H' dW'^T = ds^2 dW H dW^T exactly up to the roundings of the operands.
// ---------------------------------------------------------------------------

// Xt rows (channels) cover both operand tiles of the H product; H' rows cover
// the 384-row tiles of the candidate product; the token axis is padded to 64
void gram_pad(int64_t T, int64_t K_pad, int64_t* T_pad, int64_t* xt_rows, int64_t* h_rows) {
  *T_pad = (T + 63) / 64 * 64;
  const int64_t m = (K_pad + kBM - 1) / kBM * kBM, n = (K_pad + kBN - 1) / kBN * kBN;
  *xt_rows = m > n ? m : n;
  *h_rows = m;
}

// Token slices of the H product: enough blocks with work (tiles on or right
// of the diagonal block) for about two per compute unit, slices of at least
// 1024 tokens, at most 8 partial copies of H.
static int64_t gram_tiles_needed(int64_t K_pad) {
  int64_t n = 0;
  for (int64_t m0 = 0; m0 < K_pad; m0 += kBM)
    for (int64_t n0 = 0; n0 < K_pad; n0 += kBN) n += (n0 + kBN > m0) ? 1 : 0;
  return n;
}

void gram_slices(int64_t T_pad, int64_t K_pad, int* n_slices, int64_t* slice) {
  // s slices take about ceil(a s / 256) / s of the unsplit product's time (a
  // blocks with work, one per compute unit at a time): the s in 1..8 that
  // minimises it, with slices of at least 512 tokens and the partial copies
  // of H within 2 GiB
  const int64_t a = gram_tiles_needed(K_pad);
  const double bytes = 4.0 * (double)K_pad * (double)K_pad;
  int64_t s = 1;
  double best = (double)((a + 255) / 256);
  for (int64_t c = 2; c <= 8; ++c) {
    if (T_pad / c < 512 || c * bytes > 2147483648.0) break;
    const double t = (double)((a * c + 255) / 256) / (double)c;
    if (t < best - 1e-9) { best = t; s = c; }
  }
  const int64_t len = ((T_pad + s - 1) / s + 63) / 64 * 64;
  *slice = len;
  *n_slices = (int)((T_pad + len - 1) / len);
}

// H32 slices [n_slices][K_pad, K_pad] = Xt Xt^T over each token slice (fp32,
// on and right of the diagonal blocks, rows and columns < K_pad)
hipError_t launch_gemm_gram_h(const uint16_t* Xt, int64_t T_pad, int64_t K_pad, float* H32, hipStream_t stream) {
  int64_t tp, xr, hr, slice;
  int ns;
  gram_pad(T_pad, K_pad, &tp, &xr, &hr);
  gram_slices(T_pad, K_pad, &ns, &slice);
  const int64_t n_mt = hr / kBM, n_nt = (K_pad + kBN - 1) / kBN;
  const uint32_t bytes = (uint32_t)(xr * T_pad * 2);
  gemm_sq_kernel<kEpiStore><<<dim3((unsigned)gram_tiles_needed(K_pad), (unsigned)ns), kGemmThreads, 0, stream>>>(
      Xt, T_pad, bytes, Xt, T_pad, bytes, T_pad, n_mt, n_nt, H32, K_pad, gemm_group_m(slice), K_pad, slice);
  return hipGetLastError();
}

// c[i] = sqrt(H_ii), r[i] = 1 / c[i] (0 for a channel that is zero in every
// token); H_ii summed over the token slices in order
__global__ __launch_bounds__(256) void gram_diag_kernel(const float* __restrict__ H32, int64_t K_pad, int ns,
                                                       float* __restrict__ c, float* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= K_pad) return;
  float h = H32[i * K_pad + i];
  for (int q = 1; q < ns; ++q) h += H32[(int64_t)q * K_pad * K_pad + i * K_pad + i];
  const float ci = h > 0.0f ? __builtin_sqrtf(h) : 0.0f;
  c[i] = ci;
  r[i] = ci > 0.0f ? 1.0f / ci : 0.0f;
}

// H16 = H'' of the triangular form in two fp16 matrices [h_rows, K_pad], hi
// then lo: with x = H_ij r_i r_j in the diagonal 384-block of row i and twice
// that right of it (exact), hi = fp16(x) and lo = fp16(x - hi) (x - hi is
// exact in fp32); zeros left of the diagonal block (never read; H32 is not
// formed there) and in rows from K_pad on
__global__ __launch_bounds__(256) void gram_half_kernel(const float* __restrict__ H32, int64_t K_pad, int ns,
                                                       int64_t h_rows, const float* __restrict__ r,
                                                       uint16_t* __restrict__ H16) {
  const int64_t chunks = K_pad / 8, n = h_rows * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / chunks, j = (idx % chunks) * 8;
    const int64_t dblk = i / kBM * kBM;  // first column of row i's diagonal block
    uint32_t o[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
    if (i < K_pad && j >= dblk) {
      const float ri = j >= dblk + kBM ? 2.0f * r[i] : r[i];
      float4 h0 = *(const float4*)(H32 + i * K_pad + j), h1 = *(const float4*)(H32 + i * K_pad + j + 4);
      for (int q = 1; q < ns; ++q) {  // token slices in order
        const float* hq = H32 + (int64_t)q * K_pad * K_pad + i * K_pad + j;
        const float4 a = *(const float4*)hq, b = *(const float4*)(hq + 4);
        h0.x += a.x; h0.y += a.y; h0.z += a.z; h0.w += a.w;
        h1.x += b.x; h1.y += b.y; h1.z += b.z; h1.w += b.w;
      }
      const float4 r0 = *(const float4*)(r + j), r1 = *(const float4*)(r + j + 4);
      const float v[8] = {h0.x * ri * r0.x, h0.y * ri * r0.y, h0.z * ri * r0.z, h0.w * ri * r0.w,
                          h1.x * ri * r1.x, h1.y * ri * r1.y, h1.z * ri * r1.z, h1.w * ri * r1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint16_t a = f2h_bits(v[2 * q]), b = f2h_bits(v[2 * q + 1]);
        o[q] = (uint32_t)a | ((uint32_t)b << 16);
        lo[q] = (uint32_t)f2h_bits(v[2 * q] - h2f(a)) | ((uint32_t)f2h_bits(v[2 * q + 1] - h2f(b)) << 16);
      }
    }
    *(uint4*)(H16 + i * K_pad + j) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(H16 + (h_rows + i) * K_pad + j) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

hipError_t launch_gram_scale(const float* H32, int64_t T_pad, int64_t K_pad, int64_t h_rows, float* c, float* r,
                             uint16_t* H16, hipStream_t stream) {
  int ns;
  int64_t slice;
  gram_slices(T_pad, K_pad, &ns, &slice);
  gram_diag_kernel<<<(unsigned)((K_pad + 255) / 256), 256, 0, stream>>>(H32, K_pad, ns, c, r);
  const int64_t n = h_rows * (K_pad / 8);
  int64_t nb = (n + 255) / 256;
  if (nb > 8192) nb = 8192;
  gram_half_kernel<<<(unsigned)nb, 256, 0, stream>>>(H32, K_pad, ns, h_rows, r, H16);
  return hipGetLastError();
}

// colpart[u * ldc + n] = row unit u's share (tiles u and n_tiles - 1 - u) of
// dW'_n H' dW'_n^T over the n_cols stacked dW' rows, u < gram_units(h_rows)
// (K from each tile's diagonal block on: about half the products of the full
// form); split: H'' as hi + lo (twice the products, per-row accuracy)
int64_t gram_units(int64_t h_rows) { return (h_rows / kBM + 1) / 2; }

hipError_t launch_gemm_gram(const uint16_t* H16, int64_t h_rows, int64_t K_pad, const uint16_t* dw, int64_t n_cols,
                            float* colpart, int64_t ldc, bool split, hipStream_t stream) {
  const int64_t n_tiles = h_rows / kBM, n_units = gram_units(h_rows), n_nt = n_cols / kBN;
  const uint32_t a_bytes = (uint32_t)(h_rows * 2 * K_pad * 2), b_bytes = (uint32_t)(n_cols * K_pad * 2);
  const dim3 grid((unsigned)(n_units * n_nt));
  if (split)
    gemm_sq_kernel<kEpiGram2><<<grid, kGemmThreads, 0, stream>>>(H16, K_pad, a_bytes, dw, K_pad, b_bytes, K_pad,
                                                                 n_units, n_nt, colpart, ldc, gemm_group_m(K_pad),
                                                                 K_pad, n_tiles);
  else
    gemm_sq_kernel<kEpiGram><<<grid, kGemmThreads, 0, stream>>>(H16, K_pad, a_bytes / 2, dw, K_pad, b_bytes, K_pad,
                                                                n_units, n_nt, colpart, ldc, gemm_group_m(K_pad),
                                                                K_pad, n_tiles);
  return hipGetLastError();
}

// per-candidate totals: tot[c] = scale * inv[c] * sum_mt sum_{o < d_out} colpart[mt][c * d_out_pad + o]
// stage 1: block (chunk, c) sums 256 columns over all token tiles -> chunk_sum[c][chunk]
// stage 2: one thread per candidate adds its chunk sums in order
constexpr int kColChunk = 256;

__global__ __launch_bounds__(kColChunk) void reduce_cols_kernel(const float* __restrict__ colpart, int64_t n_mt,
                                                               int64_t ldc, int64_t d_out, int64_t d_out_pad,
                                                               double* __restrict__ chunk_sum) {
  const int c = blockIdx.y;
  const int64_t o = (int64_t)blockIdx.x * kColChunk + threadIdx.x;
  double acc = 0.0;
  if (o < d_out) {
    const float* p = colpart + (int64_t)c * d_out_pad + o;
    int64_t mt = 0;
    for (; mt + 8 <= n_mt; mt += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = p[(mt + q) * ldc];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += (double)v[q];
    }
    for (; mt < n_mt; ++mt) acc += (double)p[mt * ldc];
  }
  __shared__ double red[kColChunk];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kColChunk / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_sum[(int64_t)c * gridDim.x + blockIdx.x] = red[0];
}

int64_t reduce_cols_chunks(int64_t d_out) { return (d_out + kColChunk - 1) / kColChunk; }

hipError_t launch_reduce_cols(const float* colpart, int64_t n_mt, int64_t ldc, int64_t d_out, int64_t d_out_pad,
                              int n_cand, double* chunk_sum, hipStream_t stream) {
  const int64_t nch = reduce_cols_chunks(d_out);
  reduce_cols_kernel<<<dim3((unsigned)nch, (unsigned)n_cand), kColChunk, 0, stream>>>(colpart, n_mt, ldc, d_out,
                                                                                      d_out_pad, chunk_sum);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 3. per-row clip selection: E[o, j] = sum over token tiles (fixed order, fp64);
//    ratio of the first strict minimum over j = 0 (1.0) .. n_clip-1 (clip_lo).
// ---------------------------------------------------------------------------
__global__ void clip_select_kernel(const float* __restrict__ colpart, int64_t n_mt, int64_t ldc, int64_t d_out,
                                   int64_t d_out_pad, int n_clip, float clip_lo, const OutScales* __restrict__ sc,
                                   float* __restrict__ clip, float* __restrict__ clip_err) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= d_out) return;
  int best = 0;
  double be = 0.0;
  for (int j = 0; j < n_clip; ++j) {
    double e = 0.0;
    for (int64_t mt = 0; mt < n_mt; ++mt) e += (double)colpart[mt * ldc + (int64_t)j * d_out_pad + o];
    e *= sc->inv[j];
    if (clip_err != nullptr) clip_err[o * n_clip + j] = (float)e;
    if (j == 0 || e < be) { be = e; best = j; }
  }
  clip[o] = clip_ratio(best, n_clip, clip_lo);
}

hipError_t launch_clip_select(const float* colpart, int64_t n_mt, int64_t ldc, int64_t d_out, int64_t d_out_pad,
                              int n_clip, float clip_lo, const OutScales* sc, float* clip, float* clip_err,
                              hipStream_t stream) {
  clip_select_kernel<<<(unsigned)((d_out + 255) / 256), 256, 0, stream>>>(colpart, n_mt, ldc, d_out, d_out_pad,
                                                                          n_clip, clip_lo, sc, clip, clip_err);
  return hipGetLastError();
}

}  // namespace awq
