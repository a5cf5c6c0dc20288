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
//      (exact for bf16 inputs in range, overflow-free);
//   2. build_dw (max pass, then write pass): dW_c with the same bit-exact codes
//      as the pack kernel, scaled by a power of two from its exact maximum and
//      rounded to fp16 -- 3 more mantissa bits than bf16 at the same matrix-core
//      rate, which keeps the relative error of the errors near 1e-4 even for
//      a few tokens and rows (one pass over W per candidate, negligible next to
//      the GEMM);
//   3. gemm_sq: fp16 MFMA 32x32x16 GEMM, fp32 accumulation; the epilogue squares
//      the tile and reduces it (whole tile, or per output column for the clip
//      search), so the T x d_out product never reaches memory;
//   4. select / clip_select: fixed-order fp64 sums of the tile partials, times
//      the exact inverse of the squared operand scales.
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

// WRITE = false: per-block max |dW_c| -> dmax[(c - cand0) * gridDim.x + block]
// WRITE = true:  dW16[c - cand0] = fp16(dW_c * ds[c])
template <int G, bool WRITE>
__global__ __launch_bounds__(kDwThreads) void build_dw_kernel(
    const WParts P, int64_t d_out, int64_t d_in, int mode, const float* __restrict__ S,
    const float* __restrict__ s_best, int n_clip, float clip_lo, int cand0,
    const OutScales* __restrict__ sc, float* __restrict__ dmax, uint16_t* __restrict__ dw) {
  constexpr int LPG = G / 16;
  constexpr int RS = kDwThreads / LPG;
  const int c = cand0 + blockIdx.y;
  const float* s = (mode == 0) ? S + (int64_t)c * d_in : s_best;
  const int64_t n_gcol = d_in / G;
  const int64_t gcol = blockIdx.x % n_gcol;
  const int64_t rblk = blockIdx.x / n_gcol;
  const int tid = threadIdx.x;
  const int lg = tid % LPG, slot = tid / LPG;
  const int64_t row = rblk * RS + slot;
  // rows past d_out run the same code on zeros (dW = 0) so that every thread
  // reaches the block reduction below; only the loads and stores are skipped
  const bool valid = row < d_out;
  __shared__ float red[kDwThreads / 64];
  const int64_t col = gcol * G + lg * 16;

  float w[16], sv[16], v[16];
  if (valid) {
    const uint4* p = (const uint4*)(row_ptr(P, row, d_in) + col);
    unpack8_f16(p[0], w);
    unpack8_f16(p[1], w + 8);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 t = ((const float4*)(s + col))[j];
    sv[4 * j] = t.x; sv[4 * j + 1] = t.y; sv[4 * j + 2] = t.z; sv[4 * j + 3] = t.w;
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    v[j] = w[j] * sv[j];
    m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
  }
  m = group_max<LPG>(m);
  const float a = (mode == 1) ? clip_ratio(c, n_clip, clip_lo) * m : m;
  const float step = div7(a);
  const float inv = __builtin_amdgcn_rcpf(step);
  const float dsc = WRITE ? sc->ds[c] : 1.0f;
  uint32_t outw[8];
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float n = step > 0.0f ? code_exact(v[j], step, inv) : 0.0f;
    n = __builtin_fminf(__builtin_fmaxf(n, -7.0f), 7.0f);
    const float wh = (n * step) / sv[j];          // RN(RN(q * step) / s)
    const float d = wh - w[j];
    if constexpr (WRITE) {
      const uint32_t b = f2h_bits(d * dsc);       // exact scaling by 2^e, one rounding
      if (j & 1) outw[j >> 1] |= b << 16;
      else outw[j >> 1] = b;
    } else {
      mx = __builtin_fmaxf(mx, __builtin_fabsf(d));
    }
  }
  if constexpr (WRITE) {
    if (!valid) return;
    uint4* dst = (uint4*)(dw + (int64_t)blockIdx.y * d_out * d_in + row * d_in + col);
    dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  } else {
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
      float b = red[0];
      for (int w = 1; w < kDwThreads / 64; ++w) b = __builtin_fmaxf(b, red[w]);
      dmax[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = b;
    }
  }
}

int64_t build_dw_blocks(int group_size, int64_t d_out, int64_t d_in) {
  const int rs = kDwThreads / (group_size / 16);
  return (d_in / group_size) * ((d_out + rs - 1) / rs);
}

hipError_t launch_build_dw(int group_size, const WParts& parts, int64_t d_out, int64_t d_in,
                           int n_cand, int mode, const float* S, const float* s_best, int n_clip,
                           float clip_lo, int cand0, const OutScales* sc, float* dmax, uint16_t* dw,
                           hipStream_t stream) {
  dim3 grid((unsigned)build_dw_blocks(group_size, d_out, d_in), (unsigned)n_cand);
#define AWQ_DW(G)                                                                             \
  if (dw == nullptr) build_dw_kernel<G, false><<<grid, kDwThreads, 0, stream>>>(                \
      parts, d_out, d_in, mode, S, s_best, n_clip, clip_lo, cand0, sc, dmax, dw);               \
  else build_dw_kernel<G, true><<<grid, kDwThreads, 0, stream>>>(                               \
      parts, d_out, d_in, mode, S, s_best, n_clip, clip_lo, cand0, sc, dmax, dw);
  switch (group_size) {
    case 32: AWQ_DW(32) break;
    case 64: AWQ_DW(64) break;
    default: AWQ_DW(128) break;
  }
#undef AWQ_DW
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

// xmax: [n_x] partial maxima of |X| (nullptr: keep sc->xs); dmax: [n_cand, n_d].
__global__ __launch_bounds__(256) void out_scales_kernel(const float* __restrict__ xmax, int64_t n_x,
                                                        const float* __restrict__ dmax, int64_t n_d, int n_cand,
                                                        OutScales* __restrict__ sc) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  if (xmax != nullptr) {
    float m = 0.0f;
    for (int64_t i = tid; i < n_x; i += 256) m = __builtin_fmaxf(m, xmax[i]);
    red[tid] = m;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) red[tid] = __builtin_fmaxf(red[tid], red[tid + w]);
      __syncthreads();
    }
    if (tid == 0) sc->xs = pow2_scale_for(red[0]);
    __syncthreads();
  }
  for (int c = 0; c < n_cand; ++c) {
    float m = 0.0f;
    for (int64_t i = tid; i < n_d; i += 256) m = __builtin_fmaxf(m, dmax[(int64_t)c * n_d + i]);
    red[tid] = m;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) red[tid] = __builtin_fmaxf(red[tid], red[tid + w]);
      __syncthreads();
    }
    if (tid == 0) {
      const float ds = pow2_scale_for(red[0]);
      sc->ds[c] = ds;
      const double p = (double)sc->xs * (double)ds;
      sc->inv[c] = 1.0 / (p * p);
    }
    __syncthreads();
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t* __restrict__ X, int64_t rows, int64_t cols,
                                                       int64_t ld, const OutScales* __restrict__ sc,
                                                       uint16_t* __restrict__ X16) {
  const float xs = sc->xs;
  const int64_t chunks = cols / 8;
  const int64_t n = rows * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / chunks, c = (idx % chunks) * 8;
    const uint4 u = ld_nt(X + r * ld + c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
      const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
      o[j] = (uint32_t)f2h_bits(lo * xs) | ((uint32_t)f2h_bits(hi * xs) << 16);
    }
    *(uint4*)(X16 + r * cols + c) = make_uint4(o[0], o[1], o[2], o[3]);
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
  out_scales_kernel<<<1, 256, 0, stream>>>(xmax_part, n_x, dmax, n_d, n_cand, sc);
  return hipGetLastError();
}

hipError_t launch_convert_x(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld_x, const OutScales* sc,
                            uint16_t* X16, hipStream_t stream) {
  const int64_t n = T * (d_in / 8);
  int64_t nb = (n + 255) / 256;
  if (nb > 8192) nb = 8192;
  if (bf16) convert_x_kernel<true><<<(unsigned)nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, sc, X16);
  else convert_x_kernel<false><<<(unsigned)nb, 256, 0, stream>>>((const uint16_t*)X, T, d_in, ld_x, sc, X16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2. GEMM of squares: Y = X dW^T, keep sum(Y^2) per tile or per column.
//    Block tile 128 (tokens) x 128 (output rows) x 64 (inputs), 4 waves in a
//    2 x 2 arrangement, each wave 64 x 64 = 2 x 2 MFMA 32x32x16 tiles.
//    Operands are K-contiguous in memory and in LDS (row stride padded to
//    72 elements against bank conflicts); each lane feeds the MFMA 8
//    consecutive K values of one row (A: token row, B: output row).
// ---------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 64, kLdsW = kBK + 8;
constexpr int kGemmThreads = 256;

void gemm_sq_shape(int64_t T, int64_t d_out, int per_col, int64_t* n_mtiles, int64_t* n_ntiles) {
  (void)per_col;
  *n_mtiles = (T + kBM - 1) / kBM;
  *n_ntiles = (d_out + kBN - 1) / kBN;
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(const uint4 a, const uint4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF16, int PER_COL>
__global__ __launch_bounds__(kGemmThreads) void gemm_sq_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t ldx, const uint16_t* __restrict__ DW,
    int64_t N, int64_t K, int64_t n_mt, int64_t n_nt, float* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsW];
  __shared__ float red[2][kBN];

  const int cand = blockIdx.y;
  const uint16_t* B = DW + (int64_t)cand * N * K;
  const int64_t nt = blockIdx.x % n_nt;
  const int64_t mt = blockIdx.x / n_nt;
  const int64_t m0 = mt * kBM, n0 = nt * kBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  uint4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kGemmThreads * i;
      const int r = c >> 3, kc = c & 7;
      const int64_t kk = k0 + kc * 8;
      const int64_t gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < T && kk < K) ? *(const uint4*)(X + gm * ldx + kk) : zero4;
      rb[i] = (gn < N && kk < K) ? *(const uint4*)(B + gn * K + kk) : zero4;
    }
  };
  gload(0);
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kGemmThreads * i;
      const int r = c >> 3, kc = c & 7;
      *(uint4*)(As + r * kLdsW + kc * 8) = ra[i];
      *(uint4*)(Bs + r * kLdsW + kc * 8) = rb[i];
    }
    __syncthreads();
    if (k0 + kBK < K) gload(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const uint4*)(As + (wm * 64 + i * 32 + (lane & 31)) * kLdsW + kk + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const uint4*)(Bs + (wn * 64 + j * 32 + (lane & 31)) * kLdsW + kk + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<BF16>(a[i], b[j], acc[i][j]);
    }
  }

  if constexpr (PER_COL == 0) {
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sq = __builtin_fmaf(acc[i][j][e], acc[i][j][e], sq);
    sq = wave_sum(sq);
    if (lane == 0) red[0][wave] = sq;
    __syncthreads();
    if (tid == 0)
      partials[(int64_t)cand * (n_mt * n_nt) + blockIdx.x] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  } else {
    // D column of a 32x32 MFMA tile = lane % 32; lanes l and l + 32 hold other rows
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float cs = 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) cs = __builtin_fmaf(acc[i][j][e], acc[i][j][e], cs);
      cs += __shfl_xor(cs, 32, kWave);
      if (lane < 32) red[wm][wn * 64 + j * 32 + lane] = cs;
    }
    __syncthreads();
    if (tid < kBN && n0 + tid < N)
      partials[((int64_t)cand * n_mt + mt) * N + n0 + tid] = red[0][tid] + red[1][tid];
  }
}

hipError_t launch_gemm_sq(const uint16_t* X16, int64_t T, int64_t ld_x, const uint16_t* dw, int64_t d_out,
                          int64_t d_in, int n_cand, int per_col, float* partials, hipStream_t stream) {
  int64_t n_mt, n_nt;
  gemm_sq_shape(T, d_out, per_col, &n_mt, &n_nt);
  dim3 grid((unsigned)(n_mt * n_nt), (unsigned)n_cand);
  if (per_col) gemm_sq_kernel<false, 1><<<grid, kGemmThreads, 0, stream>>>(X16, T, ld_x, dw, d_out, d_in, n_mt, n_nt, partials);
  else gemm_sq_kernel<false, 0><<<grid, kGemmThreads, 0, stream>>>(X16, T, ld_x, dw, d_out, d_in, n_mt, n_nt, partials);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 3. per-row clip selection: E[o, j] = sum over token tiles (fixed order, fp64);
//    ratio of the first strict minimum over j = 0 (1.0) .. n_clip-1 (clip_lo).
// ---------------------------------------------------------------------------
__global__ void clip_select_kernel(const float* __restrict__ colpart, int64_t n_mt, int64_t d_out,
                                   int n_clip, float clip_lo, const OutScales* __restrict__ sc,
                                   float* __restrict__ clip, float* __restrict__ clip_err) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= d_out) return;
  int best = 0;
  double be = 0.0;
  for (int j = 0; j < n_clip; ++j) {
    double e = 0.0;
    for (int64_t mt = 0; mt < n_mt; ++mt) e += (double)colpart[((int64_t)j * n_mt + mt) * d_out + o];
    e *= sc->inv[j];
    if (clip_err != nullptr) clip_err[o * n_clip + j] = (float)e;
    if (j == 0 || e < be) { be = e; best = j; }
  }
  clip[o] = clip_ratio(best, n_clip, clip_lo);
}

hipError_t launch_clip_select(const float* colpart, int64_t n_mt, int64_t d_out, int n_clip,
                              float clip_lo, const OutScales* sc, float* clip, float* clip_err,
                              hipStream_t stream) {
  clip_select_kernel<<<(unsigned)((d_out + 255) / 256), 256, 0, stream>>>(colpart, n_mt, d_out, n_clip,
                                                                          clip_lo, sc, clip, clip_err);
  return hipGetLastError();
}

}  // namespace awq
