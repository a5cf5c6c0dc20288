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
//   2. build_dw (max pass, then write pass): dW_c with the same bit-exact codes
//      as the pack kernel, scaled by a power of two from its exact maximum and
//      rounded to fp16 -- 3 more mantissa bits than bf16 at the same matrix-core
//      rate, which keeps the relative error of the errors near 1e-4 even for
//      a few tokens and rows (one pass over W per candidate, negligible next to
//      the GEMM);
//   3. gemm_sq: fp16 MFMA 32x32x16 GEMM over all candidates of a chunk at once
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

// WRITE = false: per-block max |dW_c| -> dmax[(c - cand0) * gridDim.x + block]
// WRITE = true:  dW16[c - cand0] = fp16(dW_c * ds[c])
// ASYM: codes of the asymmetric grid (range [min(0, min v), max(0, max v)],
//   both ends times the clip ratio in mode 1, step RN(range / 15), exact zero
//   point and codes; the signed code clamp(n, -z, 15 - z) times the step)
//   dW16 rows are d_out_pad apart per candidate and K_pad elements long; rows
//   d_out .. d_out_pad-1 and columns d_in .. K_pad-1 are written as zeros.
template <int G, bool WRITE, bool ASYM>
__global__ __launch_bounds__(kDwThreads) void build_dw_kernel(
    const WParts P, int64_t d_out, int64_t d_in, int64_t d_out_pad, int64_t K_pad, int mode,
    const float* __restrict__ S, const float* __restrict__ s_best, int n_clip, float clip_lo, int cand0,
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
  const float dsc = WRITE ? sc->ds[c] : 1.0f;
  uint32_t outw[8];
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float n = step > 0.0f ? code_exact(v[j], step, inv) : 0.0f;
    n = __builtin_fminf(__builtin_fmaxf(n, qlo), qhi);
    // w_hat - w = (q * step - w * s) / s, formed in the scaled domain with one
    // fma and the hardware reciprocal of s: within a few fp32 ulp of
    // RN(RN(q * step) / s) - w, far below the fp16 rounding of the operand
    // (the codes q themselves are exact)
    const float d = __builtin_fmaf(n, step, -v[j]) * __builtin_amdgcn_rcpf(sv[j]);
    if constexpr (WRITE) {
      const uint32_t b = f2h_bits(d * dsc);       // exact scaling by 2^e, one rounding
      if (j & 1) outw[j >> 1] |= b << 16;
      else outw[j >> 1] = b;
    } else {
      mx = __builtin_fmaxf(mx, __builtin_fabsf(d));
    }
  }
  if constexpr (WRITE) {
    if (row >= d_out_pad) return;
    uint16_t* rowp = dw + (int64_t)blockIdx.y * d_out_pad * K_pad + row * K_pad;
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

hipError_t launch_build_dw(int group_size, bool asym, const WParts& parts, int64_t d_out, int64_t d_in,
                           int64_t d_out_pad, int64_t K_pad, int n_cand, int mode, const float* S, const float* s_best,
                           int n_clip, float clip_lo, int cand0, const OutScales* sc, float* dmax, uint16_t* dw,
                           hipStream_t stream) {
  // max pass: d_out rows; write pass: d_out_pad rows (zeros past d_out)
  dim3 grid((unsigned)build_dw_blocks(group_size, dw == nullptr ? d_out : d_out_pad, d_in), (unsigned)n_cand);
#define AWQ_DW2(G, A)                                                                         \
  if (dw == nullptr) build_dw_kernel<G, false, A><<<grid, kDwThreads, 0, stream>>>(             \
      parts, d_out, d_in, d_out_pad, K_pad, mode, S, s_best, n_clip, clip_lo, cand0, sc, dmax, dw); \
  else build_dw_kernel<G, true, A><<<grid, kDwThreads, 0, stream>>>(                            \
      parts, d_out, d_in, d_out_pad, K_pad, mode, S, s_best, n_clip, clip_lo, cand0, sc, dmax, dw);
#define AWQ_DW(G) \
  if (asym) { AWQ_DW2(G, true) } else { AWQ_DW2(G, false) }
  switch (group_size) {
    case 32: AWQ_DW(32) break;
    case 64: AWQ_DW(64) break;
    default: AWQ_DW(128) break;
  }
#undef AWQ_DW
#undef AWQ_DW2
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

// xmax: [n_x] partial maxima of |X|; dmax: [n_cand, n_d].  Block c sets ds[c]
// and inv[c] (every block derives the same xs from the X partials).
__global__ __launch_bounds__(256) void out_scales_kernel(const float* __restrict__ xmax, int64_t n_x,
                                                        const float* __restrict__ dmax, int64_t n_d, int n_cand,
                                                        OutScales* __restrict__ sc) {
  __shared__ float red[256];
  const int c = blockIdx.x;
  const float xs = pow2_scale_for(block_max256(xmax, n_x, red));
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
  out_scales_kernel<<<n_cand, 256, 0, stream>>>(xmax_part, n_x, dmax, n_d, n_cand, sc);
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

// ---------------------------------------------------------------------------
// 2. GEMM of squares: Y = X16 dW^T over the concatenated candidates
//    (N_total = n_cand * d_out_pad columns, each candidate padded to a multiple
//    of the tile with zero rows; M and K padded likewise with zeros), and per
//    column the sum over the block's 256 tokens of Y^2 -> colpart[mt][n].
//
//    Block tile 256 x 256, 8 waves (2 x 4), wave tile 128 x 64 = 4 x 2 MFMA
//    32x32x16 f16 tiles; 128 fp32 accumulators per lane, 168 registers in
//    all, so two waves share a SIMD and one issues MFMAs while the other
//    waits (measured 4-5% faster than 4 waves of 128 x 128 tiles with one
//    wave per SIMD, 1.5% faster than 16 waves of 64 x 64).  A wave reads 6
//    fragments (6 KiB of LDS) per 8 MFMAs.  K advances in stages of 32 through a ring of 4 LDS slots, one
//    distinct array per slot and operand: the operands go from global memory
//    straight into LDS (buffer loads with the LDS bit, 16 bytes per lane, no
//    staging registers and no LDS store instructions), three stages ahead of
//    the MFMAs.  At the end of a stage each wave waits until its loads of the
//    next stage have landed (two younger stages stay in flight) and the
//    block meets at a barrier without a memory fence, which would wait for
//    every load.  The separate slot arrays let the compiler see that fragment
//    reads never alias the loads in flight.  16-byte K-chunks are
//    XOR-swizzled by row so that fragment reads are free of bank conflicts;
//    since a direct load places lane i at byte 16 i of its 1 KiB, the swizzle
//    is applied on the global side (each lane fetches the chunk its LDS slot
//    holds).  Measured: 6-7% faster than staging the operands through
//    registers with LDS stores, identical results.
//    The block order is remapped so that each XCD owns a contiguous range of
//    tiles, walked in groups of up to 8 M-tiles: concurrent blocks of one XCD
//    share A and B tiles in its L2.
// ---------------------------------------------------------------------------
constexpr int kBM = 256, kBN = 256, kBK = 32;
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
__shared__ __attribute__((aligned(1024))) uint16_t sA3[kBM * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB0[kBN * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB1[kBN * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB2[kBN * kBK];
__shared__ __attribute__((aligned(1024))) uint16_t sB3[kBN * kBK];

// one operand tile (256 rows x 32 K) straight into LDS: wave w fetches rows
// 32w .. 32w+31 in 2 loads of 16 rows; lane i lands in row 32w + 16n + i/4,
// slot i%4, and fetches chunk (i%4) ^ swz(row) = (i%4) ^ ((i/16) & 3)
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* dst, int wave, uint32_t vo,
                                         uint32_t soff, uint32_t row16_bytes) {
#pragma unroll
  for (int n = 0; n < 2; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + (32 * wave + 16 * n) * kBK), 16, vo,
                                             soff + (uint32_t)n * row16_bytes, 0, 0);
}

__device__ __forceinline__ void mfma_stage(const uint16_t* As, const uint16_t* Bs, int wm, int wn, int lane,
                                           f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    const int kc = 2 * ks + (lane >> 5);
    uint4 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(As, wm * 128 + i * 32 + (lane & 31), kc);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = frag(Bs, wn * 64 + j * 32 + (lane & 31), kc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f16(a[i], b[j], acc[i][j]);
  }
}

__global__ __launch_bounds__(kGemmThreads, 2) void gemm_sq_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                              uint32_t a_bytes, const uint16_t* __restrict__ B,
                                                              int64_t ldb, uint32_t b_bytes, int64_t K, int64_t n_mt,
                                                              int64_t n_nt, float* __restrict__ colpart, int64_t ldc,
                                                              int group_m) {
  __shared__ float red[2][kBN];
  const int64_t nblk = (int64_t)gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % kXcds, pos = bid / kXcds;
  const int64_t q = nblk / kXcds, r = nblk % kXcds;
  const int64_t id = xcd * q + (xcd < r ? xcd : r) + pos;
  const int64_t per_group = (int64_t)group_m * n_nt;
  const int64_t first_m = (id / per_group) * group_m;
  const int64_t gsz = (n_mt - first_m) < group_m ? (n_mt - first_m) : group_m;
  const int64_t mt = first_m + (id % per_group) % gsz;
  const int64_t nt = (id % per_group) / gsz;
  const int64_t m0 = mt * kBM, n0 = nt * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (int)(K / kBK);  // even (K is a multiple of 64)
  const uint32_t ld2 = (uint32_t)(lda * 2);
  const uint32_t vo = (uint32_t)((lane >> 2) * ld2 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));
  const uint32_t row16 = 16 * ld2;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(B, b_bytes);
  const uint32_t sA = (uint32_t)((m0 + 32 * wave) * lda * 2), sB = (uint32_t)((n0 + 32 * wave) * ldb * 2);
  // k-tile t (clamped: past the end the ring re-fetches the last tile into a free buffer)
  auto koff = [&](int t) { return (uint32_t)((t < nk ? t : nk - 1) * kBK * 2); };

  // prologue: stages 0, 1, 2 in flight; wait for stage 0
  dma_tile(rsA, sA0, wave, vo, sA + koff(0), row16);
  dma_tile(rsB, sB0, wave, vo, sB + koff(0), row16);
  dma_tile(rsA, sA1, wave, vo, sA + koff(1), row16);
  dma_tile(rsB, sB1, wave, vo, sB + koff(1), row16);
  dma_tile(rsA, sA2, wave, vo, sA + koff(2), row16);
  dma_tile(rsB, sB2, wave, vo, sB + koff(2), row16);
  __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8) lgkmcnt(0): this wave's stage-0 loads are in LDS
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // stage kt on ring slot S: fetch stage kt + 3 into slot S + 3 (freed by the
  // previous barrier), MFMAs on slot S, then wait until stage kt + 1 is in
  // LDS (stages kt + 2 and kt + 3 may still be in flight) and all reads of
  // slot S are done, barrier
#define AWQ_STAGE4(S, SN)                                                       \
  {                                                                             \
    dma_tile(rsA, sA##SN, wave, vo, sA + koff(kt + 3), row16);                  \
    dma_tile(rsB, sB##SN, wave, vo, sB + koff(kt + 3), row16);                  \
    mfma_stage(sA##S, sB##S, wm, wn, lane, acc);                                \
    __builtin_amdgcn_s_waitcnt(0x0078);                                         \
    asm volatile("" ::: "memory");                                              \
    __builtin_amdgcn_s_barrier();                                               \
    asm volatile("" ::: "memory");                                              \
    ++kt;                                                                       \
  }
  int kt = 0;
  for (; kt + 4 <= nk;) {
    AWQ_STAGE4(0, 3)
    AWQ_STAGE4(1, 0)
    AWQ_STAGE4(2, 1)
    AWQ_STAGE4(3, 2)
  }
  if (kt < nk) {  // nk % 4 == 2
    AWQ_STAGE4(0, 3)
    AWQ_STAGE4(1, 0)
  }
#undef AWQ_STAGE4
  __builtin_amdgcn_s_waitcnt(0x0070);  // no load in flight past this point

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float cs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) cs = __builtin_fmaf(acc[i][j][e], acc[i][j][e], cs);
    cs += __shfl_xor(cs, 32, kWave);
    if (lane < 32) red[wm][wn * 64 + j * 32 + lane] = cs;
  }
  __syncthreads();
  if (tid < kBN) colpart[mt * ldc + n0 + tid] = red[0][tid] + red[1][tid];
}

// K is padded to a multiple of 64 = two ring stages: the stage count is even,
// so the 4-slot ring ends with zero or one pair of stages after its loop
void gemm_sq_pad(int64_t T, int64_t d_out, int64_t d_in, int64_t* T_pad, int64_t* d_out_pad, int64_t* K_pad) {
  *T_pad = (T + kBM - 1) / kBM * kBM;
  *d_out_pad = (d_out + kBN - 1) / kBN * kBN;
  *K_pad = (d_in + 2 * kBK - 1) / (2 * kBK) * (2 * kBK);
}

// M-tiles per tile group: each XCD walks its tiles in groups of group_m
// M-tiles, so the 8 XCDs keep 8 * group_m A panels (256 rows x K each) in
// use.  The largest group (up to 8) whose panels fit in ~224 MiB of the
// 256 MB MALL is taken, so that A re-reads across rounds of tiles stay there:
// 8 at K = 4096, 4 at K = 12288 (measured 6% faster there than 8).
static int gemm_group_m(int64_t K_pad) {
  const double budget = 224.0 * 1024 * 1024;
  int g = 8;
  while (g > 1 && 8.0 * g * kBM * (double)K_pad * 2.0 > budget) g /= 2;
  return g;
}

hipError_t launch_gemm_sq(const uint16_t* X16, int64_t T_pad, int64_t K_pad, const uint16_t* dw, int64_t n_cols,
                          float* colpart, int64_t ldc, hipStream_t stream) {
  const int64_t n_mt = T_pad / kBM, n_nt = n_cols / kBN;
  const uint32_t a_bytes = (uint32_t)(T_pad * K_pad * 2), b_bytes = (uint32_t)(n_cols * K_pad * 2);
  gemm_sq_kernel<<<(unsigned)(n_mt * n_nt), kGemmThreads, 0, stream>>>(X16, K_pad, a_bytes, dw, K_pad, b_bytes, K_pad,
                                                                      n_mt, n_nt, colpart, ldc, gemm_group_m(K_pad));
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
