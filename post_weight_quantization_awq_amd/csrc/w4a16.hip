// W4A16 product on the packed layout: Y [M, d_out] = X [M, d_in] W_hat^T,
// W_hat[o, i] = (u[o, i] - z[g, o]) * scale[g, o], g = i / G.
// "AWQ architecture, in depth", section "Kernels: why W4A16 is fast at
// decode": the packed 4-bit weights are dequantized in registers with the
// group's scale and zero point and multiplied with 16-bit activations; at
// decode (a few tokens) the product is bound by reading the weights.
// "Weight-Only Quantization: GPTQ and AWQ", sections "The kernels" and "6-9":
// qweight int32 [d_in, d_out/8], scales fp16 [d_in/G, d_out], zeros int32
// [d_in/G, d_out/8], nibble j of a word holding output 8m + order[j],
// order = [0,2,4,6,1,3,5,7].
//
// Decode GEMV, HBM-bound (0.5 B of codes + (2 + 0.5) / G B of scales and
// zeros per weight).  Split over the inputs so that a launch holds enough
// waves to keep HBM busy: block (c, k) owns 512 outputs (one packed word per
// lane: a wave reads 256 contiguous bytes of a qweight row) and 256 input
// rows, 32 per wave (one zero-point segment: every group size is a multiple
// of 32), all 32 loads in flight at once.  The activations of the slice are
// loaded first and staged in LDS as fp32, so the first rows' arithmetic waits
// only for their own codes and every product is a plain fp32 FMA.  The zero
// point factors out of the segment:
//   sum_i x_i (u_i - z) scale = scale * (sum_i x_i u_i - z * sum_i x_i).
// A code word is masked into two words of bytes (even and odd nibbles) and
// each byte converts to fp32 in one instruction (the masks go through an
// opaque ALU op, or the compiler re-extracts every nibble with a bit-field
// extract); products u * x are exact in fp32 and accumulate in fp32: 2.5 VALU
// operations per weight at one token.  (Pairing two rows into fp16 (u - z)
// with a byte permute and one v_dot2 per pair needs 1.75 operations per
// weight but measured 4% slower: the kernel is not issue-bound.)  The eight
// waves' results are added in LDS in a fixed order and written as one fp32
// partial per (row slice, token, output); a second launch adds the partials
// of the row slices in a fixed order and rounds once to the output type.
// (Letting the last block of each column do that sum needs a device-scope
// release before every block's arrival, which here writes back the L2 of the
// block's XCD: 6-8x slower than the second launch.)  Tokens are handled MT
// (1, 2 or 4) at a time; the weights are read once per token chunk.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kGvThreads = 512;
constexpr int kGvWaves = kGvThreads / kWave;
constexpr int kGvRows = 32;                     // input rows per wave (one zero-point segment)
constexpr int kGvSlice = kGvRows * kGvWaves;    // input rows per block
constexpr int kGvCols = kWave * 8;              // outputs per block

int64_t w4a16_slices(int64_t d_in) { return (d_in + kGvSlice - 1) / kGvSlice; }

// a & b through an opaque ALU op, so that the bytes of the result convert with
// v_cvt_f32_ubyte{0..3} instead of being re-extracted from the unmasked word
__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// (a & m) | c in one VALU op (the compiler otherwise emits an and and an or);
// m and c are held in VGPRs (a VOP3 op reads at most one scalar operand here)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

template <int MT>
__global__ __launch_bounds__(kGvThreads) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ X, int64_t ld_x, int m_valid, int64_t d_in, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int64_t d_out, int group_size,
    float* __restrict__ part) {
  constexpr int kXPer = (MT * kGvSlice + kGvThreads - 1) / kGvThreads;  // staged activations per thread
  __shared__ __align__(16) float xs[MT][kGvSlice];
  __shared__ float red[kGvWaves][MT][kGvCols];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t n_words = (uint32_t)(d_out / 8);
  const uint32_t m = blockIdx.x * kWave + lane;  // packed word column of this lane
  const uint32_t mm = m < n_words ? m : n_words - 1;
  const int64_t k0 = (int64_t)blockIdx.y * kGvSlice;
  const int64_t r0 = k0 + (int64_t)wv * kGvRows;

  // activations of the slice first, issued before the codes and
  // unconditionally (the compiler waits for a load under a branch inside the
  // branch, before the codes are requested); out-of-range entries read X[0]
  // and are masked when staged
  uint16_t xr[kXPer];
  bool xok[kXPer];
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int idx = q * kGvThreads + tid;
    const int t = idx / kGvSlice, c = idx % kGvSlice;
    const int64_t row = k0 + c;
    xok[q] = idx < MT * kGvSlice && t < m_valid && row < d_in;
    xr[q] = X[xok[q] ? t * ld_x + row : 0];
  }
  // codes: this lane's word in the wave's 32 rows (a partial last slice
  // re-reads row d_in - 1; its activations are zero)
  uint32_t w[kGvRows];
  const uint32_t* base = qweight + (uint64_t)min(r0, d_in - 1) * n_words + mm;
  if (r0 + kGvRows <= d_in) {
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) w[r] = __builtin_nontemporal_load(base + (uint32_t)r * n_words);
  } else {
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) {
      const uint32_t rr = (uint32_t)min((int64_t)r, max(d_in - 1 - r0, (int64_t)0));
      w[r] = __builtin_nontemporal_load(base + rr * n_words);
    }
  }
  const int64_t g = min(r0, d_in - 1) / group_size;
  const uint4 sraw = *(const uint4*)(scales + g * d_out + 8 * (int64_t)mm);
  const uint32_t zw = qzeros != nullptr ? qzeros[g * n_words + mm] : 0x77777777u;
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int idx = q * kGvThreads + tid;
    if (idx < MT * kGvSlice) xs[idx / kGvSlice][idx % kGvSlice] = xok[q] ? h2f(xr[q]) : 0.0f;
  }
  __syncthreads();

  float acc[MT][8], sx[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    sx[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = 0.0f;
  }
#pragma unroll
  for (int r4 = 0; r4 < kGvRows; r4 += 4) {
    float xv[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float4 v = *(const float4*)&xs[t][wv * kGvRows + r4];  // same address on every lane
      xv[t][0] = v.x; xv[t][1] = v.y; xv[t][2] = v.z; xv[t][3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t wr = w[r4 + e];
      const uint32_t lo = and_opaque(wr, 0x0F0F0F0Fu), hi = and_opaque(wr >> 4, 0x0F0F0F0Fu);
      float u[8];  // u[j]: nibble j (even j from lo, odd j from hi, byte j / 2)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
        u[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        sx[t] += xv[t][e];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = __builtin_fmaf(u[j], xv[t][e], acc[t][j]);
      }
    }
  }
  // fold the zero point and the scale; nibble j belongs to output 8m + order[j]
  constexpr int kOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  const uint32_t sw[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int o = kOrder[j];
    const float sc = h2f((uint16_t)((sw[o >> 1] >> (16 * (o & 1))) & 0xFFFFu));
    const float z = (float)((zw >> (4 * j)) & 0xFu);
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wv][t][lane * 8 + o] = sc * __builtin_fmaf(-z, sx[t], acc[t][j]);
  }
  __syncthreads();
  // the eight waves in a fixed order; 4 outputs per thread and store
  const int64_t o_base = (int64_t)blockIdx.x * kGvCols;
  for (int idx = tid; idx < MT * (kGvCols / 4); idx += kGvThreads) {
    const int t = idx / (kGvCols / 4), c4 = (idx % (kGvCols / 4)) * 4;
    if (t >= m_valid || o_base + c4 >= d_out) continue;
    float4 v = *(const float4*)&red[0][t][c4];
#pragma unroll
    for (int q = 1; q < kGvWaves; ++q) {
      const float4 a = *(const float4*)&red[q][t][c4];
      v.x += a.x;
      v.y += a.y;
      v.z += a.z;
      v.w += a.w;
    }
    *(float4*)(part + ((int64_t)blockIdx.y * MT + t) * d_out + o_base + c4) = v;
  }
}

// Y[t, o] = sum over the row slices of part[slice, t, o], rounded once to
// fp16 or kept in fp32.  Block (c, t): 64 columns of 4 outputs; thread
// (column, lane q of 4) adds slices q, q + 4, q + 8, ... in order (8 loads in
// flight), then the four sums are added in the order q = 0..3.
constexpr int kRdCols = 64;
constexpr int kRdSplit = 4;
__global__ __launch_bounds__(kRdCols * kRdSplit) void w4a16_reduce_kernel(const float* __restrict__ part,
                                                                          int64_t n_slices, int mt, int64_t d_out,
                                                                          void* __restrict__ Y, int64_t ld_y,
                                                                          int y_f16) {
  __shared__ float4 ps[kRdSplit][kRdCols];
  const int col = threadIdx.x % kRdCols, q = threadIdx.x / kRdCols;
  const int64_t t = blockIdx.y;
  const int64_t o = ((int64_t)blockIdx.x * kRdCols + col) * 4;
  const bool live = o < d_out;
  const int64_t oo = live ? o : 0;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t k0 = q; k0 < n_slices; k0 += 8 * kRdSplit) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t k = k0 + (int64_t)u * kRdSplit;
      v[u] = k < n_slices ? *(const float4*)(part + (k * mt + t) * d_out + oo) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += v[u].x;
      s.y += v[u].y;
      s.z += v[u].z;
      s.w += v[u].w;
    }
  }
  ps[q][col] = s;
  __syncthreads();
  if (q != 0 || !live) return;
  float4 r = ps[0][col];
#pragma unroll
  for (int i = 1; i < kRdSplit; ++i) {
    r.x += ps[i][col].x;
    r.y += ps[i][col].y;
    r.z += ps[i][col].z;
    r.w += ps[i][col].w;
  }
  if (y_f16) {
    uint2 h;
    h.x = (uint32_t)f2h_bits(r.x) | ((uint32_t)f2h_bits(r.y) << 16);
    h.y = (uint32_t)f2h_bits(r.z) | ((uint32_t)f2h_bits(r.w) << 16);
    *(uint2*)((uint16_t*)Y + t * ld_y + o) = h;
  } else {
    *(float4*)((float*)Y + t * ld_y + o) = r;
  }
}

int64_t w4a16_cols(int64_t d_out) { return (d_out / 8 + kWave - 1) / kWave; }

// ---------------------------------------------------------------------------
// Few tokens (2..64): one read of every packed word for all tokens, products on
// the matrix cores (v_mfma_f32_16x16x32_f16).  A = weights (16 outputs x 32
// inputs), B = the activations (32 inputs x a tile of 16 tokens, zero past the
// last token; the code words are dequantized again for every tile).  A wave owns 32 word columns (256 outputs) of a 128-row chunk; lane
// l loads the word pair of columns c0 + 2 (l & 15) + {0, 1} in rows
// k + 8 (l >> 4) + 0..7 of each 32-row step with one 8-byte load per row, so a
// load instruction reads four whole 128-byte runs of packed rows (a strip of
// 16 columns, 64-byte runs, measured 35% slower on the same bytes).  The code
// of output 8c + order[j] is nibble j of a word, so nibble position j of the
// lane's 8 words of one column is exactly lane l's part of the A fragment of
// the 16 outputs {8 (c0 + 2i + h) + order[j]}: no data moves between lanes.
// One v_perm_b32 puts byte b of two rows side by side; an and-or with 0x6400
// makes fp16 1024 + u (low nibble, j = 2b) or 1024 + 16 u (high nibble,
// j = 2b + 1), and a packed fp16 subtract of 1024 + z (or 1024 + 16 z) leaves
// the exact (u - z) or 16 (u - z): 1.25 VALU operations per weight.  The
// products of a group accumulate alone in fp32; at the group's end they are
// multiplied by the group's fp32 scale (over 16 for the odd nibbles) and added
// into the wave's slot in LDS, so no rounding touches a dequantized weight and
// no second set of accumulators is held in registers.  The 4 waves of a block
// take the 4 chunks of the block's 512-row input range, all loads of a chunk
// in flight at once (two waves per SIMD); their slots are added in a fixed
// order, and the reduction kernel adds the ranges' fp32 results in order (a
// single range writes Y directly).
// ---------------------------------------------------------------------------
constexpr int kSkTile = 16;                   // tokens per B operand
constexpr int kSkMaxTokens = 64;
constexpr int kSkWords = 32;                   // word columns per block (and per wave)
constexpr int kSkWaves = 4;
constexpr int kSkChunk = 128;                  // input rows per wave
constexpr int kSkSteps = kSkChunk / 32;
constexpr int kSkSlot = 68;                    // floats per lane in LDS (64 results, padded)

typedef _Float16 h8s __attribute__((ext_vector_type(8)));
typedef float f4s __attribute__((ext_vector_type(4)));
typedef uint32_t u2s __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_sub_f16(uint32_t a, uint32_t b) {
  const h2 r = __builtin_bit_cast(h2, a) - __builtin_bit_cast(h2, b);
  return __builtin_bit_cast(uint32_t, r);
}

// fp16 1024 + z (low nibbles) and 1024 + 16 z (high nibbles) in both halves,
// for the 8 nibbles of a packed zero-point word
__device__ __forceinline__ void zero_consts(uint32_t zw, uint32_t* zc) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t zl = (zw >> (8 * b)) & 0xFu, zh = (zw >> (8 * b + 4)) & 0xFu;
    zc[2 * b] = (0x6400u | zl) * 0x10001u;
    zc[2 * b + 1] = (0x6400u | (zh << 4)) * 0x10001u;
  }
}

// One 32-row step of word column h of the lane's pair: the 8 codes of the
// lane's rows dequantized to exact fp16 (u - z) (or 16 (u - z), odd nibbles)
// and multiplied with the activations, one product per nibble position j.
__device__ __forceinline__ void skinny_mma(const u2s (&ws)[8], int h, const uint32_t (&zc)[8], h8s bx,
                                           f4s (&acc)[8]) {
  uint32_t a[8][4];   // a[j][p]: fp16 pair (rows 2p, 2p + 1) of nibble j
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = (uint32_t)b | (12u << 8) | ((uint32_t)(4 + b) << 16) | (12u << 24);
      const uint32_t x2 = __builtin_amdgcn_perm(ws[2 * p + 1][h], ws[2 * p][h], sel);
      a[2 * b][p] = pk_sub_f16(and_or(x2, 0x000F000Fu, 0x64006400u), zc[2 * b]);
      a[2 * b + 1][p] = pk_sub_f16(and_or(x2, 0x00F000F0u, 0x64006400u), zc[2 * b + 1]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 av = make_uint4(a[j][0], a[j][1], a[j][2], a[j][3]);
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8s, av), bx, acc[j], 0, 0, 0);
  }
}

// A group's sums of word column h times the group's scales (sg: the strip's
// 256 scales of the group, in LDS) into half hs of the lane's slot: written by
// the first group of the chunk, added by the others.
__device__ __forceinline__ void skinny_fold(const f4s (&acc)[8], const uint16_t* sg, int lh, int h, int hs,
                                            float* my, bool first) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    // scales of word column c0 + 8 lh + 2 v + h
    const uint4 sv = *(const uint4*)(sg + 8 * (8 * lh + 2 * v + h));
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    float val[8];   // the 8 outputs of the word column, in output order
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      constexpr int kOrd[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      const int o = kOrd[j];
      float sc = h2f((uint16_t)((sw[o >> 1] >> (16 * (o & 1))) & 0xFFFFu));
      if (j & 1) sc *= 0.0625f;   // the odd nibbles carry 16 (u - z)
      val[o] = acc[j][v] * sc;
    }
    f4s* dst = (f4s*)(my + (hs * 4 + v) * 8);
    const f4s lo = {val[0], val[1], val[2], val[3]}, hi = {val[4], val[5], val[6], val[7]};
    if (first) {
      dst[0] = lo;
      dst[1] = hi;
    } else {
      dst[0] = dst[0] + lo;
      dst[1] = dst[1] + hi;
    }
  }
}

// MULTI: more than 16 tokens, in tiles of 16 (the B operand's columns).
template <int G, bool Y_F16, bool MULTI>
__global__ __launch_bounds__(kSkWaves * kWave, 2) void w4a16_skinny_kernel(
    const uint16_t* __restrict__ X, int64_t ld_x, int m_valid, int64_t d_in, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int64_t d_out, int n_strips,
    void* __restrict__ Y, int64_t ld_y, float* __restrict__ part) {
  constexpr int kSpg = G / 32;   // steps per quantization group
  // slot[w][lane][(h * 4 + v) * 8 + e]: wave w's sum for the lane's token and
  // output 8 (c0 + 8 (lane >> 4) + 2 v + h) + e
  __shared__ __align__(16) float slot[kSkWaves][kWave][kSkSlot];
  __shared__ __align__(16) uint16_t scl[kSkWaves][kSkSteps][kSkWords * 8];   // each wave's group scales
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n_words = d_out / 8;   // even
  // blocks go round-robin to the 8 XCDs: tile t of XCD x takes the x-th eighth of
  // the (strip, range) tiles, strips fastest, so neighbouring strips of a packed
  // row are read through the same L2
  const uint32_t nblk = gridDim.x, bid = blockIdx.x;
  const uint32_t xcd = bid % 8, q = nblk / 8, rmd = nblk % 8;
  const uint32_t tile = xcd * q + (xcd < rmd ? xcd : rmd) + bid / 8;
  const uint32_t strip = tile % (uint32_t)n_strips, range = tile / (uint32_t)n_strips;
  const int64_t c0 = (int64_t)strip * kSkWords;
  const int li = lane & 15, lh = lane >> 4;               // row of the A / B fragment, 8-input run
  // this lane's word pair (a pair past the last column re-reads the last pair;
  // its outputs are never stored)
  const int64_t cp = c0 + 2 * li + 2 <= n_words ? c0 + 2 * li : n_words - 2;
  const int64_t r0 = ((int64_t)range * kSkWaves + wv) * kSkChunk;
  const uint16_t* xrow = X + (int64_t)(li < m_valid ? li : m_valid - 1) * ld_x + 8 * lh;   // tile 0
  float* my = &slot[wv][lane][0];

  // Every step of the chunk runs, with no branch, so that all loads go out at
  // once in step order and each step waits only for its own: a step past d_in
  // (the last range only) reads the last 32 rows again and multiplies them by
  // zero activations, which adds exact zeros.
  int64_t ks[kSkSteps];
  bool live[kSkSteps];
#pragma unroll
  for (int st = 0; st < kSkSteps; ++st) {
    live[st] = r0 + 32 * st < d_in;
    ks[st] = live[st] ? r0 + 32 * st : d_in - 32;
  }
  // The zero points and scales of every group of the chunk first (the scales
  // of the strip's 256 outputs, 8 bytes a lane, staged through LDS; a lane past
  // d_out re-reads the last 4), then the code words and activations of every
  // step, so that no wait for a later group's constants drains the loads.
  constexpr int kGroups = kSkSteps / kSpg;
  uint32_t zw[kGroups][2];
  u2s sgr[kGroups];
  const int64_t so = 8 * c0 + 4 * lane + 4 <= d_out ? 8 * c0 + 4 * lane : d_out - 4;
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int64_t g = ks[gi * kSpg] / G;
    zw[gi][0] = qzeros != nullptr ? qzeros[g * n_words + cp] : 0x77777777u;
    zw[gi][1] = qzeros != nullptr ? qzeros[g * n_words + cp + 1] : 0x77777777u;
    sgr[gi] = *(const u2s*)(scales + g * d_out + so);
  }
  u2s w[kSkSteps][8];
  uint4 xv[kSkSteps];
#pragma unroll
  for (int st = 0; st < kSkSteps; ++st) {
    const uint32_t* wp = qweight + (ks[st] + 8 * lh) * n_words + cp;
#pragma unroll
    for (int r = 0; r < 8; ++r) w[st][r] = __builtin_nontemporal_load((const u2s*)(wp + r * n_words));
    xv[st] = *(const uint4*)(xrow + ks[st]);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any arithmetic below
  uint16_t* ssc = &scl[wv][0][0];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) *(u2s*)(ssc + gi * kSkWords * 8 + 4 * lane) = sgr[gi];

  // the results of one token tile of the slots: 8 consecutive outputs (word
  // column c0 + q8) of token t, half hs of lane ln's slot, the waves added in
  // order 0..3
  auto store8 = [&](int t, int q8, int ln, int hs) {
    const int64_t o = (c0 + q8) * 8;
    if (t >= m_valid || o >= d_out) return;
    const int off = (hs * 4 + ((q8 >> 1) & 3)) * 8;
    f4s lo = *(const f4s*)&slot[0][ln][off], hi = *(const f4s*)&slot[0][ln][off + 4];
#pragma unroll
    for (int w2 = 1; w2 < kSkWaves; ++w2) {
      lo = lo + *(const f4s*)&slot[w2][ln][off];
      hi = hi + *(const f4s*)&slot[w2][ln][off + 4];
    }
    const float r[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (part != nullptr) {
      float* dst = part + ((int64_t)range * m_valid + t) * d_out + o;
      *(float4*)dst = make_float4(r[0], r[1], r[2], r[3]);
      *(float4*)(dst + 4) = make_float4(r[4], r[5], r[6], r[7]);
    } else if (Y_F16) {
      uint16_t* dst = (uint16_t*)Y + t * ld_y + o;
      *(uint2*)dst = make_uint2((uint32_t)f2h_bits(r[0]) | ((uint32_t)f2h_bits(r[1]) << 16),
                                (uint32_t)f2h_bits(r[2]) | ((uint32_t)f2h_bits(r[3]) << 16));
      *(uint2*)(dst + 4) = make_uint2((uint32_t)f2h_bits(r[4]) | ((uint32_t)f2h_bits(r[5]) << 16),
                                      (uint32_t)f2h_bits(r[6]) | ((uint32_t)f2h_bits(r[7]) << 16));
    } else {
      float* dst = (float*)Y + t * ld_y + o;
      *(float4*)dst = make_float4(r[0], r[1], r[2], r[3]);
      *(float4*)(dst + 4) = make_float4(r[4], r[5], r[6], r[7]);
    }
  };

  if constexpr (!MULTI) {
    // one tile: both word columns of the pair per step
    const bool tok = li < m_valid;
    f4s acc[2][8];
    uint32_t zc[2][8];
#pragma unroll
    for (int st = 0; st < kSkSteps; ++st) {
      if (st % kSpg == 0) {   // a group starts: its zero points, fresh sums
        zero_consts(zw[st / kSpg][0], zc[0]);
        zero_consts(zw[st / kSpg][1], zc[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] = (f4s){0.0f, 0.0f, 0.0f, 0.0f};
      }
      // masked where used, so that a step waits only for its own loads
      const h8s bx = __builtin_bit_cast(h8s, (tok && live[st]) ? xv[st] : make_uint4(0u, 0u, 0u, 0u));
      skinny_mma(w[st], 0, zc[0], bx, acc[0]);
      skinny_mma(w[st], 1, zc[1], bx, acc[1]);
      if ((st + 1) % kSpg == 0) {   // the group ends: its sums times its scales into the slot
        skinny_fold(acc[0], ssc + (st / kSpg) * kSkWords * 8, lh, 0, 0, my, st + 1 == kSpg);
        skinny_fold(acc[1], ssc + (st / kSpg) * kSkWords * 8, lh, 1, 1, my, st + 1 == kSpg);
      }
    }
    __syncthreads();
    for (int idx = tid; idx < kSkTile * kSkWords; idx += kSkWaves * kWave) {
      const int t = idx / kSkWords, q8 = idx % kSkWords;   // token, word column in the strip
      store8(t, q8, t + 16 * (q8 >> 3), q8 & 1);
    }
  } else {
    // Passes of NT tiles (NT = 2 at G = 128: each dequantized fragment feeds
    // the products of both tiles; 1 at smaller groups, whose extra folds leave
    // no registers for a second set of sums).  Per pass, word column h = 0 of
    // every lane's pair, then h = 1, each through the slots (half hs = the
    // tile of the pass) and stored before the next.
    constexpr int NT = G == 128 ? 2 : 1;
    uint4 xt[NT][kSkSteps];   // activations of the pass's tiles
#pragma unroll
    for (int st = 0; st < kSkSteps; ++st) xt[0][st] = xv[st];
#pragma unroll
    for (int ti = 1; ti < NT; ++ti) {
      const int tn = kSkTile * ti + li;
      const uint16_t* xr = X + (int64_t)(tn < m_valid ? tn : m_valid - 1) * ld_x + 8 * lh;
#pragma unroll
      for (int st = 0; st < kSkSteps; ++st) xt[ti][st] = *(const uint4*)(xr + ks[st]);
    }
    const int n_pass = (m_valid + NT * kSkTile - 1) / (NT * kSkTile);
    for (int ps = 0; ps < n_pass; ++ps) {
      bool tok[NT];
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) tok[ti] = NT * kSkTile * ps + kSkTile * ti + li < m_valid;
      // The code words pass through an empty asm each pass, so the compiler
      // cannot hoist the (token-independent) dequantization out of the pass
      // loop, which would hold every step's fp16 operands in registers.
#pragma unroll
      for (int st = 0; st < kSkSteps; ++st)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          uint32_t lo = w[st][r][0], hi = w[st][r][1];
          asm volatile("" : "+v"(lo), "+v"(hi));
          w[st][r] = (u2s){lo, hi};
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f4s acc[NT][8];
        uint32_t zc[8];
#pragma unroll
        for (int st = 0; st < kSkSteps; ++st) {
          if (st % kSpg == 0) {
            zero_consts(zw[st / kSpg][h], zc);
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[ti][j] = (f4s){0.0f, 0.0f, 0.0f, 0.0f};
          }
          h8s bt[NT];
#pragma unroll
          for (int ti = 0; ti < NT; ++ti)
            bt[ti] = __builtin_bit_cast(h8s, (tok[ti] && live[st]) ? xt[ti][st] : make_uint4(0u, 0u, 0u, 0u));
          // byte b of the lane's 8 rows: nibble positions 2b and 2b + 1, the
          // products of every tile, before the next byte (few fragment
          // registers live)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            uint32_t al[4], ah[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t sel = (uint32_t)b | (12u << 8) | ((uint32_t)(4 + b) << 16) | (12u << 24);
              const uint32_t x2 = __builtin_amdgcn_perm(w[st][2 * p + 1][h], w[st][2 * p][h], sel);
              al[p] = pk_sub_f16(and_or(x2, 0x000F000Fu, 0x64006400u), zc[2 * b]);
              ah[p] = pk_sub_f16(and_or(x2, 0x00F000F0u, 0x64006400u), zc[2 * b + 1]);
            }
            const h8s avl = __builtin_bit_cast(h8s, make_uint4(al[0], al[1], al[2], al[3]));
            const h8s avh = __builtin_bit_cast(h8s, make_uint4(ah[0], ah[1], ah[2], ah[3]));
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
              acc[ti][2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(avl, bt[ti], acc[ti][2 * b], 0, 0, 0);
              acc[ti][2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(avh, bt[ti], acc[ti][2 * b + 1], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if ((st + 1) % kSpg == 0) {
            const uint16_t* sg = ssc + (st / kSpg) * kSkWords * 8;
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
              skinny_fold(acc[ti], sg, lh, h, ti, my, st + 1 == kSpg);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        if (h == 1 && ps + 1 < n_pass) {   // the next pass's activations, loading while this one is stored
#pragma unroll
          for (int ti = 0; ti < NT; ++ti) {
            const int tn = NT * kSkTile * (ps + 1) + kSkTile * ti + li;
            const uint16_t* xr = X + (int64_t)(tn < m_valid ? tn : m_valid - 1) * ld_x + 8 * lh;
#pragma unroll
            for (int st = 0; st < kSkSteps; ++st) xt[ti][st] = *(const uint4*)(xr + ks[st]);
          }
        }
        __syncthreads();
        // word columns of parity h of the pass's tiles: NT x 16 tokens x 16 columns
        for (int idx = tid; idx < NT * kSkTile * (kSkWords / 2); idx += kSkWaves * kWave) {
          const int ti = idx / (kSkTile * kSkWords / 2), rem = idx % (kSkTile * kSkWords / 2);
          const int tl = rem / (kSkWords / 2), q8 = 2 * (rem % (kSkWords / 2)) + h;
          store8(NT * kSkTile * ps + kSkTile * ti + tl, q8, tl + 16 * (q8 >> 3), ti);
        }
        __syncthreads();   // the slots are read before the next pass writes them
      }
    }
  }
}

// Input ranges of the few-token kernel: 512 rows each (one 128-row chunk per
// wave); their fp32 results (M x d_out each) cost 2 M / 512 bytes per weight
// and input row, against 0.5 + 2.5 / G bytes of codes, scales and zero points.
static int64_t skinny_splits(int64_t d_in) {
  return (d_in + kSkWaves * kSkChunk - 1) / (kSkWaves * kSkChunk);
}
int64_t w4a16_skinny_part_floats(int64_t M, int64_t d_out, int64_t d_in) {
  if (M < 2 || M > kSkMaxTokens) return 0;
  const int64_t s = skinny_splits(d_in);
  return s > 1 ? s * M * d_out : 0;
}
bool w4a16_uses_skinny(const void* X, int64_t M, int64_t ld_x, const void* qweight, int64_t d_out) {
  return M >= 2 && M <= kSkMaxTokens && ((uintptr_t)X & 15u) == 0 && ld_x % 8 == 0 &&
         ((uintptr_t)qweight & 7u) == 0 && (d_out / 8) % 2 == 0;
}

// ---------------------------------------------------------------------------
// Prefill: the W4A16 GEMM on the matrix cores ("AWQ architecture, in depth",
// "Kernels: why W4A16 is fast at decode": at prefill sizes the product is
// compute-bound and dequantization is extra work).  Block tile 256 tokens x
// 128 outputs, 8 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_f16), or for at
// most 128 tokens 128 x 128 with 8 waves of 64 x 32; a group's own
// accumulators and the result's fit 2 waves per SIMD.  K goes in stages of 32
// through a ring of four LDS buffers, a stage's tiles stored two stages ahead
// of its MFMAs.  The larger tile does twice the matrix-core work per
// dequantized code and per barrier (1.27x faster at 2048 tokens).  X goes to
// LDS as it is; the codes are
// dequantized on their way to LDS into exact fp16 (u - z): two K rows at a
// time, one byte permute puts the same byte of both rows side by side, one
// and-or makes 1024 + u (even nibbles) or 1024 + 16 u (odd nibbles) and one
// packed fp16 add subtracts 1024 + z (or 1024 + 16 z).  The MFMAs therefore
// accumulate exact products (u - z) x (16x for the odd-nibble outputs, whose
// scale takes the 1/16); a group of G rows accumulates alone and is added to
// the result times the fp32 scale of its column, so no fp16 rounding touches
// a dequantized weight.  16-byte K-chunks of an LDS tile row are swizzled by
// the row so that fragment reads are conflict-free.
// ---------------------------------------------------------------------------
constexpr int kQBN = 128, kQBK = 32;
constexpr int kQThreads = 512;
constexpr int kQBufs = 4;            // LDS stage buffers: stores run two stages ahead of the MFMAs
// from 9 tokens on, one 128-token tile (split over K when the tile grid is small)
// costs less than the three or more passes of the 4-token GEMV
constexpr int kGemmMinTokens = 17;

// 16-byte K-chunk kc (0..3) of an LDS tile row.  X rows are swizzled by bits
// 2-3 of the row, code rows by bits 3-4: the codes are written as 4-byte
// pairs to rows 8 m + c, and those rows must not share banks.
__device__ __forceinline__ int qoff_a(int row, int kc) { return row * kQBK + ((kc ^ ((row >> 2) & 3)) << 3); }
__device__ __forceinline__ int qoff_b(int row, int kc) { return row * kQBK + ((kc ^ ((row >> 3) & 3)) << 3); }

template <bool Y16, int BM>
__global__ __launch_bounds__(kQThreads, 1) void w4a16_gemm_kernel(
    const uint16_t* __restrict__ X, int64_t ld_x, int64_t M, int64_t d_in, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int64_t d_out, int group_size,
    void* __restrict__ Y, int64_t ld_y, int split_stages, float* __restrict__ part) {
  constexpr int WM = BM / 64, WN = 8 / WM;  // waves along tokens and outputs
  constexpr int NC = kQBN / WN / 32;         // 32-column tiles per wave (1 or 2)
  constexpr int XC = BM / 128;               // X chunks per thread and stage
  constexpr int kQDepth = BM == 128 ? 8 : 4;  // stages of loads in flight: the register ring fits 2 waves per SIMD
  __shared__ __align__(16) uint16_t sA[kQBufs][BM * kQBK];
  __shared__ __align__(16) uint16_t sB[kQBufs][kQBN * kQBK];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;  // wave tile rows 64 wm.., columns 32 NC wn..
  const int64_t n0 = (int64_t)blockIdx.x * kQBN, m0 = (int64_t)blockIdx.y * BM;
  const uint32_t n_words = (uint32_t)(d_out / 8);
  // K split z covers stages [z * split_stages, ...): a multiple of every group's stage count
  const int ks0 = (int)blockIdx.z * split_stages;
  const int nk = min((int)(d_in / kQBK) - ks0, split_stages);
  const int spg = group_size / kQBK;  // stages per quantization group
  const int64_t g0 = ks0 / spg;       // first group of the split
  const uint32_t kLoMask = 0x000F000Fu, kHiMask = 0x00F000F0u, kMagic = 0x64006400u;
  constexpr int kOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};

  // X: XC 16-byte chunks per thread, rows arow + 128 x (rows past M read row 0 and store zeros)
  const int arow = tid >> 2, akc = tid & 3;
  bool alive[XC];
  const uint16_t* xrow[XC];
#pragma unroll
  for (int x = 0; x < XC; ++x) {
    alive[x] = m0 + arow + 128 * x < M;
    xrow[x] = X + (alive[x] ? (m0 + arow + 128 * x) : 0) * ld_x + akc * 8 + (int64_t)ks0 * kQBK;
  }
  // codes: word column bm, K rows 2 bp and 2 bp + 1 of the stage; threads 0..255 expand bytes
  // 0-1 of the two words, threads 256..511 bytes 2-3 (both halves load the same words); a
  // column past d_out re-reads the last one: its outputs are never stored
  const int bm = tid & 15, bp = (tid >> 4) & 15;
  const int bh = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int64_t wcol = n0 / 8 + bm;
  const uint32_t wc = wcol < (int64_t)n_words ? (uint32_t)wcol : n_words - 1;
  const uint32_t* qw0 = qweight + (uint64_t)(2 * bp + ks0 * kQBK) * n_words + wc;
  // zero points: the symmetric layout (qzeros NULL) loads a code word and uses 7
  const bool has_z = qzeros != nullptr;
  const uint32_t* zp = has_z ? qzeros + (uint64_t)g0 * n_words + wc : qweight + wc;
  const uint32_t zstride = has_z ? n_words : 0u;
  // scales of this lane's NC output columns (32 apart, so alike in taking 1/16 for the
  // odd-nibble outputs); past d_out: column 0, unused
  int64_t my_col[NC];
  const uint16_t* sp[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    my_col[c] = n0 + wn * 32 * NC + c * 32 + (lane & 31);
    sp[c] = scales + g0 * d_out + (my_col[c] < d_out ? my_col[c] : 0);
  }
  const float sc_mul = (my_col[0] & 2) ? 0.0625f : 1.0f;

  // register ring: slot i holds the global data of stage kt with kt % kQDepth == i.  Every
  // thread issues the same loads per stage (stages past the end re-load the last one).
  uint4 ra[kQDepth][XC];
  uint32_t rwa[kQDepth], rwb[kQDepth], rz[kQDepth];
  uint16_t rs[kQDepth][NC];
  auto issue = [&](int slot, int kt) {
    const int ktc = kt < nk ? kt : nk - 1;
    const uint32_t k0 = (uint32_t)ktc * kQBK;
    const uint32_t g = (uint32_t)(ktc / spg);
#pragma unroll
    for (int x = 0; x < XC; ++x) ra[slot][x] = *(const uint4*)(xrow[x] + k0);
    rwa[slot] = qw0[k0 * n_words];
    rwb[slot] = qw0[(k0 + 1) * n_words];
    rz[slot] = zp[g * zstride];
#pragma unroll
    for (int c = 0; c < NC; ++c) rs[slot][c] = sp[c][(uint64_t)g * d_out];
  };
  auto store = [&](int slot, int buf) {
#pragma unroll
    for (int x = 0; x < XC; ++x)
      *(uint4*)&sA[buf][qoff_a(arow + 128 * x, akc)] = alive[x] ? ra[slot][x] : make_uint4(0, 0, 0, 0);
    const uint32_t zw = has_z ? rz[slot] : 0x77777777u;
    const int k2 = 2 * bp;  // the pair's first K row within the stage
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * bh + bb;
      const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
      const uint32_t pb = __builtin_amdgcn_perm(rwb[slot], rwa[slot], sel);  // bytes [rwa.b, 0, rwb.b, 0]
      const uint32_t ze = 0x64006400u + 0x00010001u * ((zw >> (8 * b)) & 0xFu);      // fp16 1024 + z, both halves
      const uint32_t zo = 0x64006400u + 0x00100010u * ((zw >> (8 * b + 4)) & 0xFu);  // fp16 1024 + 16 z
      const h2 ev = __builtin_bit_cast(h2, and_or(pb, kLoMask, kMagic)) - __builtin_bit_cast(h2, ze);
      const h2 od = __builtin_bit_cast(h2, and_or(pb, kHiMask, kMagic)) - __builtin_bit_cast(h2, zo);
      const int ne = 8 * bm + kOrder[2 * b], no = 8 * bm + kOrder[2 * b + 1];
      *(h2*)&sB[buf][qoff_b(ne, k2 >> 3) + (k2 & 7)] = ev;
      *(h2*)&sB[buf][qoff_b(no, k2 >> 3) + (k2 & 7)] = od;
    }
  };

  f32x16 acc[2][NC], accg[2][NC];  // [32-row tile][32-column tile]
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = accg[r][c][e] = 0.0f;

#pragma unroll
  for (int i = 0; i < kQDepth; ++i) issue(i, i);
  store(0, 0);
  if (nk > 1) store(1, 1);
  __syncthreads();
  // stage kt (ring slot i = kt % kQDepth, LDS buffer kt % kQBufs): loads of stage
  // kt + depth into slot i; fragment reads and MFMAs of stage kt; stage kt + 2 from its
  // slot into its buffer, whose last reads (stage kt - 2) ended before the last barrier
  int kt = 0;
  auto run_stage = [&](const int i, const bool has_next2) {
    float scv[NC];  // this stage's group scales, before the slot is reused
#pragma unroll
    for (int c = 0; c < NC; ++c) scv[c] = h2f(rs[i][c]) * sc_mul;
    issue(i, kt + kQDepth);
#pragma unroll
    for (int ks = 0; ks < kQBK / 16; ++ks) {
      const int kc = 2 * ks + (lane >> 5);
      uint4 a[2], b[NC];
#pragma unroll
      for (int r = 0; r < 2; ++r) a[r] = *(const uint4*)&sA[i % kQBufs][qoff_a(wm * 64 + r * 32 + (lane & 31), kc)];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        b[c] = *(const uint4*)&sB[i % kQBufs][qoff_b(wn * 32 * NC + c * 32 + (lane & 31), kc)];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          accg[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[r]),
                                                              __builtin_bit_cast(f16x8, b[c]), accg[r][c], 0, 0, 0);
    }
    if ((kt + 1) % spg == 0) {  // the group is complete: scale it into the result
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            acc[r][c][e] = __builtin_fmaf(accg[r][c][e], scv[c], acc[r][c][e]);
            accg[r][c][e] = 0.0f;
          }
    }
    if (has_next2) store((i + 2) % kQDepth, (i + 2) % kQBufs);
    __syncthreads();
    ++kt;
  };
  // full trips of kQDepth stages, each with two successors: no branch around the
  // ring's loads, so its registers stay put across trips and the compiler's
  // in-order waits leave the later stages in flight (kQDepth is a multiple of
  // kQBufs, so slot and buffer follow i)
  while (kt + kQDepth + 1 < nk) {  // run_stage advances kt
#pragma unroll
    for (int i = 0; i < kQDepth; ++i) run_stage(i, true);
  }
#pragma unroll
  for (int i = 0; i < kQDepth + 1; ++i) {  // the last 2..kQDepth + 1 stages
    if (kt < nk) run_stage(i % kQDepth, kt + 2 < nk);
  }
  // lane l holds rows 8 (e / 4) + 4 (l / 32) + e % 4 of column l % 32 of each 32 x 32 tile
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (my_col[c] >= d_out) continue;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + r * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= M) continue;
        if (part != nullptr) part[((int64_t)blockIdx.z * M + row) * d_out + my_col[c]] = acc[r][c][e];
        else if constexpr (Y16) ((uint16_t*)Y)[row * ld_y + my_col[c]] = f2h_bits(acc[r][c][e]);
        else ((float*)Y)[row * ld_y + my_col[c]] = acc[r][c][e];
      }
  }
}

// token tile of the GEMM: 256 rows (8 waves of 64 x 64: twice the matrix-core work per
// dequantized code of the 128-row tile, 1.27x faster at 2048 tokens) once there are more
// than 128 tokens, else 128 rows (8 waves of 64 x 32), which wastes less of the tile
static int gemm_bm(int64_t M) { return M > 128 ? 256 : 128; }

// K splits of the GEMM, so that a small tile grid still gives every compute
// unit a block (one block per CU): split boundaries fall on multiples of 128
// inputs (a group boundary at every group size); at most 8 splits and at most
// half as many as there are 128-input units.  The split partials [z][M][d_out]
// are added in split order by the reduction kernel.
static int gemm_split_stages(int64_t M, int64_t d_out, int64_t d_in) {
  const int nk = (int)(d_in / kQBK);
  const int64_t bmr = gemm_bm(M);
  const int64_t tiles = ((d_out + kQBN - 1) / kQBN) * ((M + bmr - 1) / bmr);
  const int units = (nk + 3) / 4;  // 128-input units, the last one possibly partial
  int64_t s = (256 + tiles - 1) / tiles;
  s = s < 8 ? s : 8;
  s = s < units / 2 ? s : units / 2;
  if (s <= 1) return nk;
  return (int)((units + s - 1) / s) * 4;
}

int64_t w4a16_gemm_part_floats(int64_t M, int64_t d_out, int64_t d_in) {
  if (M < kGemmMinTokens || d_in % kQBK) return 0;
  const int nk = (int)(d_in / kQBK), ss = gemm_split_stages(M, d_out, d_in);
  const int64_t n_split = (nk + ss - 1) / ss;
  return n_split > 1 ? n_split * M * d_out : 0;
}

bool w4a16_uses_gemm(const void* X, int64_t M, int64_t ld_x, int64_t d_in) {
  return M >= kGemmMinTokens && ((uintptr_t)X & 15u) == 0 && ld_x % 8 == 0 && d_in % kQBK == 0;
}

hipError_t launch_w4a16(const uint16_t* X, int64_t M, int64_t ld_x, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, int64_t d_out, int64_t d_in, int group_size, void* Y, int64_t ld_y,
                        bool y_f16, float* part, hipStream_t stream) {
  if (w4a16_uses_skinny(X, M, ld_x, qweight, d_out)) {
    const int64_t n_split = skinny_splits(d_in);
    const int n_strips = (int)((d_out / 8 + kSkWords - 1) / kSkWords);
    const unsigned g = (unsigned)(n_strips * n_split);
    float* sp = n_split > 1 ? part : nullptr;
#define AWQ_SKINNY(GG, YF, MU)                                                                          \
  w4a16_skinny_kernel<GG, YF, MU><<<g, kSkWaves * kWave, 0, stream>>>(X, ld_x, (int)M, d_in, qweight, scales, \
                                                                      qzeros, d_out, n_strips, Y, ld_y, sp)
#define AWQ_SKINNY_Y(GG, MU) \
  if (y_f16) AWQ_SKINNY(GG, true, MU); else AWQ_SKINNY(GG, false, MU)
#define AWQ_SKINNY_G(MU)                  \
  if (group_size == 128) {                \
    AWQ_SKINNY_Y(128, MU);                \
  } else if (group_size == 64) {          \
    AWQ_SKINNY_Y(64, MU);                 \
  } else {                                \
    AWQ_SKINNY_Y(32, MU);                 \
  }
    if (M <= kSkTile) {
      AWQ_SKINNY_G(false)
    } else {
      AWQ_SKINNY_G(true)
    }
#undef AWQ_SKINNY_G
#undef AWQ_SKINNY_Y
#undef AWQ_SKINNY
    if (n_split > 1) {
      const dim3 rgrid((unsigned)((d_out / 4 + kRdCols - 1) / kRdCols), (unsigned)M);
      w4a16_reduce_kernel<<<rgrid, kRdCols * kRdSplit, 0, stream>>>(part, n_split, (int)M, d_out, Y, ld_y,
                                                                    y_f16 ? 1 : 0);
    }
    return hipGetLastError();
  }
  if (w4a16_uses_gemm(X, M, ld_x, d_in)) {
    const int nk = (int)(d_in / kQBK), ss = gemm_split_stages(M, d_out, d_in);
    const int n_split = (nk + ss - 1) / ss;
    float* gp = n_split > 1 ? part : nullptr;
    const int bmr = gemm_bm(M);
    const dim3 g((unsigned)((d_out + kQBN - 1) / kQBN), (unsigned)((M + bmr - 1) / bmr), (unsigned)n_split);
    if (bmr == 256) {
      if (y_f16)
        w4a16_gemm_kernel<true, 256><<<g, kQThreads, 0, stream>>>(X, ld_x, M, d_in, qweight, scales, qzeros, d_out,
                                                                   group_size, Y, ld_y, ss, gp);
      else
        w4a16_gemm_kernel<false, 256><<<g, kQThreads, 0, stream>>>(X, ld_x, M, d_in, qweight, scales, qzeros,
                                                                    d_out, group_size, Y, ld_y, ss, gp);
    } else {
      if (y_f16)
        w4a16_gemm_kernel<true, 128><<<g, kQThreads, 0, stream>>>(X, ld_x, M, d_in, qweight, scales, qzeros, d_out,
                                                                   group_size, Y, ld_y, ss, gp);
      else
        w4a16_gemm_kernel<false, 128><<<g, kQThreads, 0, stream>>>(X, ld_x, M, d_in, qweight, scales, qzeros,
                                                                    d_out, group_size, Y, ld_y, ss, gp);
    }
    if (n_split > 1) {
      const dim3 rgrid((unsigned)((d_out / 4 + kRdCols - 1) / kRdCols), (unsigned)M);
      w4a16_reduce_kernel<<<rgrid, kRdCols * kRdSplit, 0, stream>>>(part, n_split, (int)M, d_out, Y, ld_y,
                                                                    y_f16 ? 1 : 0);
    }
    return hipGetLastError();
  }
  const int64_t n_slices = w4a16_slices(d_in);
  const dim3 grid((unsigned)w4a16_cols(d_out), (unsigned)n_slices);
  for (int64_t t0 = 0; t0 < M; t0 += 4) {
    const int mv = (int)((M - t0) < 4 ? (M - t0) : 4);
    const int mt = mv == 1 ? 1 : (mv == 2 ? 2 : 4);
    const uint16_t* Xc = X + t0 * ld_x;
    switch (mt) {
      case 1:
        w4a16_gemv_kernel<1><<<grid, kGvThreads, 0, stream>>>(Xc, ld_x, mv, d_in, qweight, scales, qzeros, d_out,
                                                              group_size, part);
        break;
      case 2:
        w4a16_gemv_kernel<2><<<grid, kGvThreads, 0, stream>>>(Xc, ld_x, mv, d_in, qweight, scales, qzeros, d_out,
                                                              group_size, part);
        break;
      default:
        w4a16_gemv_kernel<4><<<grid, kGvThreads, 0, stream>>>(Xc, ld_x, mv, d_in, qweight, scales, qzeros, d_out,
                                                              group_size, part);
        break;
    }
    void* Yc = y_f16 ? (void*)((uint16_t*)Y + t0 * ld_y) : (void*)((float*)Y + t0 * ld_y);
    const dim3 rgrid((unsigned)((d_out / 4 + kRdCols - 1) / kRdCols), (unsigned)mv);
    w4a16_reduce_kernel<<<rgrid, kRdCols * kRdSplit, 0, stream>>>(part, n_slices, mt, d_out, Yc, ld_y,
                                                                  y_f16 ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace awq
