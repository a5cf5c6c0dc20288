// Quantize + pack into the AutoAWQ GEMM layout, and the inverse.
// "From-Scratch AWQ INT4 Quantization on Qwen3-8B": section "Group-wise
// symmetric INT4" (step = max|group| / 7, q = round(w / step).clamp(-7, 7),
// one fp16 scale per group), section "AutoAWQ / HF-AWQ GEMM on-disk format"
// (unsigned codes, 8 per int32, pack order [0,2,4,6,1,3,5,7]) and exporter
// step 4 (zero = 7, u = q + 7, (u - zero) * scale reproduces q * scale).
// "Weight-Only Quantization: GPTQ and AWQ", section 6-9: scales [in/G, out]
// fp16, zeros [in/G, out/8] int32.
//
// Codes are bit-exact with IEEE fp32: the step is RN(a / 7) (exact divide by 7
// sequence), the code is rint(RN(v / step)) through a reciprocal fast path
// that falls back to the IEEE division near half-integers.  Unclipped, |v| is
// at most the group maximum, so |rint(v / step)| <= 7 needs no clamp.
//
// ASYM ("AWQ architecture, in depth": a 4-bit zero point per group and output
// channel, step about range / 15): range [min(0, min v), max(0, max v)] (both
// ends times the clip ratio), step RN(range / 15) (exact divide by 15), zero
// point z = clamp(rint(RN(-min / step)), 0, 15) by the IEEE division (once
// per row), code u = clamp(rint(RN(v / step)) + z, 0, 15); qzeros carry the
// eight rows' z in the qweight nibble order.
//
// HBM-bound: 2 bytes read and ~0.53 bytes written per weight.  A lane owns an
// 8 x 8 tile (8 consecutive output rows, 8 consecutive inputs): its 8 rows at
// one input column form exactly one qweight word, so packing happens in
// registers; the words of a block are transposed through LDS so that each
// qweight row (fixed input column) is written as one contiguous run.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kPackThreads = 512;  // 8 waves

template <int G>
struct PackShape {
  static constexpr int LPG = G / 8;              // lanes per group row
  static constexpr int UNITS = 64 / LPG;         // 8-row units per wave
  static constexpr int ROWS_W = UNITS * 8;       // rows per wave
  static constexpr int ROWS_B = ROWS_W * (kPackThreads / 64);
  static constexpr int MW = ROWS_B / 8;          // words per input column per block
};

// Per element: the scaled value straight from the fp16 half (mixed-precision
// fma), max (half a max3), v * rcp(step), rint, r0 - rint(r0) into a running
// max (half a max3), and one exact fp32 fma into the word (~5.5 VALU ops).
// Codes accumulate as small signed integers in fp32, even rows into the low
// 16-bit half of the word and odd rows into the high half (the pack order puts
// rows 0, 2, 4, 6 in nibbles 0-3 and rows 1, 3, 5, 7 in nibbles 4-7):
// sum_k q * 16^k is an integer of magnitude <= 7 * 0x1111, exact in fp32, and
// adding 0x7777 gives sum_k (q + 7) * 16^k since every q + 7 lies in [0, 14].
// A row whose fast codes might differ from rint(RN(v / step)) (some
// |r0 - rint r0| within 2^-15 of 1/2), or whose step is not a positive finite
// number, recomputes its 8 codes with the IEEE division.  The bound on
// |r0 - v/step| (rcp within 1 ulp, one rounding) is below 8e-6 for
// |v/step| < 32; unclipped |v/step| <= 7, and with clipping a larger quotient
// can only mis-round to a code that the clamp maps to +-7 either way for
// |v/step| >= 32 (ratios >= 7/32).  Weights are expected to be finite.
template <int G, bool HAS_S, bool HAS_CLIP, bool ASYM>
__global__ __launch_bounds__(kPackThreads) void quantize_pack_kernel(
    const uint16_t* __restrict__ W, int64_t d_out, int64_t d_in, const float* __restrict__ s,
    const float* __restrict__ clip, int32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
    int32_t* __restrict__ qzeros) {
  using SH = PackShape<G>;
  __shared__ uint32_t wt[G][SH::MW + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int lg = lane % SH::LPG, unit = lane / SH::LPG;
  const int64_t n_gcol = d_in / G;
  const int64_t gcol = blockIdx.x % n_gcol;
  const int64_t rblk = blockIdx.x / n_gcol;
  const int m_local = wv * SH::UNITS + unit;
  const int64_t row0 = rblk * SH::ROWS_B + (int64_t)m_local * 8;
  const int64_t col0 = gcol * G + lg * 8;
  const bool valid = row0 < d_out;  // d_out % 8 == 0: all 8 rows or none

  float sv[8];
  if constexpr (HAS_S) {
    const float4 a = *(const float4*)(s + col0);
    const float4 b = *(const float4*)(s + col0 + 4);
    sv[0] = a.x; sv[1] = a.y; sv[2] = a.z; sv[3] = a.w;
    sv[4] = b.x; sv[5] = b.y; sv[6] = b.z; sv[7] = b.w;
  }
  // Unconditional loads (a lane past d_out reads rows 0..7 and stores
  // nothing), so the wait before row r covers only rows 0..r.
  const int64_t lrow = valid ? row0 : 0;
  float cl[8];
  if constexpr (HAS_CLIP) {
#pragma unroll
    for (int r = 0; r < 8; ++r) cl[r] = clip[lrow + r];
  }
  uint4 raw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) raw[r] = ld_nt(W + (lrow + r) * d_in + col0);

  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  float lo[8], hi[8];  // codes of even / odd rows as exact fp32 sums of q * 16^k
#pragma unroll
  for (int j = 0; j < 8; ++j) lo[j] = hi[j] = 0.0f;
  uint32_t sbits[4];
  uint32_t zword = 0;  // ASYM: zero points of the 8 rows, nibble order of the codes

#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const h8 hv = __builtin_bit_cast(h8, raw[r]);
    float v[8];
    float m = 0.0f, mn = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = HAS_S ? __builtin_fmaf((float)hv[j], sv[j], 0.0f) : (float)hv[j];
      if constexpr (ASYM) {
        m = __builtin_fmaxf(m, v[j]);
        mn = __builtin_fmaxf(mn, -v[j]);
      } else {
        m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
      }
    }
    m = group_max_nonneg<SH::LPG>(m);
    float a = m, an = 0.0f;
    if constexpr (ASYM) an = group_max_nonneg<SH::LPG>(mn);
    if constexpr (HAS_CLIP) {
      a = cl[r] * a;
      an = cl[r] * an;
    }
    const float step = ASYM ? div15(a + an) : div7(a);
    const float inv = __builtin_amdgcn_rcpf(step);
    float n[8];
    float dev = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float r0 = v[j] * inv;
      n[j] = __builtin_rintf(r0);
      dev = __builtin_fmaxf(dev, __builtin_fabsf(r0 - n[j]));
    }
    if (!(dev < 0.5f - 0x1p-15f) || !(step > 0.0f && step < __builtin_inff())) {
      // rare: exact codes for this lane's 8 elements of row r
#pragma unroll
      for (int j = 0; j < 8; ++j) n[j] = step > 0.0f ? __builtin_rintf(v[j] / step) : 0.0f;
    }
    constexpr float kWeight[4] = {1.0f, 16.0f, 256.0f, 4096.0f};
    const float wgt = kWeight[r >> 1];
    float zf = 0.0f;
    if constexpr (ASYM) {
      zf = step > 0.0f ? __builtin_amdgcn_fmed3f(__builtin_rintf(an / step), 0.0f, (float)kUMax) : 0.0f;
      zword |= (uint32_t)zf << (4 * ((r & 1) ? 4 + (r >> 1) : (r >> 1)));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float q = n[j];
      if constexpr (ASYM) q = __builtin_amdgcn_fmed3f(q, -zf, (float)kUMax - zf) + zf;  // u in [0, 15]
      else if constexpr (HAS_CLIP) q = __builtin_amdgcn_fmed3f(q, -7.0f, 7.0f);
      if (r & 1) hi[j] = __builtin_fmaf(q, wgt, hi[j]);
      else lo[j] = __builtin_fmaf(q, wgt, lo[j]);
    }
    const uint32_t hb = f2h_bits(step);
    if (r & 1) sbits[r >> 1] |= hb << 16;
    else sbits[r >> 1] = hb;
    // keep rows apart: row r then waits only for its own load, so the
    // arithmetic of early rows overlaps the loads of later ones
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    constexpr int32_t kOff = ASYM ? 0 : 0x7777;  // symmetric codes are q + 7
    const uint32_t wlo = (uint32_t)((int32_t)lo[j] + kOff), whi = (uint32_t)((int32_t)hi[j] + kOff);
    wt[lg * 8 + j][m_local] = (whi << 16) | wlo;
  }
  if (valid && lg == 0) {
    *(uint4*)(scales + gcol * d_out + row0) = make_uint4(sbits[0], sbits[1], sbits[2], sbits[3]);
    if (qzeros != nullptr) qzeros[gcol * (d_out / 8) + row0 / 8] = ASYM ? (int32_t)zword : 0x77777777;
  }
  __syncthreads();
  const int64_t words_per_col = d_out / 8;
  const int64_t m_base = rblk * SH::MW;
  for (int idx = tid; idx < G * SH::MW; idx += kPackThreads) {
    const int c = idx / SH::MW, mm = idx % SH::MW;
    if (m_base + mm < words_per_col)
      qweight[(gcol * G + c) * words_per_col + m_base + mm] = (int32_t)wt[c][mm];
  }
}

template <int G>
static int64_t pack_blocks(int64_t d_out, int64_t d_in) {
  return (d_in / G) * ((d_out + PackShape<G>::ROWS_B - 1) / PackShape<G>::ROWS_B);
}

template <int G, bool ASYM>
static void launch_pack_g(const uint16_t* W, int64_t d_out, int64_t d_in, const float* s, const float* clip,
                          int32_t* qweight, uint16_t* scales, int32_t* qzeros, hipStream_t stream) {
  const unsigned nb = (unsigned)pack_blocks<G>(d_out, d_in);
  if (s != nullptr && clip != nullptr)
    quantize_pack_kernel<G, true, true, ASYM><<<nb, kPackThreads, 0, stream>>>(W, d_out, d_in, s, clip, qweight, scales, qzeros);
  else if (s != nullptr)
    quantize_pack_kernel<G, true, false, ASYM><<<nb, kPackThreads, 0, stream>>>(W, d_out, d_in, s, clip, qweight, scales, qzeros);
  else if (clip != nullptr)
    quantize_pack_kernel<G, false, true, ASYM><<<nb, kPackThreads, 0, stream>>>(W, d_out, d_in, s, clip, qweight, scales, qzeros);
  else
    quantize_pack_kernel<G, false, false, ASYM><<<nb, kPackThreads, 0, stream>>>(W, d_out, d_in, s, clip, qweight, scales, qzeros);
}

hipError_t launch_quantize_pack(const uint16_t* W, int64_t d_out, int64_t d_in, int group_size, bool asym,
                                const float* s, const float* clip, int32_t* qweight,
                                uint16_t* scales, int32_t* qzeros, hipStream_t stream) {
#define AWQ_PK(G) \
  if (asym) launch_pack_g<G, true>(W, d_out, d_in, s, clip, qweight, scales, qzeros, stream); \
  else launch_pack_g<G, false>(W, d_out, d_in, s, clip, qweight, scales, qzeros, stream);
  switch (group_size) {
    case 32: AWQ_PK(32) break;
    case 64: AWQ_PK(64) break;
    default: AWQ_PK(128) break;
  }
#undef AWQ_PK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// unpack + dequantize (verification): thread per (input column, word); the
// consecutive threads of a wave take consecutive input columns so the fp32 /
// fp16 output rows are written coalesced.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpack_dequant_kernel(
    const int32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const int32_t* __restrict__ qzeros, int64_t d_out, int64_t d_in, int group_size,
    const float* __restrict__ s, void* __restrict__ out, int out_f16) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t words_per_col = d_out / 8;
  if (idx >= d_in * words_per_col) return;
  const int64_t i = idx % d_in;
  const int64_t m = idx / d_in;
  const int64_t g = i / group_size;
  const uint32_t word = (uint32_t)qweight[i * words_per_col + m];
  const uint32_t zw = qzeros != nullptr ? (uint32_t)qzeros[g * words_per_col + m] : 0x77777777u;
  const float sdiv = s != nullptr ? s[i] : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = 8 * m + ((j < 4) ? 2 * j : 2 * (j - 4) + 1);
    const int u = (int)((word >> (4 * j)) & 0xFu);
    const int z = (int)((zw >> (4 * j)) & 0xFu);
    float val = (float)(u - z) * h2f(scales[g * d_out + row]);
    if (s != nullptr) val = val / sdiv;
    if (out_f16) ((uint16_t*)out)[row * d_in + i] = f2h_bits(val);
    else ((float*)out)[row * d_in + i] = val;
  }
}

// Tiled form for d_out % 32 == 0 and 16-byte aligned qweight / qzeros: a block
// takes 64 input rows x 16 words (128 outputs).  Thread t loads words
// 4 (t % 4) .. + 3 of input row t / 4 as one 16-byte load (a wave reads 16
// rows x 64 contiguous bytes), decodes its 32 values with the same arithmetic
// as above into an LDS tile [128 outputs][64 inputs], and after a barrier the
// block writes each output row's 64 inputs as contiguous 16-byte stores.
constexpr int kUnpI = 64, kUnpW = 16;
template <bool F16>
__global__ __launch_bounds__(256) void unpack_dequant_tile_kernel(
    const int32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const int32_t* __restrict__ qzeros, int64_t d_out, int64_t d_in, int group_size,
    const float* __restrict__ s, void* __restrict__ out) {
  typedef typename std::conditional<F16, uint16_t, float>::type T;
  constexpr int kPad = 16 / sizeof(T);  // row padding (one 16-byte chunk) against bank conflicts
  __shared__ __align__(16) T tile[kUnpW * 8][kUnpI + kPad];
  const int64_t wpc = d_out / 8;
  const int64_t i0 = (int64_t)blockIdx.x * kUnpI, m0 = (int64_t)blockIdx.y * kUnpW;
  const int t = threadIdx.x, il = t >> 2, wq = t & 3;
  const int64_t i = i0 + il, m = m0 + 4 * wq;
  if (i < d_in && m < wpc) {
    const int64_t g = i / group_size;
    const uint4 wv4 = *(const uint4*)(qweight + i * wpc + m);
    const uint4 zv4 = qzeros != nullptr ? *(const uint4*)(qzeros + g * wpc + m)
                                        : make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
    const float sdiv = s != nullptr ? s[i] : 1.0f;
    const uint32_t wv[4] = {wv4.x, wv4.y, wv4.z, wv4.w}, zv[4] = {zv4.x, zv4.y, zv4.z, zv4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ol = 8 * (4 * wq + q) + ((j < 4) ? 2 * j : 2 * (j - 4) + 1);
        const int u = (int)((wv[q] >> (4 * j)) & 0xFu);
        const int z = (int)((zv[q] >> (4 * j)) & 0xFu);
        float val = (float)(u - z) * h2f(scales[g * d_out + 8 * m0 + ol]);
        if (s != nullptr) val = val / sdiv;
        if constexpr (F16) tile[ol][il] = f2h_bits(val);
        else tile[ol][il] = val;
      }
    }
  }
  __syncthreads();
  constexpr int kChunks = kUnpI * (int)sizeof(T) / 16;  // 16-byte chunks per output row of the tile
  constexpr int kPer = 16 / (int)sizeof(T);             // values per chunk
  for (int c = t; c < kUnpW * 8 * kChunks; c += 256) {
    const int ol = c / kChunks, ch = c % kChunks;
    const int64_t o = 8 * m0 + ol, ii = i0 + (int64_t)ch * kPer;
    if (o >= d_out || ii >= d_in) continue;  // d_in is a multiple of 8, so a chunk is whole or out
    *(uint4*)((T*)out + o * d_in + ii) = *(const uint4*)&tile[ol][ch * kPer];
  }
}

hipError_t launch_unpack_dequant(const int32_t* qweight, const uint16_t* scales,
                                 const int32_t* qzeros, int64_t d_out, int64_t d_in, int group_size,
                                 const float* s, void* out, bool out_f16, hipStream_t stream) {
  if (d_out % 32 == 0 && d_in % 8 == 0 && (uintptr_t)qweight % 16 == 0 && (uintptr_t)qzeros % 16 == 0 &&
      (uintptr_t)out % 16 == 0) {
    const dim3 grid((unsigned)((d_in + kUnpI - 1) / kUnpI), (unsigned)((d_out / 8 + kUnpW - 1) / kUnpW));
    if (out_f16)
      unpack_dequant_tile_kernel<true><<<grid, 256, 0, stream>>>(qweight, scales, qzeros, d_out, d_in, group_size,
                                                                 s, out);
    else
      unpack_dequant_tile_kernel<false><<<grid, 256, 0, stream>>>(qweight, scales, qzeros, d_out, d_in, group_size,
                                                                  s, out);
    return hipGetLastError();
  }
  const int64_t n = d_in * (d_out / 8);
  unpack_dequant_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      qweight, scales, qzeros, d_out, d_in, group_size, s, out, out_f16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace awq
