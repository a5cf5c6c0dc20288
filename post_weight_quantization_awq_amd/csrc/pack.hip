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
// that falls back to the IEEE division near half-integers.
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

// nibble that holds row r of an 8-row run: order = {0,2,4,6,1,3,5,7} => inverse {0,4,1,5,2,6,3,7}
__device__ __forceinline__ constexpr int nibble_of_row(int r) {
  return (r & 1) ? 4 + (r >> 1) : (r >> 1);
}

template <int G>
struct PackShape {
  static constexpr int LPG = G / 8;              // lanes per group row
  static constexpr int UNITS = 64 / LPG;         // 8-row units per wave
  static constexpr int ROWS_W = UNITS * 8;       // rows per wave
  static constexpr int ROWS_B = ROWS_W * (kPackThreads / 64);
  static constexpr int MW = ROWS_B / 8;          // words per input column per block
};

template <int G>
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
  if (s != nullptr) {
    const float4 a = *(const float4*)(s + col0);
    const float4 b = *(const float4*)(s + col0 + 4);
    sv[0] = a.x; sv[1] = a.y; sv[2] = a.z; sv[3] = a.w;
    sv[4] = b.x; sv[5] = b.y; sv[6] = b.z; sv[7] = b.w;
  }
  uint32_t words[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) words[j] = 0u;
  uint32_t sbits[4];

#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float v[8];
    if (valid) {
      const uint4 u = ld_nt(W + (row0 + r) * d_in + col0);
      unpack8_f16(u, v);
      if (s != nullptr) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * sv[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
    m = group_max<SH::LPG>(m);
    const float a = (clip != nullptr && valid) ? clip[row0 + r] * m : m;
    const float step = div7(a);
    const float inv = __builtin_amdgcn_rcpf(step);
    const int sh = 4 * nibble_of_row(r);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float n = step > 0.0f ? code_exact(v[j], step, inv) : 0.0f;
      n = __builtin_fminf(__builtin_fmaxf(n, -7.0f), 7.0f);
      words[j] |= (uint32_t)((int)n + 7) << sh;
    }
    const uint32_t hb = f2h_bits(step);
    if (r & 1) sbits[r >> 1] |= hb << 16;
    else sbits[r >> 1] = hb;
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) wt[lg * 8 + j][m_local] = words[j];
  if (valid && lg == 0) {
    *(uint4*)(scales + gcol * d_out + row0) = make_uint4(sbits[0], sbits[1], sbits[2], sbits[3]);
    if (qzeros != nullptr) qzeros[gcol * (d_out / 8) + row0 / 8] = 0x77777777;
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

hipError_t launch_quantize_pack(const uint16_t* W, int64_t d_out, int64_t d_in, int group_size,
                                const float* s, const float* clip, int32_t* qweight,
                                uint16_t* scales, int32_t* qzeros, hipStream_t stream) {
  switch (group_size) {
    case 32:
      quantize_pack_kernel<32><<<(unsigned)pack_blocks<32>(d_out, d_in), kPackThreads, 0, stream>>>(
          W, d_out, d_in, s, clip, qweight, scales, qzeros);
      break;
    case 64:
      quantize_pack_kernel<64><<<(unsigned)pack_blocks<64>(d_out, d_in), kPackThreads, 0, stream>>>(
          W, d_out, d_in, s, clip, qweight, scales, qzeros);
      break;
    default:
      quantize_pack_kernel<128><<<(unsigned)pack_blocks<128>(d_out, d_in), kPackThreads, 0, stream>>>(
          W, d_out, d_in, s, clip, qweight, scales, qzeros);
      break;
  }
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

hipError_t launch_unpack_dequant(const int32_t* qweight, const uint16_t* scales,
                                 const int32_t* qzeros, int64_t d_out, int64_t d_in, int group_size,
                                 const float* s, void* out, bool out_f16, hipStream_t stream) {
  const int64_t n = d_in * (d_out / 8);
  unpack_dequant_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      qweight, scales, qzeros, d_out, d_in, group_size, s, out, out_f16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace awq
