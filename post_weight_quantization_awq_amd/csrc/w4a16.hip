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
// lane: a wave reads 256 contiguous bytes of a qweight row) and 128 input
// rows, 32 per wave; a wave's rows lie in one quantization group (G >= 32),
// so the zero point factors out of its sum:
//   sum_i x_i (u_i - z) scale = scale * (sum_i x_i u_i - z * sum_i x_i).
// Codes become fp32 by byte conversions (nibbles masked into bytes), products
// u * x are exact in fp32 and accumulate in fp32.  The four waves' results
// are added in LDS in a fixed order and written as one fp32 partial per
// (row slice, token, output); a second launch adds the partials of the row
// slices in a fixed order and rounds once to the output type.  Tokens are
// handled MT (1, 2 or 4) at a time; the weights of a launch are read once
// per token chunk.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = kGvThreads / kWave;
constexpr int kGvRows = 32;                     // input rows per wave
constexpr int kGvSlice = kGvRows * kGvWaves;    // input rows per block
constexpr int kGvCols = kWave * 8;              // outputs per block

int64_t w4a16_slices(int64_t d_in) { return (d_in + kGvSlice - 1) / kGvSlice; }

template <int MT>
__global__ __launch_bounds__(kGvThreads) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ X, int64_t ld_x, int m_valid, int64_t d_in, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int64_t d_out, int group_size,
    float* __restrict__ part) {
  __shared__ __align__(16) _Float16 xs[MT][kGvSlice];
  __shared__ float red[kGvWaves][MT][kGvCols];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n_words = d_out / 8;
  const int64_t m = (int64_t)blockIdx.x * kWave + lane;  // packed word column of this lane
  const bool live = m < n_words;
  const int64_t mm = live ? m : n_words - 1;
  const int64_t k0 = (int64_t)blockIdx.y * kGvSlice;
  const int64_t r0 = k0 + (int64_t)wv * kGvRows;

  // codes first: 32 rows of this lane's word (rows past d_in re-read the last
  // row; their activations are staged as zeros)
  uint32_t w[kGvRows];
#pragma unroll
  for (int r = 0; r < kGvRows; ++r) {
    const int64_t row = min(r0 + r, d_in - 1);
    w[r] = __builtin_nontemporal_load(qweight + row * n_words + mm);
  }
  const int64_t g = min(r0, d_in - 1) / group_size;
  const uint4 sraw = *(const uint4*)(scales + g * d_out + 8 * mm);
  const uint32_t zw = qzeros != nullptr ? qzeros[g * n_words + mm] : 0x77777777u;

  for (int idx = tid; idx < MT * kGvSlice; idx += kGvThreads) {
    const int t = idx / kGvSlice, c = idx % kGvSlice;
    const int64_t row = k0 + c;
    xs[t][c] = (t < m_valid && row < d_in) ? __builtin_bit_cast(_Float16, X[t * ld_x + row]) : (_Float16)0.0f;
  }
  __syncthreads();

  float acc[MT][8], sx[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    sx[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = 0.0f;
  }
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int r8 = 0; r8 < kGvRows; r8 += 8) {
    float xv[MT][8];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const h8 hx = *(const h8*)&xs[t][wv * kGvRows + r8];  // the same address on every lane: a broadcast
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[t][e] = (float)hx[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = w[r8 + e] & 0x0F0F0F0Fu, hi = (w[r8 + e] >> 4) & 0x0F0F0F0Fu;
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
  // the four waves in a fixed order; 4 outputs per thread and store
  const int64_t o_base = (int64_t)blockIdx.x * kGvCols;
  for (int idx = tid; idx < MT * (kGvCols / 4); idx += kGvThreads) {
    const int t = idx / (kGvCols / 4), c4 = (idx % (kGvCols / 4)) * 4;
    if (t >= m_valid || o_base + c4 >= d_out) continue;
    float4 v;
    v.x = ((red[0][t][c4] + red[1][t][c4]) + red[2][t][c4]) + red[3][t][c4];
    v.y = ((red[0][t][c4 + 1] + red[1][t][c4 + 1]) + red[2][t][c4 + 1]) + red[3][t][c4 + 1];
    v.z = ((red[0][t][c4 + 2] + red[1][t][c4 + 2]) + red[2][t][c4 + 2]) + red[3][t][c4 + 2];
    v.w = ((red[0][t][c4 + 3] + red[1][t][c4 + 3]) + red[2][t][c4 + 3]) + red[3][t][c4 + 3];
    *(float4*)(part + ((int64_t)blockIdx.y * MT + t) * d_out + o_base + c4) = v;
  }
}

// Y[t, o] = sum over the row slices (in order) of part[slice, t, o], rounded
// once to fp16 or kept in fp32; 4 outputs per thread.
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float* __restrict__ part, int64_t n_slices, int mt,
                                                           int m_valid, int64_t d_out, void* __restrict__ Y,
                                                           int64_t ld_y, int y_f16) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_t = d_out / 4;
  if (idx >= (int64_t)m_valid * per_t) return;
  const int64_t t = idx / per_t, o = (idx % per_t) * 4;
  float4 s = *(const float4*)(part + t * d_out + o);
  for (int64_t k = 1; k < n_slices; ++k) {
    const float4 v = *(const float4*)(part + (k * mt + t) * d_out + o);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  if (y_f16) {
    uint2 h;
    h.x = (uint32_t)f2h_bits(s.x) | ((uint32_t)f2h_bits(s.y) << 16);
    h.y = (uint32_t)f2h_bits(s.z) | ((uint32_t)f2h_bits(s.w) << 16);
    *(uint2*)((uint16_t*)Y + t * ld_y + o) = h;
  } else {
    *(float4*)((float*)Y + t * ld_y + o) = s;
  }
}

hipError_t launch_w4a16(const uint16_t* X, int64_t M, int64_t ld_x, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, int64_t d_out, int64_t d_in, int group_size, void* Y, int64_t ld_y,
                        bool y_f16, float* part, hipStream_t stream) {
  const int64_t n_slices = w4a16_slices(d_in);
  const dim3 grid((unsigned)((d_out / 8 + kWave - 1) / kWave), (unsigned)n_slices);
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
    const int64_t n = (int64_t)mv * (d_out / 4);
    void* Yc = y_f16 ? (void*)((uint16_t*)Y + t0 * ld_y) : (void*)((float*)Y + t0 * ld_y);
    w4a16_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(part, n_slices, mt, mv, d_out, Yc, ld_y,
                                                                         y_f16 ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace awq
