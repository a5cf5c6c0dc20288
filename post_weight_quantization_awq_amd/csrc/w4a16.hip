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

  // activations of the slice first (issued before the codes)
  uint16_t xr[kXPer];
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int idx = q * kGvThreads + tid;
    const int t = idx / kGvSlice, c = idx % kGvSlice;
    const int64_t row = k0 + c;
    xr[q] = (idx < MT * kGvSlice && t < m_valid && row < d_in) ? X[t * ld_x + row] : (uint16_t)0;
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
    if (idx < MT * kGvSlice) xs[idx / kGvSlice][idx % kGvSlice] = h2f(xr[q]);
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

hipError_t launch_w4a16(const uint16_t* X, int64_t M, int64_t ld_x, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, int64_t d_out, int64_t d_in, int group_size, void* Y, int64_t ld_y,
                        bool y_f16, float* part, hipStream_t stream) {
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
