// Weight-score scale search: for every candidate scale s_k, the activation-
// weighted reconstruction error of the group-wise INT4 fake quantization of
// W*s_k.  "From-Scratch AWQ INT4 Quantization on Qwen3-8B", sections "AWQ
// scaling" (error ||(W - Q(W s)/s) diag(x)||^2, grid search over alpha) and
// "Group-wise symmetric INT4" (step = max|group| / 7, round, clamp to [-7, 7]).
//
// The pages re-quantize all of W once per grid point.  Here every block loads
// its tile of W once into registers and evaluates all n_grid candidates on it,
// so HBM is read once per search and the kernel is bound by VALU issue:
//   per element and candidate: v = w*s (mul), group max (max3, half an op),
//   r = v * (1/step) (mul), rint (rndne), d = v - q*step (fma), acc += d*d (fma).
// The activation weight is factored out of the element loop: in the scaled
// domain (w - q*step/s) * x = (v - q*step) * (x/s), so each lane accumulates
// d^2 per column over its rows and weights the column sums by (x/s)^2 once.
//
// Tile: one quantization group column (G inputs) by 32*R rows (G = 128); each
// lane holds 16 consecutive inputs of R rows; the G/16 lanes of a row combine
// their maxima with DPP row permutes.  The candidate scales and (x/s)^2 of the
// block's columns are staged in LDS.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kSearchThreads = 256;
constexpr int kSearchR = 4;  // rows per lane

template <int G>
constexpr int search_rows_per_block() { return (kSearchThreads / (G / 16)) * kSearchR; }

template <int G, int R>
__global__ __launch_bounds__(kSearchThreads) void search_weight_kernel(
    const WParts P, int64_t d_out, int64_t d_in, int n_grid, const float* __restrict__ S,
    const float* __restrict__ C2, float* __restrict__ partials) {
  constexpr int LPG = G / 16;                  // lanes per group row
  constexpr int RS = kSearchThreads / LPG;     // row slots per block
  constexpr int RB = RS * R;                   // rows per block
  extern __shared__ float lds[];               // s [n_grid][G], then (x/s)^2 [n_grid][G]
  float* s_l = lds;
  float* c_l = lds + n_grid * G;
  __shared__ float red[kMaxGrid][4];

  const int64_t n_gcol = d_in / G;
  const int64_t gcol = blockIdx.x % n_gcol;
  const int64_t rblk = blockIdx.x / n_gcol;
  const int64_t c0 = gcol * G;
  const int tid = threadIdx.x;

  for (int idx = tid; idx < n_grid * (G / 4); idx += kSearchThreads) {
    const int k = idx / (G / 4), j = idx % (G / 4);
    ((float4*)s_l)[idx] = *(const float4*)(S + (int64_t)k * d_in + c0 + 4 * j);
    ((float4*)c_l)[idx] = *(const float4*)(C2 + (int64_t)k * d_in + c0 + 4 * j);
  }

  const int lg = tid % LPG;
  const int slot = tid / LPG;
  const int cc = lg * 16;
  float w[R][16];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = rblk * RB + slot + (int64_t)RS * r;
    if (row < d_out) {
      const uint4* p = (const uint4*)(row_ptr(P, row, d_in) + c0 + cc);
      const uint4 a = ld_nt(p);
      const uint4 b = ld_nt(p + 1);
      unpack8_f16(a, w[r]);
      unpack8_f16(b, w[r] + 8);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) w[r][j] = 0.0f;
    }
  }
  __syncthreads();

  for (int k = 0; k < n_grid; ++k) {
    float s[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 t = ((const float4*)(s_l + k * G + cc))[j];
      s[4 * j] = t.x; s[4 * j + 1] = t.y; s[4 * j + 2] = t.z; s[4 * j + 3] = t.w;
    }
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[16];
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = w[r][j] * s[j];
        m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
      }
      m = group_max<LPG>(m);
      const float step = div7(m);
      const float inv = m > 0.0f ? __builtin_amdgcn_rcpf(step) : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float q = __builtin_rintf(v[j] * inv);
        const float d = __builtin_fmaf(-step, q, v[j]);
        acc[j] = __builtin_fmaf(d, d, acc[j]);
      }
    }
    float e = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 t = ((const float4*)(c_l + k * G + cc))[j];
      e = __builtin_fmaf(t.x, acc[4 * j], e);
      e = __builtin_fmaf(t.y, acc[4 * j + 1], e);
      e = __builtin_fmaf(t.z, acc[4 * j + 2], e);
      e = __builtin_fmaf(t.w, acc[4 * j + 3], e);
    }
    e = wave_sum(e);
    if ((tid & 63) == 0) red[k][tid >> 6] = e;
  }
  __syncthreads();
  if (tid < n_grid)  // candidate-major: partials[k * n_blocks + block]
    partials[(int64_t)tid * gridDim.x + blockIdx.x] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
}

int64_t search_weight_blocks(int group_size, int64_t d_out, int64_t d_in) {
  int64_t rb = 0;
  switch (group_size) {
    case 32: rb = search_rows_per_block<32>(); break;
    case 64: rb = search_rows_per_block<64>(); break;
    default: rb = search_rows_per_block<128>(); break;
  }
  return (d_in / group_size) * ((d_out + rb - 1) / rb);
}

hipError_t launch_search_weight(int group_size, const WParts& parts, int64_t d_out, int64_t d_in,
                                int n_grid, const float* S, const float* C2, float* partials,
                                hipStream_t stream) {
  const int64_t nb = search_weight_blocks(group_size, d_out, d_in);
  const size_t shm = (size_t)2 * n_grid * group_size * sizeof(float);
  switch (group_size) {
    case 32:
      search_weight_kernel<32, kSearchR><<<(unsigned)nb, kSearchThreads, shm, stream>>>(
          parts, d_out, d_in, n_grid, S, C2, partials);
      break;
    case 64:
      search_weight_kernel<64, kSearchR><<<(unsigned)nb, kSearchThreads, shm, stream>>>(
          parts, d_out, d_in, n_grid, S, C2, partials);
      break;
    default:
      search_weight_kernel<128, kSearchR><<<(unsigned)nb, kSearchThreads, shm, stream>>>(
          parts, d_out, d_in, n_grid, S, C2, partials);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection ("AWQ architecture, in depth", "The scale search as code": keep the
// candidate when err < best, i.e. the first minimum).  One block per candidate
// sums its partials in a fixed order in fp64; one block then picks the first
// minimum and copies the winner's scale row.
// ---------------------------------------------------------------------------
constexpr int kRedThreads = 256;

__global__ __launch_bounds__(kRedThreads) void reduce_cand_kernel(const float* __restrict__ partials,
                                                                 int64_t n_blocks, int64_t stride_b,
                                                                 int64_t stride_c, double scale,
                                                                 const double* __restrict__ cand_scale,
                                                                 double* __restrict__ tot) {
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const float* p = partials + (int64_t)c * stride_c;
  double acc = 0.0;
  for (int64_t b = tid; b < n_blocks; b += kRedThreads) acc += (double)p[b * stride_b];
  __shared__ double red[kRedThreads];
  red[tid] = acc;
  __syncthreads();
  for (int w = kRedThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) tot[c] = red[0] * scale * (cand_scale != nullptr ? cand_scale[c] : 1.0);
}

__global__ __launch_bounds__(kRedThreads) void argmin_kernel(const double* __restrict__ tot, int n_cand,
                                                            float* __restrict__ err, int32_t* __restrict__ best_idx,
                                                            const float* __restrict__ S, int64_t d_in,
                                                            float* __restrict__ best_s) {
  __shared__ int best_sh;
  if (threadIdx.x == 0) {
    int b = 0;
    double be = tot[0];
    for (int c = 0; c < n_cand; ++c) {
      err[c] = (float)tot[c];
      if (tot[c] < be) { be = tot[c]; b = c; }
    }
    best_idx[0] = b;
    best_sh = b;
  }
  __syncthreads();
  if (S != nullptr) {
    const float* src = S + (int64_t)best_sh * d_in;
    for (int64_t i = threadIdx.x; i < d_in; i += kRedThreads) best_s[i] = src[i];
  }
}

hipError_t launch_argmin(const double* tot, int n_cand, float* err, int32_t* best_idx, const float* S, int64_t d_in,
                         float* best_s, hipStream_t stream) {
  argmin_kernel<<<1, kRedThreads, 0, stream>>>(tot, n_cand, err, best_idx, S, d_in, best_s);
  return hipGetLastError();
}

hipError_t launch_select(const float* partials, int64_t n_blocks, int n_cand, int64_t stride_b,
                         int64_t stride_c, double scale, const double* cand_scale, double* tot, float* err,
                         int32_t* best_idx, const float* S, int64_t d_in, float* best_s,
                         hipStream_t stream) {
  reduce_cand_kernel<<<n_cand, kRedThreads, 0, stream>>>(partials, n_blocks, stride_b, stride_c, scale,
                                                         cand_scale, tot);
  argmin_kernel<<<1, kRedThreads, 0, stream>>>(tot, n_cand, err, best_idx, S, d_in, best_s);
  return hipGetLastError();
}

}  // namespace awq
