// Duo scaling, "AWQ architecture, in depth", section "The scale search as
// code" (duo_scaling=True): each candidate divides x_mean^r by the group's
// row-normalised mean weight magnitude per input channel raised to 1 - r.
//
//   w_mean[i] = (1/d_out) sum_o |W[o, i]| / max_j |W[o, j]|   (quotients IEEE
//               fp32, an all-zero row contributing 0; sums in fp64)
//   t_k[i]    = max(x_mean[i]^r / (w_mean[i]^(1-r) + 1e-4), s_min),  r = k / n_grid
//   s_k[i]    = RN32(t_k[i] / sqrt(max_i t_k[i] * min_i t_k[i]))        (fp64)
//
// Unlike the plain candidates, t is not monotone in x_mean, so the extrema
// need every channel: one launch evaluates t (kept in fp64) with per-block
// extrema, a second normalises.  w_mean takes a pass for the row maxima and a
// split column reduction (fixed order, like the activation statistics).
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kDuoThreads = 256;
constexpr int kDuoCols = 64 * 8;    // channels per column block (8 per lane)
constexpr int kDuoSplitRows = 64;   // rows per split (16 per wave)

// one wave per row: the largest |w| of the row (fp16 magnitudes order like
// their bit patterns with the sign cleared; weights are finite).  A lane's
// loads of a stretch of 8 chunks are all issued before the first max.
__global__ __launch_bounds__(kDuoThreads) void row_absmax_kernel(const WParts P, int64_t d_out, int64_t d_in,
                                                                 float* __restrict__ rmax) {
  constexpr int kU = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kDuoThreads / kWave) + (threadIdx.x >> 6);
  if (row >= d_out) return;  // uniform over the wave
  const uint4* p = (const uint4*)row_ptr(P, row, d_in);
  const int n = (int)(d_in / 8);
  uint32_t m = 0;
  for (int c0 = 0; c0 < n; c0 += kU * kWave) {
    uint4 u[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int c = c0 + j * kWave + lane;
      u[j] = c < n ? p[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) m = max(m, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, kWave));
  if (lane == 0) rmax[row] = h2f((uint16_t)m);
}

// IEEE fp32 quotient a / b of fp16 magnitudes 0 <= a <= b, b > 0, given y
// within one ulp of 1/b: q0 = a*y, the residual a - q0*b is exact in one FMA
// (b has 11 significant bits), and one correction step rounds to the IEEE
// quotient.  Checked on the host for every such pair of finite fp16 values
// and each of the three y (RN(1/b) and its two neighbours).
__device__ __forceinline__ float div_f16_mag(float a, float b, float y) {
  const float q0 = a * y;
  const float r = __builtin_fmaf(-q0, b, a);
  return __builtin_fmaf(r, y, q0);
}

// split y, column block x: sum over the split's rows of |w| / rowmax for 8
// channels per lane; wave v takes rows y*64 + v + 4i, loads all 16 first
__global__ __launch_bounds__(kDuoThreads) void wmean_partial_kernel(const WParts P, int64_t d_out, int64_t d_in,
                                                                    const float* __restrict__ rmax,
                                                                    double* __restrict__ part) {
  constexpr int RPW = kDuoSplitRows / 4;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t col0 = ((int64_t)blockIdx.x * kWave + lane) * 8;
  const int64_t r0 = (int64_t)blockIdx.y * kDuoSplitRows + wv;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  if (col0 < d_in) {
    uint4 u[RPW];
    float m[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {  // rows past d_out load row d_out - 1 and add nothing
      const int64_t row = min(r0 + 4 * i, d_out - 1);
      u[i] = *(const uint4*)(row_ptr(P, row, d_in) + col0);
      m[i] = rmax[row];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const bool use = r0 + 4 * i < d_out && m[i] > 0.0f;
      const float y = __builtin_amdgcn_rcpf(m[i]);  // v_rcp_f32: within 1 ulp
      const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = div_f16_mag(h2f((uint16_t)(w[j] & 0x7FFFu)), m[i], y);
        const float hi = div_f16_mag(h2f((uint16_t)((w[j] >> 16) & 0x7FFFu)), m[i], y);
        acc[2 * j] += use ? (double)lo : 0.0;
        acc[2 * j + 1] += use ? (double)hi : 0.0;
      }
    }
  }
  __shared__ double red[4][kDuoCols];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wv][lane * 8 + j] = acc[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kDuoCols; idx += kDuoThreads) {
    const int64_t c = (int64_t)blockIdx.x * kDuoCols + idx;
    if (c < d_in) part[blockIdx.y * d_in + c] = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
  }
}

int64_t wmean_splits(int64_t d_out) { return (d_out + kDuoSplitRows - 1) / kDuoSplitRows; }

hipError_t launch_weight_channel_mean(const WParts& parts, int64_t d_out, int64_t d_in, float* rmax, double* part,
                                      float* w_mean, hipStream_t stream) {
  row_absmax_kernel<<<(unsigned)((d_out + 3) / 4), kDuoThreads, 0, stream>>>(parts, d_out, d_in, rmax);
  const int64_t n_split = wmean_splits(d_out);
  wmean_partial_kernel<<<dim3((unsigned)((d_in + kDuoCols - 1) / kDuoCols), (unsigned)n_split), kDuoThreads, 0,
                         stream>>>(parts, d_out, d_in, rmax, part);
  return launch_split_mean(part, n_split, d_in, 1.0 / (double)d_out, w_mean, stream);
}

// ---- duo candidates --------------------------------------------------------
constexpr int kDuoCandThreads = 256;

__global__ __launch_bounds__(kDuoCandThreads) void duo_t_kernel(const float* __restrict__ x_mean,
                                                                const float* __restrict__ w_mean, int64_t d_in,
                                                                int n_grid, double s_min, double* __restrict__ T,
                                                                double* __restrict__ ext) {
  const int k = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * kDuoCandThreads + threadIdx.x;
  const double alpha = (double)k / (double)n_grid;
  double tmax = -__builtin_inf(), tmin = __builtin_inf();
  if (i < d_in) {
    const double x = (double)x_mean[i], w = (double)w_mean[i];
    const double num = k == 0 ? 1.0 : pow(x, alpha);
    const double den = (k == 0 ? w : pow(w, 1.0 - alpha)) + 1e-4;
    double t = num / den;
    t = t > s_min ? t : s_min;
    T[(int64_t)k * d_in + i] = t;
    tmax = tmin = t;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    tmax = fmax(tmax, __shfl_xor(tmax, m, kWave));
    tmin = fmin(tmin, __shfl_xor(tmin, m, kWave));
  }
  __shared__ double smax[kDuoCandThreads / kWave], smin[kDuoCandThreads / kWave];
  const int wave = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    smax[wave] = tmax;
    smin[wave] = tmin;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int v = 1; v < kDuoCandThreads / kWave; ++v) {
      tmax = fmax(tmax, smax[v]);
      tmin = fmin(tmin, smin[v]);
    }
    ext[((int64_t)k * gridDim.x + blockIdx.x) * 2] = tmax;
    ext[((int64_t)k * gridDim.x + blockIdx.x) * 2 + 1] = tmin;
  }
}

__global__ __launch_bounds__(kDuoCandThreads) void duo_norm_kernel(const float* __restrict__ x_mean,
                                                                   const double* __restrict__ T,
                                                                   const double* __restrict__ ext, int64_t d_in,
                                                                   int n_blk, float* __restrict__ S,
                                                                   float* __restrict__ C2) {
  const int k = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * kDuoCandThreads + threadIdx.x;
  // every thread folds the (few) block extrema of candidate k in the same order
  double tmax = -__builtin_inf(), tmin = __builtin_inf();
  for (int b = 0; b < n_blk; ++b) {
    tmax = fmax(tmax, ext[((int64_t)k * n_blk + b) * 2]);
    tmin = fmin(tmin, ext[((int64_t)k * n_blk + b) * 2 + 1]);
  }
  if (i >= d_in) return;
  const double norm = sqrt(tmax * tmin);
  const float s = (float)(T[(int64_t)k * d_in + i] / norm);
  S[(int64_t)k * d_in + i] = s;
  if (C2) {
    const float c = x_mean[i] / s;
    C2[(int64_t)k * d_in + i] = c * c;
  }
}

int64_t duo_cand_blocks(int64_t d_in) { return (d_in + kDuoCandThreads - 1) / kDuoCandThreads; }

hipError_t launch_candidates_duo(const float* x_mean, const float* w_mean, int64_t d_in, int n_grid, double s_min,
                                 double* T, double* ext, float* S, float* C2, hipStream_t stream) {
  const int64_t nb = duo_cand_blocks(d_in);
  const dim3 grid((unsigned)nb, (unsigned)n_grid);
  duo_t_kernel<<<grid, kDuoCandThreads, 0, stream>>>(x_mean, w_mean, d_in, n_grid, s_min, T, ext);
  duo_norm_kernel<<<grid, kDuoCandThreads, 0, stream>>>(x_mean, T, ext, d_in, (int)nb, S, C2);
  return hipGetLastError();
}

}  // namespace awq
