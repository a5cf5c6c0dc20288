// Candidate scale table of the alpha grid search.
// "AWQ architecture, in depth", section "The scale search as code" (non-duo
// branch): for r = i / n_grid, s = x_mean^r, clamped below at 1e-4, then
// divided by sqrt(max(s) * min(s)) so the scales stay centred near 1.
// "Weight-Only Quantization: GPTQ and AWQ", section 5 (AWQ): s = |X|^alpha.
//
// Two fully parallel passes over (grid point, channel): the first evaluates
// t = max(x^alpha, s_min) in fp64 and keeps the extrema per block, the second
// evaluates t again, normalises and rounds once to fp32.  alpha = 0 is
// special-cased (x^0 = 1 for every x, including 0), so row 0 is exactly 1.0
// and candidate 0 is plain round-to-nearest.  For the
// weight score the kernel also stores (x / s)^2 in fp32, the per-column weight
// of the squared error in the scaled domain: (w - q*step/s) * x = (v - q*step) * x/s.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

__device__ __forceinline__ double cand_t(float x, int k, double alpha, double s_min) {
  double t = (k == 0) ? 1.0 : pow((double)x, alpha);
  return t > s_min ? t : s_min;
}

constexpr int kCandThreads = 256;

// pass 1: per-block max / min of t[k, i]
__global__ __launch_bounds__(kCandThreads) void cand_ext_kernel(const float* __restrict__ x_mean, int64_t d_in,
                                                               int n_grid, double s_min, double* __restrict__ bmax,
                                                               double* __restrict__ bmin) {
  const int k = blockIdx.y;
  const double alpha = (double)k / (double)n_grid;
  const int64_t i = (int64_t)blockIdx.x * kCandThreads + threadIdx.x;
  double vmax = 0.0, vmin = __builtin_inf();
  if (i < d_in) {
    vmax = cand_t(x_mean[i], k, alpha, s_min);
    vmin = vmax;
  }
  __shared__ double smax[kCandThreads], smin[kCandThreads];
  smax[threadIdx.x] = vmax;
  smin[threadIdx.x] = vmin;
  __syncthreads();
  for (int w = kCandThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
      smax[threadIdx.x] = smax[threadIdx.x] > smax[threadIdx.x + w] ? smax[threadIdx.x] : smax[threadIdx.x + w];
      smin[threadIdx.x] = smin[threadIdx.x] < smin[threadIdx.x + w] ? smin[threadIdx.x] : smin[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    bmax[(int64_t)k * gridDim.x + blockIdx.x] = smax[0];
    bmin[(int64_t)k * gridDim.x + blockIdx.x] = smin[0];
  }
}

// pass 2: norm_k = sqrt(max t * min t) from the block extrema; S = fp32(t / norm)
__global__ __launch_bounds__(kCandThreads) void cand_s_kernel(const float* __restrict__ x_mean, int64_t d_in,
                                                             int n_grid, double s_min,
                                                             const double* __restrict__ bmax,
                                                             const double* __restrict__ bmin, int n_blk,
                                                             float* __restrict__ S, float* __restrict__ C2) {
  const int k = blockIdx.y;
  __shared__ double norm_sh;
  if (threadIdx.x == 0) {
    double mx = 0.0, mn = __builtin_inf();
    for (int b = 0; b < n_blk; ++b) {
      const double a = bmax[(int64_t)k * n_blk + b], c = bmin[(int64_t)k * n_blk + b];
      mx = a > mx ? a : mx;
      mn = c < mn ? c : mn;
    }
    norm_sh = sqrt(mx * mn);
  }
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kCandThreads + threadIdx.x;
  if (i >= d_in) return;
  const double alpha = (double)k / (double)n_grid;
  const float s = (float)(cand_t(x_mean[i], k, alpha, s_min) / norm_sh);
  S[(int64_t)k * d_in + i] = s;
  if (C2) {
    const float c = x_mean[i] / s;
    C2[(int64_t)k * d_in + i] = c * c;
  }
}

size_t candidates_workspace_bytes(int64_t d_in, int n_grid) {
  const int64_t n_blk = (d_in + kCandThreads - 1) / kCandThreads;
  return (size_t)n_grid * 2 * n_blk * sizeof(double);
}

hipError_t launch_candidates(const float* x_mean, int64_t d_in, int n_grid, double s_min, float* S, float* C2,
                             void* ws, hipStream_t stream) {
  const int n_blk = (int)((d_in + kCandThreads - 1) / kCandThreads);
  double* bmax = (double*)ws;
  double* bmin = bmax + (int64_t)n_grid * n_blk;
  dim3 grid((unsigned)n_blk, (unsigned)n_grid);
  cand_ext_kernel<<<grid, kCandThreads, 0, stream>>>(x_mean, d_in, n_grid, s_min, bmax, bmin);
  cand_s_kernel<<<grid, kCandThreads, 0, stream>>>(x_mean, d_in, n_grid, s_min, bmax, bmin, n_blk, S, C2);
  return hipGetLastError();
}

}  // namespace awq
