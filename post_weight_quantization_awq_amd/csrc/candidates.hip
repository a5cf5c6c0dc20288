// Candidate scale table of the alpha grid search.
// "AWQ architecture, in depth", section "The scale search as code" (non-duo
// branch): for r = i / n_grid, s = x_mean^r, clamped below at 1e-4, then
// divided by sqrt(max(s) * min(s)) so the scales stay centred near 1.
// "Weight-Only Quantization: GPTQ and AWQ", section 5 (AWQ): s = |X|^alpha.
//
// One block per grid point; the values are evaluated in fp64 and rounded once
// to fp32.  alpha = 0 is special-cased (x^0 = 1 for every x, including 0), so
// row 0 is exactly 1.0 and candidate 0 is plain round-to-nearest.  For the
// weight score the kernel also stores (x / s)^2 in fp32, the per-column weight
// of the squared error in the scaled domain: (w - q*step/s) * x = (v - q*step) * x/s.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

__device__ __forceinline__ double cand_t(float x, int k, double alpha, double s_min) {
  double t = (k == 0) ? 1.0 : pow((double)x, alpha);
  return t > s_min ? t : s_min;
}

__global__ __launch_bounds__(256) void candidates_kernel(const float* __restrict__ x_mean, int64_t d_in,
                                                         int n_grid, double s_min, float* __restrict__ S,
                                                         float* __restrict__ C2) {
  const int k = blockIdx.x;
  const double alpha = (double)k / (double)n_grid;
  double tmax = 0.0, tmin = __builtin_inf();
  for (int64_t i = threadIdx.x; i < d_in; i += blockDim.x) {
    double t = cand_t(x_mean[i], k, alpha, s_min);
    tmax = t > tmax ? t : tmax;
    tmin = t < tmin ? t : tmin;
  }
  __shared__ double smax[256], smin[256];
  smax[threadIdx.x] = tmax;
  smin[threadIdx.x] = tmin;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
      smax[threadIdx.x] = smax[threadIdx.x] > smax[threadIdx.x + w] ? smax[threadIdx.x] : smax[threadIdx.x + w];
      smin[threadIdx.x] = smin[threadIdx.x] < smin[threadIdx.x + w] ? smin[threadIdx.x] : smin[threadIdx.x + w];
    }
    __syncthreads();
  }
  const double norm = sqrt(smax[0] * smin[0]);
  for (int64_t i = threadIdx.x; i < d_in; i += blockDim.x) {
    const float x = x_mean[i];
    const float s = (float)(cand_t(x, k, alpha, s_min) / norm);
    S[(int64_t)k * d_in + i] = s;
    if (C2) {
      const float c = x / s;
      C2[(int64_t)k * d_in + i] = c * c;
    }
  }
}

hipError_t launch_candidates(const float* x_mean, int64_t d_in, int n_grid, double s_min, float* S,
                             float* C2, hipStream_t stream) {
  candidates_kernel<<<n_grid, 256, 0, stream>>>(x_mean, d_in, n_grid, s_min, S, C2);
  return hipGetLastError();
}

}  // namespace awq
