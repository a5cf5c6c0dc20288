// Candidate scale table of the alpha grid search.
// "AWQ architecture, in depth", section "The scale search as code" (non-duo
// branch): for r = i / n_grid, s = x_mean^r, clamped below at 1e-4, then
// divided by sqrt(max(s) * min(s)) so the scales stay centred near 1.
// "Weight-Only Quantization: GPTQ and AWQ", section 5 (AWQ): s = |X|^alpha.
//
// t = max(x^alpha, s_min) is evaluated in fp64 and rounded once to fp32 after
// the division.  x^alpha is non-decreasing in x for alpha > 0, and so is
// max(., s_min), so the extrema of t over the channels are t at the largest
// and at the smallest x: every block reduces max/min of x_mean itself (a few
// KB from L2) and evaluates two extra powers, which makes the table one wide
// launch with no cross-block step.  alpha = 0 is special-cased (x^0 = 1 for
// every x, including 0), so row 0 is exactly 1.0 and candidate 0 is plain
// round-to-nearest.  For the weight score the kernel also stores (x / s)^2 in
// fp32, the per-column weight of the squared error in the scaled domain:
// (w - q*step/s) * x = (v - q*step) * x/s.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

__device__ __forceinline__ double cand_t(float x, int k, double alpha, double s_min) {
  double t = (k == 0) ? 1.0 : pow((double)x, alpha);
  return t > s_min ? t : s_min;
}

constexpr int kCandThreads = 256;

constexpr int kCandBatch = 16;  // x_mean loads in flight per thread

__global__ __launch_bounds__(kCandThreads) void cand_table_kernel(const float* __restrict__ x_mean, int64_t d_in,
                                                                 int n_grid, double s_min, float* __restrict__ S,
                                                                 float* __restrict__ C2) {
  const int k = blockIdx.y;
  const int tid = threadIdx.x;
  // max / min of x over all channels
  float xmax = 0.0f, xmin = __builtin_inff();
  for (int64_t i0 = 0; i0 < d_in; i0 += (int64_t)kCandThreads * kCandBatch) {
    float v[kCandBatch];  // loads in flight; a clamped index past d_in repeats x[d_in - 1]
#pragma unroll
    for (int u = 0; u < kCandBatch; ++u) {
      const int64_t i = i0 + (int64_t)u * kCandThreads + tid;
      v[u] = x_mean[i < d_in ? i : d_in - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kCandBatch; ++u) {
      xmax = __builtin_fmaxf(xmax, v[u]);
      xmin = __builtin_fminf(xmin, v[u]);
    }
  }
  xmax = wave_max(xmax);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) xmin = __builtin_fminf(xmin, __shfl_xor(xmin, m, kWave));
  __shared__ float smax[kCandThreads / kWave], smin[kCandThreads / kWave];
  if (tid % kWave == 0) {
    smax[tid / kWave] = xmax;
    smin[tid / kWave] = xmin;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCandThreads / kWave; ++w) {
    xmax = __builtin_fmaxf(xmax, smax[w]);
    xmin = __builtin_fminf(xmin, smin[w]);
  }
  const double alpha = (double)k / (double)n_grid;
  const double norm = sqrt(cand_t(xmax, k, alpha, s_min) * cand_t(xmin, k, alpha, s_min));
  const int64_t i = (int64_t)blockIdx.x * kCandThreads + tid;
  if (i >= d_in) return;
  const float x = x_mean[i];
  const float s = (float)(cand_t(x, k, alpha, s_min) / norm);
  S[(int64_t)k * d_in + i] = s;
  if (C2) {
    const float c = x / s;
    C2[(int64_t)k * d_in + i] = c * c;
  }
}

hipError_t launch_candidates(const float* x_mean, int64_t d_in, int n_grid, double s_min, float* S, float* C2,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((d_in + kCandThreads - 1) / kCandThreads), (unsigned)n_grid);
  cand_table_kernel<<<grid, kCandThreads, 0, stream>>>(x_mean, d_in, n_grid, s_min, S, C2);
  return hipGetLastError();
}

}  // namespace awq
