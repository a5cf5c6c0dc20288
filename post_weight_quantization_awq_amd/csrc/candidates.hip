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
// KB from L2) and evaluates the two extra powers on a wave of its own, which
// makes the table one wide launch with no cross-block step.  alpha = 0 is special-cased (x^0 = 1 for
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

// A block covers kCandChan channels of one grid point with one thread each,
// plus a fifth wave whose first two lanes evaluate t at the largest and the
// smallest x while the channel waves evaluate theirs, so only one fp64 power
// lies on the kernel's critical path.
constexpr int kCandChan = 256;
constexpr int kCandThreads = kCandChan + kWave;
constexpr int kCandBatch = 16;  // x_mean loads in flight per thread

__global__ __launch_bounds__(kCandThreads) void cand_table_kernel(const float* __restrict__ x_mean, int64_t d_in,
                                                                 int n_grid, double s_min, float* __restrict__ S,
                                                                 float* __restrict__ C2) {
  const int k = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool chan = tid < kCandChan;
  const int64_t i = (int64_t)blockIdx.x * kCandChan + tid;
  const float x = x_mean[i < d_in ? i : d_in - 1];
  // max / min of x over all channels, every thread taking a share
  float xmax = 0.0f, xmin = __builtin_inff();
  for (int64_t i0 = 0; i0 < d_in; i0 += (int64_t)kCandThreads * kCandBatch) {
    float v[kCandBatch];  // loads in flight; a clamped index past d_in repeats x[d_in - 1]
#pragma unroll
    for (int u = 0; u < kCandBatch; ++u) {
      const int64_t j = i0 + (int64_t)u * kCandThreads + tid;
      v[u] = x_mean[j < d_in ? j : d_in - 1];
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
  __shared__ double t_ext[2];
  if (lane == 0) {
    smax[wave] = xmax;
    smin[wave] = xmin;
  }
  __syncthreads();
  const double alpha = (double)k / (double)n_grid;
  float y = x;
  if (!chan) {
#pragma unroll
    for (int w = 0; w < kCandThreads / kWave; ++w) {
      xmax = __builtin_fmaxf(xmax, smax[w]);
      xmin = __builtin_fminf(xmin, smin[w]);
    }
    y = lane == 0 ? xmax : xmin;
  }
  const double t = cand_t(y, k, alpha, s_min);
  if (!chan && lane < 2) t_ext[lane] = t;
  __syncthreads();
  if (!chan || i >= d_in) return;
  const double norm = sqrt(t_ext[0] * t_ext[1]);
  const float s = (float)(t / norm);
  S[(int64_t)k * d_in + i] = s;
  if (C2) {
    const float c = x / s;
    C2[(int64_t)k * d_in + i] = c * c;
  }
}

hipError_t launch_candidates(const float* x_mean, int64_t d_in, int n_grid, double s_min, float* S, float* C2,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((d_in + kCandChan - 1) / kCandChan), (unsigned)n_grid);
  cand_table_kernel<<<grid, kCandThreads, 0, stream>>>(x_mean, d_in, n_grid, s_min, S, C2);
  return hipGetLastError();
}

}  // namespace awq
