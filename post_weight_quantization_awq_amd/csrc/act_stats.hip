// Per-input-channel mean |x| over calibration tokens.
// "From-Scratch AWQ INT4 Quantization on Qwen3-8B", section "AWQ scaling"
// (x = |X|.mean(0)); "AWQ architecture, in depth", section "The scale search
// as code" (x.abs().float().mean(dim=0)).
//
// HBM-bound column reduction: 2 bytes read per element.  Each lane owns 8
// consecutive channels (one 16-byte load per token row) and keeps 16 row loads
// in flight; the 4 waves of a block take 16-row slices; blocks split the token
// axis.  Per-lane sums are
// fp64 (full rate on CDNA4 VALU), the split partials are combined in a fixed
// order by a second kernel, so the result is deterministic and independent of
// the launch shape up to fp64 rounding.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = 64 * 8;  // channels per block

constexpr int kRowsPerWaveIter = 16;  // rows whose loads one lane keeps in flight

template <bool BF16>
__device__ __forceinline__ void acc8(const uint4 u, bool in, double* acc) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
    const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
    acc[2 * j] += in ? (double)__builtin_fabsf(lo) : 0.0;
    acc[2 * j + 1] += in ? (double)__builtin_fabsf(hi) : 0.0;
  }
}

// Block: 64 lanes x 8 channels wide, 4 waves; the block's token range is walked
// in 64-row steps, wave w taking rows w*16 .. w*16+15 of each step with all 16
// loads issued before any is used.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kStatsThreads) void act_stats_partial_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t d_in, int64_t ld, int64_t rows_per_split,
    double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r_end = min(T, r_begin + rows_per_split);
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;

  if (col0 < d_in) {
    if (VEC && col0 + 8 <= d_in) {
      const uint16_t* p = X + col0;
      for (int64_t base = r_begin + wv * kRowsPerWaveIter; base < r_end; base += 4 * kRowsPerWaveIter) {
        // unconditional loads of a clamped row (rows past r_end add nothing):
        // no branch between the loads and their uses, all 16 issue first and
        // each use waits for its own load only
        uint4 u[kRowsPerWaveIter];
#pragma unroll
        for (int q = 0; q < kRowsPerWaveIter; ++q) {
          const int64_t r = base + q < r_end ? base + q : r_end - 1;
          u[q] = ld_nt(p + r * ld);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kRowsPerWaveIter; ++q) acc8<BF16>(u[q], base + q < r_end, acc);
      }
    } else {
      for (int64_t base = r_begin + wv * kRowsPerWaveIter; base < r_end; base += 4 * kRowsPerWaveIter) {
        for (int64_t r = base; r < base + kRowsPerWaveIter && r < r_end; ++r) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (col0 + j < d_in) {
              const uint16_t b = X[r * ld + col0 + j];
              acc[j] += (double)__builtin_fabsf(BF16 ? bf2f(b) : h2f(b));
            }
          }
        }
      }
    }
  }

  __shared__ double red[4][64 * 8];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wv][lane * 8 + j] = acc[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 8; idx += kStatsThreads) {
    const int64_t c = (int64_t)blockIdx.x * kStatsCols + idx;
    if (c < d_in) {
      double s = red[0][idx];
      s += red[1][idx];
      s += red[2][idx];
      s += red[3][idx];
      part[(int64_t)blockIdx.y * d_in + c] = s;
    }
  }
}

// 32 channels x 8 split-slices per block: each thread sums every 8th split
// partial of one channel, the 8 slice sums are then added in a fixed order.
constexpr int kFinalBatch = 8;
__global__ __launch_bounds__(256) void act_stats_final_kernel(const double* __restrict__ part, int64_t n_split,
                                                             int64_t d_in, double inv_count, int accumulate,
                                                             float* __restrict__ x_mean) {
  const int lane = threadIdx.x & 31, slice = threadIdx.x >> 5;
  const int64_t i = (int64_t)blockIdx.x * 32 + lane;
  double s = 0.0;
  if (i < d_in) {
    for (int64_t p0 = slice; p0 < n_split; p0 += 8 * kFinalBatch) {
      double v[kFinalBatch];  // loads in flight (clamped index), added in increasing p
#pragma unroll
      for (int u = 0; u < kFinalBatch; ++u) {
        const int64_t p = p0 + 8 * (int64_t)u;
        v[u] = part[(p < n_split ? p : n_split - 1) * d_in + i];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kFinalBatch; ++u) s += p0 + 8 * (int64_t)u < n_split ? v[u] : 0.0;
    }
  }
  __shared__ double red[8][32];
  red[slice][lane] = s;
  __syncthreads();
  if (slice == 0 && i < d_in) {
    double t = red[0][lane];
#pragma unroll
    for (int q = 1; q < 8; ++q) t += red[q][lane];
    double v = t * inv_count;
    if (accumulate) v += (double)x_mean[i];
    x_mean[i] = (float)v;
  }
}

void act_stats_plan(int64_t T, int64_t d_in, int64_t* n_split, int64_t* rows_per_split) {
  if (T <= 0 || d_in <= 0) {
    *n_split = 0;
    *rows_per_split = 64;
    return;
  }
  // 64 token rows per split (one row step of the 4 waves) up to 512 for long
  // calibration sets, keeping the fp64 partials a few percent of X
  int64_t rps = T / 256;
  rps = rps < 64 ? 64 : (rps > 512 ? 512 : rps);
  rps = (rps + 63) / 64 * 64;
  *rows_per_split = rps;
  *n_split = (T + rps - 1) / rps;
}

hipError_t launch_act_stats(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld,
                            float inv_count, int accumulate, float* x_mean, void* ws,
                            hipStream_t stream) {
  int64_t n_split, rps;
  act_stats_plan(T, d_in, &n_split, &rps);
  double* part = (double*)ws;
  if (n_split > 0) {
    const bool vec = ((uintptr_t)X % 16 == 0) && (ld % 8 == 0);
    dim3 grid((unsigned)((d_in + kStatsCols - 1) / kStatsCols), (unsigned)n_split);
    const uint16_t* x = (const uint16_t*)X;
    if (bf16) {
      if (vec) act_stats_partial_kernel<true, true><<<grid, kStatsThreads, 0, stream>>>(x, T, d_in, ld, rps, part);
      else act_stats_partial_kernel<true, false><<<grid, kStatsThreads, 0, stream>>>(x, T, d_in, ld, rps, part);
    } else {
      if (vec) act_stats_partial_kernel<false, true><<<grid, kStatsThreads, 0, stream>>>(x, T, d_in, ld, rps, part);
      else act_stats_partial_kernel<false, false><<<grid, kStatsThreads, 0, stream>>>(x, T, d_in, ld, rps, part);
    }
  }
  act_stats_final_kernel<<<(unsigned)((d_in + 31) / 32), 256, 0, stream>>>(
      part, n_split, d_in, (double)inv_count, accumulate, x_mean);
  return hipGetLastError();
}

}  // namespace awq
