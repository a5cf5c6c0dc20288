// Per-input-channel mean |x| over calibration tokens.
// "From-Scratch AWQ INT4 Quantization on Qwen3-8B", section "AWQ scaling"
// (x = |X|.mean(0)); "AWQ architecture, in depth", section "The scale search
// as code" (x.abs().float().mean(dim=0)).
//
// HBM-bound column reduction: 2 bytes read per element.  Each lane owns 8
// consecutive channels (one 16-byte load per token row); a block is 64 lanes
// wide and 4 waves tall, the 4 waves taking 16-row slices of each 64-row
// step; blocks split the token axis.  Per-lane sums are fp64 (full rate on
// CDNA4 VALU), the split partials are combined in a fixed order by a second
// kernel, so the result is deterministic and independent of the launch shape
// up to fp64 rounding.
//
// The token axis is cut into whole splits of a multiple of 64 rows, streamed
// by the main kernel (no bounds logic: every 16-row batch is full), and the
// leftover rows, cut into 64-row splits for the generic kernel, which also
// covers unaligned inputs.
#include <algorithm>

#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = 64 * 8;    // channels per block
constexpr int kRowsPerWaveIter = 16;  // rows per batch of one wave
constexpr int64_t kStepRows = 4 * kRowsPerWaveIter;

template <bool BF16>
__device__ __forceinline__ void acc8(const uint4 u, double* acc) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
    const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
    acc[2 * j] += (double)__builtin_fabsf(lo);
    acc[2 * j + 1] += (double)__builtin_fabsf(hi);
  }
}

// Four rows at once: per channel the four |x| are added in fp32, in row
// order, and the sum once in fp64.  The fp32 adds of non-negative terms err by
// at most 3 * 2^-24 of the four-row sum, so the channel total stays within
// 1.8e-7 of its fp64 value, while the half-rate fp64 conversion and add run
// once per four rows instead of per row (the kernel shares the SIMDs with the
// weight-score search in the calibration sweep).
template <bool BF16>
__device__ __forceinline__ float absx(uint32_t w, bool hi) {
  if (BF16) return __builtin_fabsf(__builtin_bit_cast(float, hi ? (w & 0xFFFF0000u) : (w << 16)));
  return __builtin_fabsf(h2f((uint16_t)(hi ? (w >> 16) : (w & 0xFFFFu))));
}
template <bool BF16>
__device__ __forceinline__ void acc8_rows4(const uint4* u, double* acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w0 = j == 0 ? u[0].x : j == 1 ? u[0].y : j == 2 ? u[0].z : u[0].w;
    const uint32_t w1 = j == 0 ? u[1].x : j == 1 ? u[1].y : j == 2 ? u[1].z : u[1].w;
    const uint32_t w2 = j == 0 ? u[2].x : j == 1 ? u[2].y : j == 2 ? u[2].z : u[2].w;
    const uint32_t w3 = j == 0 ? u[3].x : j == 1 ? u[3].y : j == 2 ? u[3].z : u[3].w;
    const float lo = ((absx<BF16>(w0, false) + absx<BF16>(w1, false)) + absx<BF16>(w2, false)) + absx<BF16>(w3, false);
    const float hi = ((absx<BF16>(w0, true) + absx<BF16>(w1, true)) + absx<BF16>(w2, true)) + absx<BF16>(w3, true);
    acc[2 * j] += (double)lo;
    acc[2 * j + 1] += (double)hi;
  }
}

template <bool BF16>
__device__ __forceinline__ void acc8_masked(const uint4 u, bool in, double* acc) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = BF16 ? bf2f((uint16_t)(w[j] & 0xFFFFu)) : h2f((uint16_t)(w[j] & 0xFFFFu));
    const float hi = BF16 ? bf2f((uint16_t)(w[j] >> 16)) : h2f((uint16_t)(w[j] >> 16));
    acc[2 * j] += in ? (double)__builtin_fabsf(lo) : 0.0;
    acc[2 * j + 1] += in ? (double)__builtin_fabsf(hi) : 0.0;
  }
}

// The WAVES waves' 8 channel sums of the block -> part[split][channel], added
// in wave order.
template <int WAVES>
__device__ __forceinline__ void store_partials(const double* acc, int wv, int lane, int64_t split, int64_t d_in,
                                               double* __restrict__ part) {
  __shared__ double red[WAVES][64 * 8];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wv][lane * 8 + j] = acc[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 8; idx += WAVES * 64) {
    const int64_t c = (int64_t)blockIdx.x * kStatsCols + idx;
    if (c < d_in) {
      double s = red[0][idx];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s += red[w][idx];
      part[split * d_in + c] = s;
    }
  }
}

// Main kernel: a block of 4 waves covers rows [y * 4 ROWS, (y + 1) * 4 ROWS),
// all inside X (X 16-byte aligned, ld and d_in multiples of 8); every wave
// issues its ROWS row loads at once and adds them as they arrive.  One batch
// per wave and small blocks dispatched split by split keep the rows read at
// any moment contiguous in memory and leave several blocks per CU to cover
// each other's reduction tails: on 0.5-1.6 GB inputs this streams ~6.2 TB/s
// (a plain streaming read reaches ~7.1), where waves that stream several
// batches each (two register sets, a rolling prefetch) or 16-wave blocks (one
// per CU) reached 4.7-6 TB/s.
template <bool BF16, int ROWS>
__global__ __launch_bounds__(kStatsThreads) void act_stats_main_kernel(const uint16_t* __restrict__ X, int64_t d_in,
                                                                      int64_t ld, double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  if (col0 < d_in) {
    const uint16_t* p = X + ((int64_t)blockIdx.y * (4 * ROWS) + wv * ROWS) * ld + col0;
    uint4 u[ROWS];
#pragma unroll
    for (int q = 0; q < ROWS; ++q) u[q] = ld_nt(p + q * ld);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < ROWS; q += 4) acc8_rows4<BF16>(&u[q], acc);
  }
  store_partials<4>(acc, wv, lane, blockIdx.y, d_in, part);
}

// Lean main kernel, used for 128-row splits: the rows of
// act_stats_main_kernel<BF16, 32>, with the wave's 32 rows in batches of 8
// loads, so that a wave fits in 80 registers, and a persistent grid of about
// three blocks per four compute units that loops over the splits.  A block keeps its
// fp64 channel sums across all its splits (y, y + gridDim.y, ... in order) and
// writes one partial per block row, so its waves never meet at a barrier
// inside the loop and the final kernel adds gridDim.y partials instead of one
// per split.  A statistics block then runs on a compute unit beside three
// blocks of the weight-score search (3 x 144 registers of each SIMD's 512),
// and the statistics of the next linears stream from HBM while the search
// computes, instead of taking every free slot of the machine and stalling it.
//
// Grid size: the search alone already holds the chip at its sustained power
// limit (~1.34 kW at a ~2.2 GHz shader clock on the 36-block Qwen3-8B sweep;
// the statistics alone draw ~1.08 kW), and with both running the clock drops
// to ~2.0 GHz, so the stream rate that suits the pair is below this kernel's
// best alone.  On that sweep 192 blocks (6.4 TB/s alone) measured 30.7-31.0
// ms per step against 31.8-32.1 with 256 (6.9 TB/s alone), 31.2-31.3 with
// 160 and 31.4 with 224, in interleaved runs on one machine.
constexpr int64_t kLeanBlocks = 192;   // blocks of the persistent grid

template <bool BF16>
__global__ __launch_bounds__(kStatsThreads, 6) void act_stats_lean_kernel(const uint16_t* __restrict__ X,
                                                                         int64_t d_in, int64_t ld, int64_t n_split,
                                                                         double* __restrict__ part) {
  constexpr int ROWS = 32, BATCH = 8;
  // Beside the search's waves, a statistics wave whose loads have landed
  // issues first, adds its rows and sends the next loads, so the bytes in
  // flight do not wait on the search's instruction stream (the sweep step
  // measured 32.9 ms with this and the four-row fp32 sums, 33.8-34.0 without).
  __builtin_amdgcn_s_setprio(3);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  if (col0 < d_in) {
    for (int64_t y = blockIdx.y; y < n_split; y += gridDim.y) {   // persistent over the splits
      const uint16_t* p = X + (y * (4 * ROWS) + wv * ROWS) * ld + col0;
#pragma unroll
      for (int b0 = 0; b0 < ROWS; b0 += BATCH) {
        uint4 u[BATCH];
#pragma unroll
        for (int q = 0; q < BATCH; ++q) u[q] = ld_nt(p + (b0 + q) * ld);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < BATCH; q += 4) acc8_rows4<BF16>(&u[q], acc);
      }
    }
  }
  store_partials<4>(acc, wv, lane, blockIdx.y, d_in, part);
}

// Generic kernel: split y covers rows [row0 + y * rps, min(T, ... + rps)) and
// writes partial row split0 + y.  Rows past the end load a clamped row and add
// nothing (no branch between the 16 loads and their uses); unaligned inputs
// take scalar loads.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kStatsThreads) void act_stats_partial_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t d_in, int64_t ld, int64_t row0, int64_t rps, int64_t split0,
    double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const int64_t r_begin = row0 + (int64_t)blockIdx.y * rps;
  const int64_t r_end = min(T, r_begin + rps);
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;

  if (col0 < d_in) {
    if (VEC && col0 + 8 <= d_in) {
      const uint16_t* p = X + col0;
      for (int64_t base = r_begin + wv * kRowsPerWaveIter; base < r_end; base += kStepRows) {
        uint4 u[kRowsPerWaveIter];
#pragma unroll
        for (int q = 0; q < kRowsPerWaveIter; ++q) {
          const int64_t r = base + q < r_end ? base + q : r_end - 1;
          u[q] = ld_nt(p + r * ld);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kRowsPerWaveIter; ++q) acc8_masked<BF16>(u[q], base + q < r_end, acc);
      }
    } else {
      for (int64_t base = r_begin + wv * kRowsPerWaveIter; base < r_end; base += kStepRows) {
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
  store_partials<4>(acc, wv, lane, split0 + blockIdx.y, d_in, part);
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

// Whole splits of rps rows for the main kernels: 128 rows (32 per wave, fp64
// partials at 1/32 of X's bytes) when that still gives at least 1024 splits
// x column blocks, else 64; then the T % rps leftover rows in 64-row splits
// for the generic kernel.
static void stats_split(int64_t T, int64_t d_in, int64_t* rps, int64_t* n_main, int64_t* n_tail) {
  const int64_t n_cb = (d_in + kStatsCols - 1) / kStatsCols;
  *rps = (T / (2 * kStepRows)) * n_cb >= 1024 ? 2 * kStepRows : kStepRows;
  *n_main = T / *rps;
  *n_tail = (T - *n_main * *rps + kStepRows - 1) / kStepRows;
}

void act_stats_plan(int64_t T, int64_t d_in, int64_t* n_split, int64_t* rows_per_split) {
  if (T <= 0 || d_in <= 0) {
    *n_split = 0;
    *rows_per_split = kStepRows;
    return;
  }
  int64_t rps, n_main, n_tail;
  stats_split(T, d_in, &rps, &n_main, &n_tail);
  *rows_per_split = rps;
  *n_split = n_main + n_tail;
}

// Launches the partial kernels; returns the number of partial rows written
// (at most the plan's n_split: the lean kernel writes one per block row).
template <bool BF16>
static int64_t launch_stats_t(const uint16_t* x, int64_t T, int64_t d_in, int64_t ld, double* part,
                              hipStream_t stream) {
  int64_t rps, n_main, n_tail;
  stats_split(T, d_in, &rps, &n_main, &n_tail);
  const unsigned n_cb = (unsigned)((d_in + kStatsCols - 1) / kStatsCols);
  const bool vec = ((uintptr_t)x % 16 == 0) && (ld % 8 == 0);
  if (vec) {
    int64_t n_written = n_main;
    if (n_main > 0) {
      const dim3 grid(n_cb, (unsigned)n_main);
      if (d_in % 8 == 0) {
        if (rps == kStepRows) {
          act_stats_main_kernel<BF16, 16><<<grid, kStatsThreads, 0, stream>>>(x, d_in, ld, part);
        } else {
          n_written = std::max<int64_t>(1, std::min<int64_t>(n_main, kLeanBlocks / n_cb));
          act_stats_lean_kernel<BF16><<<dim3(n_cb, (unsigned)n_written), kStatsThreads, 0, stream>>>(
              x, d_in, ld, n_main, part);
        }
      } else {
        act_stats_partial_kernel<BF16, true><<<dim3(n_cb, (unsigned)n_main), kStatsThreads, 0, stream>>>(
            x, T, d_in, ld, 0, rps, 0, part);
      }
    }
    if (n_tail > 0)
      act_stats_partial_kernel<BF16, true><<<dim3(n_cb, (unsigned)n_tail), kStatsThreads, 0, stream>>>(
          x, T, d_in, ld, n_main * rps, kStepRows, n_written, part);
    return n_written + n_tail;
  } else {
    if (n_main > 0)
      act_stats_partial_kernel<BF16, false><<<dim3(n_cb, (unsigned)n_main), kStatsThreads, 0, stream>>>(
          x, T, d_in, ld, 0, rps, 0, part);
    if (n_tail > 0)
      act_stats_partial_kernel<BF16, false><<<dim3(n_cb, (unsigned)n_tail), kStatsThreads, 0, stream>>>(
          x, T, d_in, ld, n_main * rps, kStepRows, n_main, part);
    return n_main + n_tail;
  }
}

hipError_t launch_act_stats(const void* X, bool bf16, int64_t T, int64_t d_in, int64_t ld,
                            float inv_count, int accumulate, float* x_mean, void* ws,
                            hipStream_t stream) {
  int64_t n_split, rps;
  act_stats_plan(T, d_in, &n_split, &rps);
  double* part = (double*)ws;
  if (n_split > 0)
    n_split = bf16 ? launch_stats_t<true>((const uint16_t*)X, T, d_in, ld, part, stream)
                   : launch_stats_t<false>((const uint16_t*)X, T, d_in, ld, part, stream);
  act_stats_final_kernel<<<(unsigned)((d_in + 31) / 32), 256, 0, stream>>>(
      part, n_split, d_in, (double)inv_count, accumulate, x_mean);
  return hipGetLastError();
}

hipError_t launch_split_mean(const double* part, int64_t n_split, int64_t d_in, double inv_count, float* out,
                             hipStream_t stream) {
  act_stats_final_kernel<<<(unsigned)((d_in + 31) / 32), 256, 0, stream>>>(part, n_split, d_in, inv_count, 0, out);
  return hipGetLastError();
}

}  // namespace awq
