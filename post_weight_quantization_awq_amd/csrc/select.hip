// First-minimum selection over the candidates' partial errors and the copy of
// the winning scale row.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

// ---------------------------------------------------------------------------
// Selection ("AWQ architecture, in depth", "The scale search as code": keep the
// candidate when err < best, i.e. the first minimum).
//
// Wave w of a block owns candidates w, w + 4, ...; lane l sums the partials
// b = l, l + 64, ... of each in fp64, in increasing b (kSelBatch loads in
// flight, clamped and masked), and a fixed shuffle tree finishes the
// candidate's sum, so the totals do not depend on scheduling.  The launch has
// one block per kSelChannels channels of the scale row: every block reduces
// all partials the same way and so finds the same winner, block 0 stores the
// totals and the index, and each block copies its channels of the winner's
// scale row.  Blocks are 4 waves of at most 80 VGPRs, so that one fits on a
// compute unit beside three waves per SIMD of the search kernel and the
// selection of one group need not wait for another group's search to drain.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;
constexpr int kSelChannels = 1024;   // scale-row channels copied per block
constexpr int kSelBatch = 16;

template <typename TP>
__global__ __launch_bounds__(kSelThreads, 6) void select_kernel(const TP* __restrict__ part, int n_blocks,
                                                               int n_cand, double scale,
                                                               const double* __restrict__ cand_scale,
                                                               double* __restrict__ tot, float* __restrict__ err,
                                                               int32_t* __restrict__ best_idx,
                                                               const float* __restrict__ S, int64_t d_in,
                                                               float* __restrict__ best_s) {
  constexpr int NW = kSelThreads / kWave;
  __shared__ double red[kMaxGrid];
  __shared__ int best_sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n_u = (n_blocks + kWave - 1) / kWave;  // loads per lane and candidate
  for (int c = wave; c < n_cand; c += NW) {
    const TP* pc = part + (int64_t)c * n_blocks;
    double acc = 0.0;
    for (int u0 = 0; u0 < n_u; u0 += kSelBatch) {
      TP v[kSelBatch];
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {  // unconditional loads (clamped), masked when added
        const int b = (u0 + u) * kWave + lane;
        v[u] = pc[b < n_blocks ? b : n_blocks - 1];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) acc += (u0 + u) * kWave + lane < n_blocks ? (double)v[u] : 0.0;
    }
    const double t = wave_sum_d(acc);
    if (lane == 0) red[c] = t;
  }
  __syncthreads();
  if (wave == 0) {
    const bool live = lane < n_cand;
    double t = __builtin_inf();
    if (live) {
      t = red[lane] * scale * (cand_scale != nullptr ? cand_scale[lane] : 1.0);
      if (blockIdx.x == 0) {
        tot[lane] = t;
        err[lane] = (float)t;
      }
    }
    double mn = t;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double o = __shfl_xor(mn, m, kWave);
      mn = o < mn ? o : mn;
    }
    const unsigned long long hit = __ballot(live && t == mn);
    const int b = hit ? __ffsll((long long)hit) - 1 : 0;
    if (lane == 0) {
      if (blockIdx.x == 0) best_idx[0] = b;
      best_sh = b;
    }
  }
  __syncthreads();
  if (S != nullptr) {
    const float* row = S + (int64_t)best_sh * d_in;
#pragma unroll
    for (int j = 0; j < kSelChannels / kSelThreads; ++j) {
      const int64_t ch = (int64_t)blockIdx.x * kSelChannels + j * kSelThreads + tid;
      if (ch < d_in) best_s[ch] = row[ch];
    }
  }
}

static unsigned select_grid(const float* S, int64_t d_in) {
  return S != nullptr ? (unsigned)((d_in + kSelChannels - 1) / kSelChannels) : 1u;
}

hipError_t launch_select(const float* partials, int64_t n_blocks, int n_cand, double scale,
                         const double* cand_scale, double* tot, float* err, int32_t* best_idx, const float* S,
                         int64_t d_in, float* best_s, hipStream_t stream) {
  select_kernel<float><<<select_grid(S, d_in), kSelThreads, 0, stream>>>(partials, (int)n_blocks, n_cand, scale,
                                                                         cand_scale, tot, err, best_idx, S, d_in, best_s);
  return hipGetLastError();
}

hipError_t launch_select(const double* partials, int64_t n_blocks, int n_cand, double scale,
                         const double* cand_scale, double* tot, float* err, int32_t* best_idx, const float* S,
                         int64_t d_in, float* best_s, hipStream_t stream) {
  select_kernel<double><<<select_grid(S, d_in), kSelThreads, 0, stream>>>(partials, (int)n_blocks, n_cand, scale,
                                                                          cand_scale, tot, err, best_idx, S, d_in, best_s);
  return hipGetLastError();
}

}  // namespace awq
