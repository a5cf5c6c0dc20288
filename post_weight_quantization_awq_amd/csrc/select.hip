// First-minimum selection over the candidates' partial errors and the copy of
// the winning scale row.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

// ---------------------------------------------------------------------------
// Selection ("AWQ architecture, in depth", "The scale search as code": keep the
// candidate when err < best, i.e. the first minimum).
//
// Wave w of a block owns candidates w, w + 16, ...; lane l sums the partials
// b = l, l + 64, ... of each in fp64, in increasing b, and a fixed shuffle tree
// finishes the candidate's sum, so the totals do not depend on scheduling.
// The launch has one block per kSelThreads channels of the scale row: every
// block reduces all partials the same way and so finds the same winner, block
// 0 stores the totals and the index, and each block copies its own channels
// of the winner's scale row.
//   * Up to 1024 fp32 (256 fp64) partials per candidate and 32 candidates (one
//     or two candidates per wave, 16 (4) loads per lane each), straight-line code: the
//     partial loads, then every thread's scale for each candidate of its
//     channel, all in one trip to memory, so the copy needs no second one.
//   * Otherwise the loads go kSelBatch at a time across the wave's candidates
//     (unconditional, clamped, masked when added) and the scale row is read
//     once the winner is known.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelBatch = 32;
// loads per lane and candidate on the fast path (fp64 partials are few: chunk sums)
template <typename TP>
constexpr int sel_fast_u() { return sizeof(TP) == 8 ? 4 : 16; }
constexpr int kSelPrefetch = 32;   // candidates whose scales are loaded up front

template <typename TP>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const TP* __restrict__ part, int n_blocks, int n_cand,
                                                            double scale, const double* __restrict__ cand_scale,
                                                            double* __restrict__ tot, float* __restrict__ err,
                                                            int32_t* __restrict__ best_idx,
                                                            const float* __restrict__ S, int64_t d_in,
                                                            float* __restrict__ best_s) {
  constexpr int NW = kSelThreads / kWave;
  __shared__ double red[kMaxGrid];
  __shared__ int best_sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t ch = (int64_t)blockIdx.x * kSelThreads + tid;
  constexpr int FU = sel_fast_u<TP>();
  const bool fast = n_blocks <= FU * kWave && n_cand <= 2 * NW && n_cand <= kSelPrefetch;
  float sv[kSelPrefetch];
  if (fast) {
    const int c0 = wave < n_cand ? wave : 0;
    const int c1 = wave + NW < n_cand ? wave + NW : c0;
    TP v0[FU], v1[FU];
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      const int b = min(u * kWave + lane, n_blocks - 1);
      v0[u] = part[c0 * n_blocks + b];
      v1[u] = part[c1 * n_blocks + b];
    }
    if (S != nullptr) {
      const int64_t chc = ch < d_in ? ch : d_in - 1;
#pragma unroll
      for (int c = 0; c < kSelPrefetch; ++c) sv[c] = S[(int64_t)(c < n_cand ? c : n_cand - 1) * d_in + chc];
    }
    __builtin_amdgcn_sched_barrier(0);
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      const bool ok = u * kWave + lane < n_blocks;
      a0 += ok ? (double)v0[u] : 0.0;
      a1 += ok ? (double)v1[u] : 0.0;
    }
    a0 = wave_sum_d(a0);
    a1 = wave_sum_d(a1);
    if (lane == 0) {
      if (wave < n_cand) red[c0] = a0;
      if (wave + NW < n_cand) red[c1] = a1;
    }
  } else {
    const int n_u = (n_blocks + kWave - 1) / kWave;  // loads per lane and candidate
    const int my_c = wave < n_cand ? (n_cand - wave + NW - 1) / NW : 0;
    const int total = my_c * n_u;
    double acc = 0.0;
    int ci = 0, uu = 0;  // position of load j0: candidate wave + ci * NW, lane block uu * 64 + lane
    for (int j0 = 0; j0 < total; j0 += kSelBatch) {
      TP v[kSelBatch];
      bool ok[kSelBatch];
      int c = ci, q = uu;
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {  // unconditional loads (clamped), masked when added
        const int b = q * kWave + lane;
        ok[u] = j0 + u < total && b < n_blocks;
        v[u] = part[ok[u] ? (int64_t)(wave + c * NW) * n_blocks + b : 0];
        if (++q == n_u) {
          q = 0;
          ++c;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {
        if (j0 + u < total) {
          acc += ok[u] ? (double)v[u] : 0.0;
          if (++uu == n_u) {  // last load of this candidate (uniform over the wave)
            const double t = wave_sum_d(acc);
            if (lane == 0) red[wave + ci * NW] = t;
            acc = 0.0;
            uu = 0;
            ++ci;
          }
        }
      }
    }
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
  if (S != nullptr && ch < d_in) {
    const int k = best_sh;
    float val;
    if (fast) {
      val = sv[0];
#pragma unroll
      for (int c = 1; c < kSelPrefetch; ++c) val = c == k ? sv[c] : val;
    } else {
      val = S[(int64_t)k * d_in + ch];
    }
    best_s[ch] = val;
  }
}

static unsigned select_grid(const float* S, int64_t d_in) {
  return S != nullptr ? (unsigned)((d_in + kSelThreads - 1) / kSelThreads) : 1u;
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
