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
// Tile: one quantization group column (G inputs) by 8192*R/G rows (128 rows
// for G = 128, R = 2).  Each lane holds 32 inputs of R rows, loaded as packed
// fp16 (four 16-byte chunks, interleaved with the other G/32 lanes of the row
// so that one load instruction reads G/32 * 16 contiguous bytes of a row) and
// widened to fp32 once, outside the candidate loop.  The G/32 lanes of a row
// combine their maxima with DPP row permutes.  The candidate scales and
// (x/s)^2 of the block's columns are staged in LDS.  Each row's chain (group
// max, step, reciprocal) is serial, so the kernel is sized for three resident
// blocks per compute unit (three waves per SIMD, at most 168 VGPRs): with two
// rows per lane that measured 9-14% faster than four rows at two waves per
// SIMD.
//
// ASYM: the asymmetric grid ("AWQ architecture, in depth", a 4-bit zero point
// per group, step ~ range / 15).  Each row tracks max(v) and max(-v) (both
// start non-negative, so the range contains 0), step = RN(range / 15), and per
// element the code rint(v / step): the zero point z only bounds the codes to
// [-z, 15 - z], which changes a code only at a half-way tie of the range's
// ends (see the loop), so the error sums run 6.5 lane-ops per element·point.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kSearchThreads = 256;
constexpr int kSearchE = 32;  // inputs per lane per row
constexpr int kSearchR = 2;   // rows per lane
constexpr int kStageV = 4;    // float4 per candidate table and thread per staging batch
// Initial value of a group's running max: zero groups then get a tiny positive
// step, so q = 0 and d = 0 exactly without a select (any group whose max is
// below it contributes less than 2^-200 to the score).
constexpr float kTinyMax = 0x1p-100f;

template <int G>
constexpr int search_rows_per_block() { return (kSearchThreads / (G / kSearchE)) * kSearchR; }

// rint(v * inv) for |v * inv| < 2^22: fma(v, inv, 1.5 * 2^23) rounds the exact
// product to an integer (the sum's ulp is 1; ties to even, 1.5 * 2^23 being
// even), and subtracting 1.5 * 2^23 is exact.  Two dual-issue operations in
// place of a multiply and the single-pipe round (measured 2% faster on the
// sweep); it differs from rint(RN(v * inv)) only when the rounding of the
// product would cross a half-way point.
__device__ __forceinline__ float round_scaled(float v, float inv) {
  return __builtin_fmaf(v, inv, 12582912.0f) - 12582912.0f;
}

template <int G, bool ASYM>
__global__ __launch_bounds__(kSearchThreads, 3) void search_weight_kernel(
    const WParts P, int64_t d_out, int64_t d_in, int n_grid, const float* __restrict__ S,
    const float* __restrict__ C2, float* __restrict__ partials) {
  constexpr int R = kSearchR;
  constexpr int LPG = G / kSearchE;            // lanes per group row (1, 2 or 4)
  constexpr int RS = kSearchThreads / LPG;     // row slots per block
  constexpr int RB = RS * R;                   // rows per block
  constexpr int NC = kSearchE / 8;             // 16-byte chunks per lane and row
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  extern __shared__ float lds[];               // s [n_grid][G], then (x/s)^2 [n_grid][G]
  float* s_l = lds;
  float* c_l = lds + n_grid * G;
  __shared__ float red[kMaxGrid][kSearchThreads / 16];

  const uint32_t n_gcol = (uint32_t)(d_in / G);
  const uint32_t gcol = blockIdx.x % n_gcol;
  const int64_t rblk = blockIdx.x / n_gcol;
  const int64_t c0 = (int64_t)gcol * G;
  const int tid = threadIdx.x;

  // W tile first: it is the bulk of the kernel's traffic.  Every lane loads a
  // row that exists (rows past d_out read row d_out - 1) and those rows are
  // cleared once all loads have landed, so no load waits behind a branch.
  const int lg = tid % LPG;
  const int slot = tid / LPG;
  // chunk c of this lane covers group columns (c * LPG + lg) * 8 .. + 7
  uint4 w[R][NC];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = min(rblk * RB + slot + (int64_t)RS * r, d_out - 1);
    const uint4* p = (const uint4*)(row_ptr(P, row, d_in) + c0);
#pragma unroll
    for (int c = 0; c < NC; ++c) w[r][c] = ld_nt(p + c * LPG + lg);
  }
  // Candidate scales and (x/s)^2 of the block's columns into LDS, issued
  // while the W loads are in flight, kStageV float4 per table and thread at a
  // time.  Indices past the table are clamped to its last entry, for the loads
  // and the stores alike (those lanes write the value that entry holds), so
  // no load sits behind a branch and waits alone.
  const int n_st = n_grid * (G / 4);
  for (int base = 0; base < n_st; base += kStageV * kSearchThreads) {
    float4 a[kStageV], b[kStageV];
    int ix[kStageV];
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
      ix[u] = min(base + u * kSearchThreads + tid, n_st - 1);
      const int64_t off = (int64_t)(ix[u] / (G / 4)) * d_in + c0 + 4 * (ix[u] % (G / 4));
      a[u] = *(const float4*)(S + off);
      b[u] = *(const float4*)(C2 + off);
    }
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
      ((float4*)s_l)[ix[u]] = a[u];
      ((float4*)c_l)[ix[u]] = b[u];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (rblk * RB + slot + (int64_t)RS * r >= d_out) {
#pragma unroll
      for (int c = 0; c < NC; ++c) w[r][c] = make_uint4(0, 0, 0, 0);
    }
  }

  for (int k = 0; k < n_grid; ++k) {
    float s[kSearchE];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4* sp = (const float4*)(s_l + k * G + (c * LPG + lg) * 8);
      const float4 t0 = sp[0], t1 = sp[1];
      s[8 * c + 0] = t0.x; s[8 * c + 1] = t0.y; s[8 * c + 2] = t0.z; s[8 * c + 3] = t0.w;
      s[8 * c + 4] = t1.x; s[8 * c + 5] = t1.y; s[8 * c + 6] = t1.z; s[8 * c + 7] = t1.w;
    }
    float acc[kSearchE];
#pragma unroll
    for (int j = 0; j < kSearchE; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[kSearchE];
      float m = kTinyMax;
      float mn = 0.0f;  // ASYM: max(-v), the range's lower end negated
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const h8 h = __builtin_bit_cast(h8, w[r][c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[8 * c + e] = __builtin_fmaf((float)h[e], s[8 * c + e], 0.0f);
          if constexpr (ASYM) {
            m = __builtin_fmaxf(m, v[8 * c + e]);
            mn = __builtin_fmaxf(mn, -v[8 * c + e]);
          } else {
            m = __builtin_fmaxf(m, __builtin_fabsf(v[8 * c + e]));
          }
        }
      }
      m = group_max_nonneg<LPG>(m);
      if constexpr (ASYM) {
        mn = group_max_nonneg<LPG>(mn);
        const float step = div15(m + mn);
        const float inv = __builtin_amdgcn_rcpf(step);
        // The code clamp to [-z, 15 - z] only changes a code when an end of the
        // range sits on a half-way tie that the zero point's rounding resolved
        // the other way (v / step within an ulp or two of k + 1/2 at the group's
        // extreme element): it is left out of the error sums here (one element's
        // error differs by at most a step^2 in such a case), and kept, exactly,
        // where codes are stored (pack) or form the output-score operand.
#pragma unroll
        for (int j = 0; j < kSearchE; ++j) {
          const float q = round_scaled(v[j], inv);
          const float d = __builtin_fmaf(-step, q, v[j]);
          acc[j] = __builtin_fmaf(d, d, acc[j]);
        }
      } else {
        const float step = div7(m);
        const float inv = __builtin_amdgcn_rcpf(step);
#pragma unroll
        for (int j = 0; j < kSearchE; ++j) {
          const float q = round_scaled(v[j], inv);
          const float d = __builtin_fmaf(-step, q, v[j]);
          acc[j] = __builtin_fmaf(d, d, acc[j]);
        }
      }
    }
    float e = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4* cp = (const float4*)(c_l + k * G + (c * LPG + lg) * 8);
      const float4 t0 = cp[0], t1 = cp[1];
      e = __builtin_fmaf(t0.x, acc[8 * c + 0], e);
      e = __builtin_fmaf(t0.y, acc[8 * c + 1], e);
      e = __builtin_fmaf(t0.z, acc[8 * c + 2], e);
      e = __builtin_fmaf(t0.w, acc[8 * c + 3], e);
      e = __builtin_fmaf(t1.x, acc[8 * c + 4], e);
      e = __builtin_fmaf(t1.y, acc[8 * c + 5], e);
      e = __builtin_fmaf(t1.z, acc[8 * c + 6], e);
      e = __builtin_fmaf(t1.w, acc[8 * c + 7], e);
    }
    e = row16_sum(e);
    if ((tid & 15) == 0) red[k][tid >> 4] = e;
  }
  __syncthreads();
  if (tid < n_grid) {  // candidate-major: partials[k * n_blocks + block]
    const float* q = red[tid];
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = q[2 * i] + q[2 * i + 1];
    partials[(int64_t)tid * gridDim.x + blockIdx.x] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  }
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

template <bool ASYM>
static void launch_search_weight_t(int group_size, const WParts& parts, int64_t d_out, int64_t d_in, int n_grid,
                                   const float* S, const float* C2, float* partials, hipStream_t stream) {
  const unsigned nb = (unsigned)search_weight_blocks(group_size, d_out, d_in);
  const size_t shm = (size_t)2 * n_grid * group_size * sizeof(float);
  switch (group_size) {
    case 32:
      search_weight_kernel<32, ASYM><<<nb, kSearchThreads, shm, stream>>>(parts, d_out, d_in, n_grid, S, C2, partials);
      break;
    case 64:
      search_weight_kernel<64, ASYM><<<nb, kSearchThreads, shm, stream>>>(parts, d_out, d_in, n_grid, S, C2, partials);
      break;
    default:
      search_weight_kernel<128, ASYM><<<nb, kSearchThreads, shm, stream>>>(parts, d_out, d_in, n_grid, S, C2, partials);
      break;
  }
}

hipError_t launch_search_weight(int group_size, bool asym, const WParts& parts, int64_t d_out, int64_t d_in,
                                int n_grid, const float* S, const float* C2, float* partials,
                                hipStream_t stream) {
  if (asym) launch_search_weight_t<true>(group_size, parts, d_out, d_in, n_grid, S, C2, partials, stream);
  else launch_search_weight_t<false>(group_size, parts, d_out, d_in, n_grid, S, C2, partials, stream);
  return hipGetLastError();
}

}  // namespace awq
