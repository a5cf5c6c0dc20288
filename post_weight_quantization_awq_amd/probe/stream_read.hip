// Launch and streaming-read floors for gfx950: an empty kernel, and a kernel
// that reads a buffer once with 16-byte nontemporal loads (8 per thread, all
// in flight at once, one round per 256-thread block: the shape of the W4A16
// decode kernels without their arithmetic).  Timed one launch per packed
// linear of a decode step, they bound what any kernel of that step can reach:
// a launch that reads B bytes cannot finish faster than the read probe over B
// bytes, and a second launch per linear costs at least the empty kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int kRdThreads = 256;
constexpr int kRdUnroll = 8;
constexpr int64_t kRdPerBlock = (int64_t)kRdThreads * kRdUnroll;   // 16-byte words per block

__global__ void empty_kernel() {}

__global__ __launch_bounds__(kRdThreads) void stream_read_kernel(const u4v* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kRdPerBlock + threadIdx.x;
  u4v v[kRdUnroll];
#pragma unroll
  for (int u = 0; u < kRdUnroll; ++u) {   // clamped, so every load is unconditional
    const int64_t i = base + (int64_t)u * kRdThreads;
    v[u] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kRdUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u && threadIdx.x == 0) out[blockIdx.x] = acc;   // keeps the loads live
}

// The loads of the few-token W4A16 kernel without its arithmetic: a packed
// [d_in, n_words] word matrix read in strips of W word columns by blocks of 4
// waves; lane l reads W / 16 consecutive words of column group (l & 15) in the
// 8 rows 8 (l >> 4) + 0..7 of each 32-row step, `steps` steps per wave (all in
// flight at once), blocks mapped round-robin to the 8 XCDs with strips
// fastest.  W = 16 reads two 64-byte runs of a row per load instruction
// group of 16 lanes (one word each), W = 32 one 128-byte run (two words each).
template <int WPL>
__global__ __launch_bounds__(256) void strip_read_kernel(const uint32_t* __restrict__ q, int64_t d_in,
                                                         int64_t n_words, int steps_per_wave, int n_strips,
                                                         uint32_t* __restrict__ out) {
  constexpr int kW = 16 * WPL;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t nblk = gridDim.x, bid = blockIdx.x;
  const uint32_t xcd = bid % 8, qq = nblk / 8, rmd = nblk % 8;
  const uint32_t tile = xcd * qq + (xcd < rmd ? xcd : rmd) + bid / 8;
  const uint32_t strip = tile % (uint32_t)n_strips, range = tile / (uint32_t)n_strips;
  const int64_t col = (int64_t)strip * kW + WPL * (lane & 15);
  const int64_t cc = col + WPL <= n_words ? col : n_words - WPL;
  const int64_t r0 = ((int64_t)range * 4 + wv) * 32 * steps_per_wave;
  uint32_t acc = 0;
  for (int st0 = 0; st0 < steps_per_wave; st0 += 4) {
    uint32_t w[4][8][WPL];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      int64_t k = r0 + 32 * (st0 + st) + 8 * (lane >> 4);
      k = k + 8 <= d_in ? k : d_in - 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t* p = q + (k + r) * n_words + cc;
        if constexpr (WPL == 1) {
          w[st][r][0] = __builtin_nontemporal_load(p);
        } else {
          typedef uint32_t u2v __attribute__((ext_vector_type(2)));
          const u2v v = __builtin_nontemporal_load((const u2v*)p);
          w[st][r][0] = v.x;
          w[st][r][1] = v.y;
        }
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < WPL; ++e) acc ^= w[st][r][e];
  }
  if (acc == 0x9E3779B9u && lane == 0) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads a packed [d_in, n_words] word matrix (4-byte aligned) with the few-token
// kernel's pattern: `words_per_lane` 1 or 2 (strips of 16 or 32 words),
// `steps_per_wave` a multiple of 4, d_in a multiple of 128 * steps_per_wave,
// n_words a multiple of 2.  `out` holds one word per block (written only for an
// impossible value).  Returns 0, 1 for bad arguments, else the HIP error.
int awq_probe_strip_read(const void* q, int64_t d_in, int64_t n_words, int words_per_lane, int steps_per_wave,
                         uint32_t* out, void* stream) {
  if ((words_per_lane != 1 && words_per_lane != 2) || steps_per_wave < 4 || steps_per_wave % 4 != 0 ||
      d_in % (128 * steps_per_wave) != 0 || n_words < 32 || n_words % 2 != 0 || ((uintptr_t)q & 7u) != 0)
    return 1;
  const int64_t strip_w = 16 * words_per_lane;
  const int n_strips = (int)((n_words + strip_w - 1) / strip_w);
  const int64_t n_ranges = d_in / (128 * steps_per_wave);
  const unsigned g = (unsigned)(n_strips * n_ranges);
  if (words_per_lane == 1)
    strip_read_kernel<1><<<g, 256, 0, (hipStream_t)stream>>>((const uint32_t*)q, d_in, n_words, steps_per_wave,
                                                             n_strips, out);
  else
    strip_read_kernel<2><<<g, 256, 0, (hipStream_t)stream>>>((const uint32_t*)q, d_in, n_words, steps_per_wave,
                                                             n_strips, out);
  return (int)hipGetLastError();
}

// Blocks of awq_probe_strip_read (the size of its `out` in words).
int64_t awq_probe_strip_read_blocks(int64_t d_in, int64_t n_words, int words_per_lane, int steps_per_wave) {
  const int64_t strip_w = 16 * words_per_lane;
  return ((n_words + strip_w - 1) / strip_w) * (d_in / (128 * steps_per_wave));
}

// Launches `blocks` blocks of `threads` threads of an empty kernel.
int awq_probe_empty(int blocks, int threads, void* stream) {
  empty_kernel<<<blocks, threads, 0, (hipStream_t)stream>>>();
  return (int)hipGetLastError();
}

// Blocks of the read probe over `bytes` bytes (the size of `out` in words).
int64_t awq_probe_read_blocks(int64_t bytes) { return (bytes / 16 + kRdPerBlock - 1) / kRdPerBlock; }

// Reads `bytes` (a positive multiple of 16) from `src` (16-byte aligned) once;
// `out` holds awq_probe_read_blocks(bytes) words, written only for an
// impossible value.  Returns 0, 1 for a bad size, else the HIP error.
int awq_probe_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src & 15u) != 0) return 1;
  const int64_t n16 = bytes / 16;
  stream_read_kernel<<<(unsigned)awq_probe_read_blocks(bytes), kRdThreads, 0, (hipStream_t)stream>>>(
      (const u4v*)src, n16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
