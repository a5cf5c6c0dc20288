// Device-side helpers shared by the libawq kernels (gfx950, wave64).
//
// Quantizer conventions follow "From-Scratch AWQ INT4 Quantization on
// Qwen3-8B", section "Group-wise symmetric INT4": the step of a group is
// max|group| / 7 and codes are round(v / step) clamped to [-7, 7], rounding
// half to even; the whole library decides codes in fp32.  The asymmetric
// variant ("AWQ architecture, in depth": a 4-bit zero point per group, step
// about range / 15) takes the range [min(0, min v), max(0, max v)], step
// RN(range / 15), zero point z = rint(-min / step) in [0, 15] and codes
// rint(v / step) + z clamped to [0, 15].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

constexpr int kWave = 64;
constexpr int kQMax = 7;
constexpr int kMaxParts = 8;
constexpr int kMaxGrid = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: nontemporal hint)
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4v v = __builtin_nontemporal_load((const u32x4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Row-concatenated group of fp16 weight matrices, passed by value to kernels.
// The member scale vectors of a norm group: n device pointers to fp32 [d_in].
struct ScaleSet {
  const float* p[kMaxParts];
  int32_t n;
};

struct WParts {
  const uint16_t* ptr[kMaxParts];
  int64_t row_start[kMaxParts + 1];  // prefix sums of rows; row_start[n] = d_out
  int32_t n;
};

// Start of global row `row` of the concatenated parts.  The part's pointer and
// first row are chosen by selects over constant indices, so the kernel-argument
// arrays stay in scalar registers (indexing them by a per-lane part number
// would read the argument block with vector loads and wait on them).
__device__ __forceinline__ const uint16_t* row_ptr(const WParts& P, int64_t row, int64_t d_in) {
  const uint16_t* base = P.ptr[0];
  int64_t r0 = 0;
#pragma unroll
  for (int j = 1; j < kMaxParts; ++j) {
    const bool in = j < P.n && row >= P.row_start[j];
    base = in ? P.ptr[j] : base;
    r0 = in ? P.row_start[j] : r0;
  }
  return base + (row - r0) * d_in;
}

// Power-of-two operand scales of the output-score GEMM (in the workspace):
// X16 = fp16(X * xs), dW16[c] = fp16(dW_c * ds[c]); sums of squares of the
// product are multiplied back by inv[c] = 1 / (xs * ds[c])^2 (exact).
struct OutScales {
  float xs;
  float ds[kMaxGrid];
  double inv[kMaxGrid];
};

// 2^e with x * 2^e in [2^14, 2^15) (1 for x == 0): keeps a maximum magnitude
// well inside the fp16 range while using its precision.
__device__ __forceinline__ float pow2_scale_for(float x) {
  if (!(x > 0.0f)) return 1.0f;
  int p;
  (void)frexpf(x, &p);  // x = f * 2^p, f in [0.5, 1)
  int e = 15 - p;
  e = e > 120 ? 120 : (e < -120 ? -120 : e);
  return ldexpf(1.0f, e);
}

// ---- conversions ----------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default mode)
__device__ __forceinline__ uint16_t f2h_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Unpack 8 fp16 held in a uint4 to fp32.
__device__ __forceinline__ void unpack8_f16(const uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = h2f((uint16_t)(w[j] & 0xFFFFu));
    f[2 * j + 1] = h2f((uint16_t)(w[j] >> 16));
  }
}

// ---- exact step: RN(a / 7) -------------------------------------------------
// q0 = RN(a * RN(1/7)); the residual a - 7 q0 is exact under one FMA, and one
// correction step q0 + r * RN(1/7) rounds to the IEEE quotient.  Checked on the
// host against IEEE division for every finite non-negative float.
__device__ __forceinline__ float div7(float a) {
  const float z = 1.0f / 7.0f;
  float q0 = a * z;
  float r = __builtin_fmaf(-7.0f, q0, a);
  return __builtin_fmaf(r, z, q0);
}

// ---- exact step of the asymmetric grid: RN(a / 15) ---------------------------
// Same sequence with RN(1/15); checked on the host against IEEE division for
// every finite non-negative float.
__device__ __forceinline__ float div15(float a) {
  const float z = 1.0f / 15.0f;
  float q0 = a * z;
  float r = __builtin_fmaf(-15.0f, q0, a);
  return __builtin_fmaf(r, z, q0);
}
constexpr int kUMax = 15;  // asymmetric codes 0..15

// ---- code of v for a step (fp32, round half to even) -------------------------
// Fast path: r0 = v * rcp(step) lies within 8e-6 of v/step for |v/step| < 32,
// so rint(r0) equals rint(RN(v/step)) unless r0 is within 2^-12 of a
// half-integer; those (and any non-finite r0) take the IEEE division.
__device__ __forceinline__ float code_exact(float v, float step, float inv) {
  float r0 = v * inv;
  float n = __builtin_rintf(r0);
  float dist = 0.5f - __builtin_fabsf(r0 - n);
  if (!(dist > 0x1p-12f) || !(__builtin_fabsf(r0) < 32.0f)) {
    n = __builtin_rintf(v / step);
  }
  return n;
}

// ---- lane reductions (DPP within a row of 16 lanes) -------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// max over aligned groups of N lanes (N in 1, 2, 4, 8, 16); every lane gets it.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = __builtin_fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x = __builtin_fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x = __builtin_fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  if constexpr (N >= 16) x = __builtin_fmaxf(x, dpp_f<0x140>(x)); // row_mirror
  return x;
}

// Same for non-negative finite floats: their bit patterns order like the
// values, so the unsigned max folds into one DPP-modified VALU op per step
// (a float max would first canonicalize the permuted operand).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
template <int N>
__device__ __forceinline__ float group_max_nonneg(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if constexpr (N >= 2) u = max(u, dpp_u<0xB1>(u));
  if constexpr (N >= 4) u = max(u, dpp_u<0x4E>(u));
  if constexpr (N >= 8) u = max(u, dpp_u<0x141>(u));
  if constexpr (N >= 16) u = max(u, dpp_u<0x140>(u));
  return __builtin_bit_cast(float, u);
}
// Sum over each aligned row of 16 lanes (every lane of the row gets it);
// fixed pairing, so the result does not depend on scheduling.
template <int CTRL>
__device__ __forceinline__ float dpp_m(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_m<0xB1>(x);
  x += dpp_m<0x4E>(x);
  x += dpp_m<0x141>(x);
  x += dpp_m<0x140>(x);
  return x;
}

// Sum over the 64 lanes of a wave, fixed pairing (deterministic).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

}  // namespace awq
