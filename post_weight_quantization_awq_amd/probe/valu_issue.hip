// Issue-rate probes for gfx950.  VALU: how many wave64 VALU instructions a
// SIMD issues per second, by instruction class and for pairs of classes, with
// W waves per SIMD; this grounds the peak that the weight-score search kernel
// is measured against (it is bound by VALU issue, not by HBM).  Matrix cores:
// the rate of back-to-back 32x32x16 fp16 products on register operands, on
// zero and on random data (the output-score GEMM's ceiling on this machine).
//
// Each lane runs 8 independent chains (no chain waits on its own previous
// result for 8 instructions), unrolled 4 times per loop trip, so the loop's
// scalar branch is 1 instruction per 32 VALU ones.  Every instruction is
// written out in inline asm so the compiler can neither fold nor reorder
// them; none of them touches memory.  The host times the whole launch with
// HIP events; instructions per second per SIMD follow from the launch shape
// (one 256-thread block = 4 waves per compute unit and round of blocks).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

enum Kind : int {
  kFma = 0,       // v_fma_f32 d, a, b, d   (three VGPR sources)
  kMul = 1,       // v_mul_f32 d, a, d
  kAdd = 2,       // v_add_f32 d, a, d
  kMax3 = 3,      // v_max3_f32 d, a, b, d
  kRndne = 4,     // v_rndne_f32 d, d
  kFmac = 5,      // v_fmac_f32 d, a, b
  kCvt = 6,       // v_cvt_f32_f16 d, d
  kDppMax = 7,    // v_max_u32 d, d, d row_half_mirror (DPP)
  kFmaRndne = 8,  // alternating v_fma_f32 / v_rndne_f32
  kFmaMul = 9,    // alternating v_fma_f32 / v_mul_f32
  kFmaMax3 = 10,  // alternating v_fma_f32 / v_max3_f32
  kSearchMix = 11, // the weight-score element loop's mix: mul, max3 (half), fma, add, fma, fma
  kFmaMix = 12     // v_fma_mix_f32 d, a.f16, b, d (an fp16 operand widened in the multiply)
};

#define OP8(INS)                                                                         \
  INS(x0) INS(x1) INS(x2) INS(x3) INS(x4) INS(x5) INS(x6) INS(x7)

template <int K>
__global__ __launch_bounds__(256) void valu_issue_kernel(float* __restrict__ out, int iters, float a, float b) {
  float x0 = threadIdx.x * 1e-7f, x1 = x0 + 1.0f, x2 = x0 + 2.0f, x3 = x0 + 3.0f;
  float x4 = x0 + 4.0f, x5 = x0 + 5.0f, x6 = x0 + 6.0f, x7 = x0 + 7.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (K == kFma) {
#define I(x) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x) : "v"(a), "v"(b));
        OP8(I)
#undef I
      } else if constexpr (K == kMul) {
#define I(x) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(a));
        OP8(I)
#undef I
      } else if constexpr (K == kAdd) {
#define I(x) asm volatile("v_add_f32 %0, %1, %0" : "+v"(x) : "v"(a));
        OP8(I)
#undef I
      } else if constexpr (K == kMax3) {
#define I(x) asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x) : "v"(a), "v"(b));
        OP8(I)
#undef I
      } else if constexpr (K == kRndne) {
#define I(x) asm volatile("v_rndne_f32 %0, %0" : "+v"(x));
        OP8(I)
#undef I
      } else if constexpr (K == kFmac) {
#define I(x) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
        OP8(I)
#undef I
      } else if constexpr (K == kCvt) {
#define I(x) asm volatile("v_cvt_f32_f16 %0, %0" : "+v"(x));
        OP8(I)
#undef I
      } else if constexpr (K == kDppMax) {
#define I(x) asm volatile("v_max_u32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf" : "+v"(x));
        OP8(I)
#undef I
      } else if constexpr (K == kFmaRndne) {
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x0) : "v"(a), "v"(b));
        asm volatile("v_rndne_f32 %0, %0" : "+v"(x1));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x2) : "v"(a), "v"(b));
        asm volatile("v_rndne_f32 %0, %0" : "+v"(x3));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x4) : "v"(a), "v"(b));
        asm volatile("v_rndne_f32 %0, %0" : "+v"(x5));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x6) : "v"(a), "v"(b));
        asm volatile("v_rndne_f32 %0, %0" : "+v"(x7));
      } else if constexpr (K == kFmaMul) {
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x0) : "v"(a), "v"(b));
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x1) : "v"(a));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x2) : "v"(a), "v"(b));
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x3) : "v"(a));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x4) : "v"(a), "v"(b));
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x5) : "v"(a));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x6) : "v"(a), "v"(b));
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x7) : "v"(a));
      } else if constexpr (K == kFmaMax3) {
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x0) : "v"(a), "v"(b));
        asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x1) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x2) : "v"(a), "v"(b));
        asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x3) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x4) : "v"(a), "v"(b));
        asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x5) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x6) : "v"(a), "v"(b));
        asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x7) : "v"(a), "v"(b));
      } else if constexpr (K == kFmaMix) {
#define I(x) asm volatile("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,0,0]" : "+v"(x) : "v"(a), "v"(b));
        OP8(I)
#undef I
      } else {  // kSearchMix: per pair of elements mul, mul, max3, fma, fma, add, add, fma, fma, fma, fma (11 for 2)
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x0) : "v"(a));
        asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x1) : "v"(a));
        asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x2) : "v"(x0), "v"(x1));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x3) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x4) : "v"(a), "v"(b));
        asm volatile("v_add_f32 %0, %1, %0" : "+v"(x5) : "v"(b));
        asm volatile("v_add_f32 %0, %1, %0" : "+v"(x6) : "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x7) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x3) : "v"(a), "v"(b));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x4) : "v"(x5), "v"(x5));
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x7) : "v"(x6), "v"(x6));
      }
    }
  }
  const float r = ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7));
  if (r == 123.456f) out[blockIdx.x * blockDim.x + threadIdx.x] = r;  // keeps the chains live
}

// VALU instructions per lane per loop trip of each kind
int insts_per_trip(int kind) { return kind == kSearchMix ? 4 * 11 : 4 * 8; }

template <int K>
hipError_t launch(int blocks, int iters, float* out, hipStream_t s) {
  valu_issue_kernel<K><<<blocks, 256, 0, s>>>(out, iters, 1.0000001f, 1e-7f);
  return hipGetLastError();
}

// Matrix-core issue probe: each wave loads 8 fragments of v_mfma_f32_32x32x16_f16
// operands (4 of A, 2 of B, from the given buffers) once, then runs `iters`
// rounds of the 8 independent 32x32x16 products (4 x 2 accumulator tiles, as
// the output-score GEMM's wave tile) with no memory traffic.  The operand
// values set the power the matrix cores draw, and with it the clock: the host
// runs it on all-zero and on random fp16 operands.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256, 2) void mfma_issue_kernel(const uint4* __restrict__ A, const uint4* __restrict__ B,
                                                            float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  h8v a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(h8v, A[i * 64 + lane]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = __builtin_bit_cast(h8v, B[j * 64 + lane]);
  f16v acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) r += acc[i][j][e];
  if (r == 123.456f) out[blockIdx.x * blockDim.x + threadIdx.x] = r;  // keeps the products live
}

}  // namespace

extern "C" {

// Launches `blocks` blocks of 256 threads (4 waves) of the matrix-core probe:
// A holds 4 x 64 and B 2 x 64 16-byte fragments (fp16), out blocks * 256 floats.
// Flops per launch: blocks * 4 waves * iters * 8 * 2 * 32 * 32 * 16.
int awq_probe_mfma(int blocks, int iters, const void* A, const void* B, float* out, void* stream) {
  mfma_issue_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4*)A, (const uint4*)B, out, iters);
  return (int)hipGetLastError();
}

// Number of kinds, and VALU instructions per lane and loop trip of a kind.
int awq_probe_valu_kinds(void) { return kFmaMix + 1; }
int awq_probe_valu_insts_per_trip(int kind) { return insts_per_trip(kind); }

// Launches `blocks` blocks of 256 threads running `iters` loop trips of `kind`
// on `stream`; `out` is a device buffer of blocks * 256 floats (written only
// for an impossible value).  Returns 0, 1 for a bad kind, else the HIP error.
int awq_probe_valu(int kind, int blocks, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case kFma: return launch<kFma>(blocks, iters, out, s);
    case kMul: return launch<kMul>(blocks, iters, out, s);
    case kAdd: return launch<kAdd>(blocks, iters, out, s);
    case kMax3: return launch<kMax3>(blocks, iters, out, s);
    case kRndne: return launch<kRndne>(blocks, iters, out, s);
    case kFmac: return launch<kFmac>(blocks, iters, out, s);
    case kCvt: return launch<kCvt>(blocks, iters, out, s);
    case kDppMax: return launch<kDppMax>(blocks, iters, out, s);
    case kFmaRndne: return launch<kFmaRndne>(blocks, iters, out, s);
    case kFmaMul: return launch<kFmaMul>(blocks, iters, out, s);
    case kFmaMax3: return launch<kFmaMax3>(blocks, iters, out, s);
    case kSearchMix: return launch<kSearchMix>(blocks, iters, out, s);
    case kFmaMix: return launch<kFmaMix>(blocks, iters, out, s);
    default: return 1;
  }
}

}  // extern "C"
