// VALU issue-rate probe for gfx950: how many wave64 VALU instructions a SIMD
// issues per second, by instruction class and for pairs of classes, with
// W waves per SIMD.  This grounds the peak that the weight-score search
// kernel is measured against (it is bound by VALU issue, not by HBM).
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
  kSearchMix = 11 // the weight-score element loop's mix: mul, max3 (half), fma, add, fma, fma
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

}  // namespace

extern "C" {

// Number of kinds, and VALU instructions per lane and loop trip of a kind.
int awq_probe_valu_kinds(void) { return kSearchMix + 1; }
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
    default: return 1;
  }
}

}  // extern "C"
