// Norm-group export, "From-Scratch AWQ INT4 Quantization on Qwen3-8B", the
// exporter's steps 1-3: q/k/v share input_layernorm and gate/up share
// post_attention_layernorm, so the per-linear scales of a group are reduced
// to one shared scale -- the per-channel geometric mean over the member
// linears -- which is folded into the norm (norm.weight /= s_shared); the
// members are then re-quantized with the shared scale by the packing kernel,
// and o_proj / down_proj are packed at s = 1.
//
//   s_shared[i] = RN32(exp((1/M) sum_m ln s_m[i]))   (logarithms, sum in member
//                                                       order, exponential: fp64)
//   norm_out[i] = RN_dtype(norm[i] / s_shared[i])     (IEEE fp32 quotient)
//
// One thread per channel: a d_in-long elementwise pass, latency-bound at the
// sizes of a norm (a few thousand channels).
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kFoldThreads = 256;

// DT: AWQ norm dtype code (0 fp16, 1 bf16, 2 fp32), or -1 for no norm.  norm
// and norm_out may be the same buffer (each thread reads its element first).
template <int DT>
__global__ __launch_bounds__(kFoldThreads) void norm_group_fold_kernel(const ScaleSet S, int64_t d_in,
                                                                      const void* norm, void* norm_out,
                                                                      float* __restrict__ s_shared) {
  const int64_t i = (int64_t)blockIdx.x * kFoldThreads + threadIdx.x;
  if (i >= d_in) return;
  double acc = 0.0;
#pragma unroll
  for (int m = 0; m < kMaxParts; ++m)
    if (m < S.n) acc += log((double)S.p[m][i]);
  const float sh = (float)exp(acc / (double)S.n);
  s_shared[i] = sh;
  if constexpr (DT == 0) {
    const float q = h2f(((const uint16_t*)norm)[i]) / sh;
    ((uint16_t*)norm_out)[i] = f2h_bits(q);
  } else if constexpr (DT == 1) {
    const float q = bf2f(((const uint16_t*)norm)[i]) / sh;
    ((uint16_t*)norm_out)[i] = f2bf_bits(q);
  } else if constexpr (DT == 2) {
    ((float*)norm_out)[i] = ((const float*)norm)[i] / sh;
  }
}

hipError_t launch_norm_group_fold(const ScaleSet& S, int64_t d_in, const void* norm, int norm_dtype, void* norm_out,
                                  float* s_shared, hipStream_t stream) {
  const unsigned nb = (unsigned)((d_in + kFoldThreads - 1) / kFoldThreads);
  switch (norm != nullptr ? norm_dtype : -1) {
    case 0: norm_group_fold_kernel<0><<<nb, kFoldThreads, 0, stream>>>(S, d_in, norm, norm_out, s_shared); break;
    case 1: norm_group_fold_kernel<1><<<nb, kFoldThreads, 0, stream>>>(S, d_in, norm, norm_out, s_shared); break;
    case 2: norm_group_fold_kernel<2><<<nb, kFoldThreads, 0, stream>>>(S, d_in, norm, norm_out, s_shared); break;
    default: norm_group_fold_kernel<-1><<<nb, kFoldThreads, 0, stream>>>(S, d_in, norm, norm_out, s_shared); break;
  }
  return hipGetLastError();
}

}  // namespace awq
