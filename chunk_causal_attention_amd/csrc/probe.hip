// Measurement aid: the dense bf16 MFMA rate the device sustains, for pricing the attention kernel
// against what the hardware delivers at its running clock beside the 2.4 GHz specification.
//
// Every wave keeps four independent accumulator chains of v_mfma_f32_32x32x16_bf16 busy with
// register operands (no memory traffic in the loop), two workgroups of eight waves per compute
// unit, so each SIMD always has an instruction ready.  Each thread writes one float (the sum of
// its accumulators), so the work cannot be dropped.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ out, int32_t iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __bf16(0.001f * float((threadIdx.x + e) & 31));
    b[e] = __bf16(0.5f);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[size_t(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int32_t workgroups, int32_t iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace sr
