// Measurement aids.  mfma_probe_kernel: the dense bf16 MFMA rate the device sustains, for pricing
// the attention kernel against what the hardware delivers at its running clock beside the 2.4
// GHz specification.  lds_read_probe_kernel: a buffer read once with the global-to-LDS loads
// the attention kernel streams its pages with, so that the profiler's byte counter for those
// loads can be scaled the way a plain copy's is.
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup g (256 threads) reads bytes [64 KiB g, 64 KiB (g + 1)) of src into LDS, wave w the
// 1 KiB blocks w, w + 4, ..., lane i 16 bytes of each, and writes one float per thread.
__global__ __launch_bounds__(kLdsProbeThreads) void lds_read_probe_kernel(const char* __restrict__ src,
                                                                         float* __restrict__ out) {
  __shared__ __align__(1024) char buf[kLdsProbeBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned base = unsigned(size_t((lds_ptr_t)buf));
  const char* g = src + size_t(blockIdx.x) * kLdsProbeBlock;
  constexpr int kWaves = kLdsProbeThreads / 64, kBlocks = kLdsProbeBlock / 1024;
#pragma unroll
  for (int j = 0; j < kBlocks / kWaves; ++j) {
    const int b = j * kWaves + wave;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(
                     __builtin_amdgcn_readfirstlane(int(base) + b * 1024)),
                 "v"(g + b * 1024 + lane * 16)
                 : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  out[size_t(blockIdx.x) * kLdsProbeThreads + threadIdx.x] = float(buf[threadIdx.x * 16]);
}

}  // namespace

hipError_t launch_lds_read_probe(const void* src, int64_t bytes, float* out, hipStream_t st) {
  hipLaunchKernelGGL(lds_read_probe_kernel, dim3(unsigned(bytes / kLdsProbeBlock)), dim3(kLdsProbeThreads), 0, st,
                     static_cast<const char*>(src), out);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int32_t workgroups, int32_t iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace sr
