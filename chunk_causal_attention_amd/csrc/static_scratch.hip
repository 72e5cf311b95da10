// Library-owned scratch for callers that cannot allocate device memory (code under graph
// capture, serving loops or harnesses that forbid hipMalloc): a fixed file-scope device array
// that the no-allocation entry point (sr_global_attention_static) uses as its workspace.
//
// The array's name is a host-side stand-in in host code, not a device address.  The device
// address of each GPU's copy is looked up once per device, with that device current, by
// hipGetSymbolAddress and kept in a per-device table; host code only ever passes that address
// to kernels.  Every call on a device shares its copy: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace sr {
namespace {

// Records of the split-K global-token kernel, then its per-head arrival counters.
constexpr size_t kScratchFloats = size_t(kStaticRecordFloats) + size_t(kStaticCounters);
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_ptr[kMaxDevices] = {};

__global__ void zero_counters_kernel(int32_t* c, int32_t n) {
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

}  // namespace

hipError_t static_scratch_workspace(SplitWorkspace* ws, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    float* p = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // The counters must start at zero; every call leaves them at zero again.  A fill kernel, not
    // a memset, so that a first call under graph capture records an ordinary kernel node.
    hipLaunchKernelGGL(zero_counters_kernel, dim3(16), dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(p + kStaticRecordFloats), kStaticCounters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  ws->cus_per_xcd = 1;  // marks the workspace as present for the few-row kernel
  ws->records = g_ptr[dev];
  ws->counters = reinterpret_cast<int32_t*>(g_ptr[dev] + kStaticRecordFloats);
  return hipSuccess;
}

}  // namespace sr
