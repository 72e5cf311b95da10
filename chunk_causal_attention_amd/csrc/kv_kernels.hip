// KV-cache kernels: pool zeroing, chunk append (K rows + V transposed into pages), gather.
// These are HBM-bound copies; the append writes exactly the layout the attention kernel
// reads (StreamRender-H3 project page, "3.3 Inference Acceleration and End-to-End
// Deployment", persistent KV layout), so no repacking happens at attention time.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sr {
namespace {

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

constexpr int kAppendTokens = 64;  // tokens per workgroup (half a page)

// Workgroup (token tile of 64, head).  K rows are copied straight through in 16-byte
// pieces; V goes through LDS and is written transposed: for each feature d, the tile's
// 64 tokens are contiguous in the page.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(const T* __restrict__ k, const T* __restrict__ v, int n, int H,
                                                     T* __restrict__ kpool, T* __restrict__ vpool, int total_pages,
                                                     int page0) {
  constexpr int EPC = 16 / int(sizeof(T));  // elements per 16-byte piece
  constexpr int CPR = D / EPC;              // pieces per token row
  constexpr int PITCH = D + EPC;            // LDS row pitch (elements), padded by 16 bytes
  __shared__ __align__(16) T tile[kAppendTokens * PITCH];

  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kAppendTokens;
  const size_t page = size_t(h) * total_pages + page0 + t0 / SR_PAGE_TOKENS;
  T* kdst = kpool + (page * SR_PAGE_TOKENS + t0 % SR_PAGE_TOKENS) * D;
  const uint4 z = make_uint4(0, 0, 0, 0);

  for (int ci = threadIdx.x; ci < kAppendTokens * CPR; ci += blockDim.x) {
    const int r = ci / CPR, c = ci % CPR, t = t0 + r;
    const size_t src = (size_t(t) * H + h) * D + c * EPC;
    const uint4 kv = t < n ? *reinterpret_cast<const uint4*>(k + src) : z;
    const uint4 vv = t < n ? *reinterpret_cast<const uint4*>(v + src) : z;
    *reinterpret_cast<uint4*>(kdst + r * D + c * EPC) = kv;
    *reinterpret_cast<uint4*>(tile + r * PITCH + c * EPC) = vv;
  }
  __syncthreads();

  T* vdst = vpool + page * D * SR_PAGE_TOKENS + t0 % SR_PAGE_TOKENS;
  constexpr int CPD = kAppendTokens / EPC;  // pieces per feature row of the tile
  for (int ci = threadIdx.x; ci < D * CPD; ci += blockDim.x) {
    const int d = ci / CPD, c = ci % CPD;
    union {
      T e[EPC];
      uint4 u;
    } pk;
#pragma unroll
    for (int e = 0; e < EPC; ++e) pk.e[e] = tile[(c * EPC + e) * PITCH + d];
    *reinterpret_cast<uint4*>(vdst + size_t(d) * SR_PAGE_TOKENS + c * EPC) = pk.u;
  }
}

// Thread per (token, feature) with the token index fastest, so the transposed V pages are
// read along their contiguous direction.  Test/debug path; not tuned.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ kpool, const T* __restrict__ vpool,
                                                     SegTable tab, int total_pages, int H, int ntok,
                                                     T* __restrict__ kout, T* __restrict__ vout) {
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  for (int idx = threadIdx.x; idx < 64 * D; idx += blockDim.x) {
    const int tt = idx % 64, d = idx / 64, t = t0 + tt;
    if (t >= ntok) continue;
    int s = 0, off = t;
    while (s < tab.n - 1 && off >= tab.s[s].len) {
      off -= tab.s[s].len;
      ++s;
    }
    const size_t page = size_t(h) * total_pages + tab.s[s].page + off / SR_PAGE_TOKENS;
    const int row = off % SR_PAGE_TOKENS;
    kout[(size_t(t) * H + h) * D + d] = kpool[(page * SR_PAGE_TOKENS + row) * D + d];
    vout[(size_t(t) * H + h) * D + d] = vpool[(page * D + d) * SR_PAGE_TOKENS + row];
  }
}

template <typename T, int D>
hipError_t append_t(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0, int32_t npages,
                    hipStream_t st) {
  T* kpool = static_cast<T*>(pool);
  T* vpool = reinterpret_cast<T*>(static_cast<char*>(pool) + L.half_bytes);
  dim3 grid(npages * (SR_PAGE_TOKENS / kAppendTokens), L.H);
  hipLaunchKernelGGL((append_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(k),
                     static_cast<const T*>(v), n, L.H, kpool, vpool, L.total_pages, page0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t gather_t(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                    hipStream_t st) {
  const T* kpool = static_cast<const T*>(pool);
  const T* vpool = reinterpret_cast<const T*>(static_cast<const char*>(pool) + L.half_bytes);
  dim3 grid((ntok + 63) / 64, L.H);
  hipLaunchKernelGGL((gather_kernel<T, D>), grid, dim3(256), 0, st, kpool, vpool, t, L.total_pages, L.H, ntok,
                     static_cast<T*>(kout), static_cast<T*>(vout));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_append(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0,
                         int32_t npages, hipStream_t st) {
  if (npages == 0) return hipSuccess;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? append_t<uint16_t, 128>(L, pool, k, v, n, page0, npages, st)
                      : append_t<uint16_t, 64>(L, pool, k, v, n, page0, npages, st);
  return L.D == 128 ? append_t<float, 128>(L, pool, k, v, n, page0, npages, st)
                    : append_t<float, 64>(L, pool, k, v, n, page0, npages, st);
}

hipError_t launch_gather(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                         hipStream_t st) {
  if (ntok == 0) return hipSuccess;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? gather_t<uint16_t, 128>(L, pool, t, ntok, kout, vout, st)
                      : gather_t<uint16_t, 64>(L, pool, t, ntok, kout, vout, st);
  return L.D == 128 ? gather_t<float, 128>(L, pool, t, ntok, kout, vout, st)
                    : gather_t<float, 64>(L, pool, t, ntok, kout, vout, st);
}

}  // namespace sr
