// KV-cache kernels: pool zeroing, chunk append (K rows + V transposed into pages), gather.
// These are HBM-bound copies; the append writes exactly the layout the attention kernel
// reads (StreamRender-H3 project page, "3.3 Inference Acceleration and End-to-End
// Deployment", persistent KV layout), so no repacking happens at attention time.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sr {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte piece

__global__ __launch_bounds__(256) void zero_kernel(u32x4_t* __restrict__ p, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = u32x4_t{0, 0, 0, 0};
}

constexpr int kAppendTokens = 64;  // tokens per workgroup (half a page)

// Page layout (one head, one page of 128 tokens), with E = 16 / sizeof(T) elements per
// 16-byte piece:
//   K  element (token t, feature d) at ((d / E) * 128 + row_pos(t)) * E + d % E
//   V  element (token t, feature d) at ((t / E) * D + d) * E + t % E
// i.e. K is stored piece-column by piece-column with its 128 rows in the order the
// attention kernel's matrix operands want them (row_pos permutes rows inside each block of
// 32), and V is stored transposed, E consecutive tokens of one feature per piece.  A page
// is then copied into LDS as is, and every operand read is one 16-byte piece per lane with
// 32 lanes reading 512 contiguous bytes.
template <typename T>
__device__ __forceinline__ int row_pos(int t) {
  const int r = t & 31;
  if constexpr (sizeof(T) == 2) return (t & ~31) | (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
  return (t & ~31) | (8 * (r / 8) + 4 * (r % 2) + (r / 2) % 4);
}

// The 16-byte piece made of E elements of one LDS column (stride `pitch` elements).
__device__ __forceinline__ u32x4_t column_piece(const uint16_t* p, int pitch) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = unsigned(p[(2 * i) * pitch]) | (unsigned(p[(2 * i + 1) * pitch]) << 16);
  return w;
}
__device__ __forceinline__ u32x4_t column_piece(const float* p, int pitch) {
  return u32x4_t{__float_as_uint(p[0]), __float_as_uint(p[pitch]), __float_as_uint(p[2 * pitch]),
                 __float_as_uint(p[3 * pitch])};
}

// Workgroup (64-token half page, head).  Both K and V rows go through LDS (coalesced
// 16-byte reads along the features), then are written piece by piece in page order
// (coalesced 16-byte writes).  Tokens >= n are written as zeros.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(const T* __restrict__ k, const T* __restrict__ v, int n, int H,
                                                     T* __restrict__ kpool, T* __restrict__ vpool, int total_pages,
                                                     int page0) {
  constexpr int E = 16 / int(sizeof(T));  // elements per 16-byte piece
  constexpr int CPR = D / E;              // pieces per token row
  constexpr int PITCH = D + E;            // LDS row pitch (elements), padded by one piece
  __shared__ __align__(16) T ktile[kAppendTokens * PITCH];
  __shared__ __align__(16) T vtile[kAppendTokens * PITCH];

  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kAppendTokens;  // first token of this half page (slot-relative)
  const int tp = t0 % SR_PAGE_TOKENS;         // its position inside the page
  const size_t page = size_t(h) * total_pages + page0 + t0 / SR_PAGE_TOKENS;
  const u32x4_t z = {0, 0, 0, 0};

  for (int ci = threadIdx.x; ci < kAppendTokens * CPR; ci += blockDim.x) {
    const int r = ci / CPR, x = ci % CPR, t = t0 + r;
    const size_t src = (size_t(t) * H + h) * D + x * E;
    *reinterpret_cast<u32x4_t*>(ktile + r * PITCH + x * E) = t < n ? *reinterpret_cast<const u32x4_t*>(k + src) : z;
    *reinterpret_cast<u32x4_t*>(vtile + r * PITCH + x * E) = t < n ? *reinterpret_cast<const u32x4_t*>(v + src) : z;
  }
  __syncthreads();

  // K: piece x of row r goes to ((x * 128 + row_pos(tp + r)) * E); consecutive threads take
  // consecutive rows of one piece column.
  T* kpage = kpool + page * SR_PAGE_TOKENS * D;
  for (int ci = threadIdx.x; ci < kAppendTokens * CPR; ci += blockDim.x) {
    const int x = ci / kAppendTokens, r = ci % kAppendTokens;
    *reinterpret_cast<u32x4_t*>(kpage + (size_t(x) * SR_PAGE_TOKENS + row_pos<T>(tp + r)) * E) =
        *reinterpret_cast<const u32x4_t*>(ktile + r * PITCH + x * E);
  }
  // V: piece (token group g, feature d) holds tokens E*g .. E*g+E-1 of feature d.
  T* vpage = vpool + page * SR_PAGE_TOKENS * D;
  constexpr int GROUPS = kAppendTokens / E;
  for (int ci = threadIdx.x; ci < GROUPS * D; ci += blockDim.x) {
    const int g = ci / D, d = ci % D;
    *reinterpret_cast<u32x4_t*>(vpage + (size_t(tp / E + g) * D + d) * E) = column_piece(vtile + g * E * PITCH + d, PITCH);
  }
}

// Thread per (token, feature).  Test/debug path; not tuned.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ kpool, const T* __restrict__ vpool,
                                                     SegTable tab, int total_pages, int H, int ntok,
                                                     T* __restrict__ kout, T* __restrict__ vout) {
  constexpr int E = 16 / int(sizeof(T));
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
    const int tp = off % SR_PAGE_TOKENS;
    const T* kpage = kpool + page * SR_PAGE_TOKENS * D;
    const T* vpage = vpool + page * SR_PAGE_TOKENS * D;
    kout[(size_t(t) * H + h) * D + d] = kpage[(size_t(d / E) * SR_PAGE_TOKENS + row_pos<T>(tp)) * E + d % E];
    vout[(size_t(t) * H + h) * D + d] = vpage[(size_t(tp / E) * D + d) * E + tp % E];
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
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<u32x4_t*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_append(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0,
                         int32_t npages, hipStream_t st) {
  if (npages == 0) return hipSuccess;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? append_t<uint16_t, 128>(L, pool, k, v, n, page0, npages, st)
                      : append_t<uint16_t, 64>(L, pool, k, v, n, page0, npages, st);
  return append_t<float, 64>(L, pool, k, v, n, page0, npages, st);
}

hipError_t launch_gather(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                         hipStream_t st) {
  if (ntok == 0) return hipSuccess;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? gather_t<uint16_t, 128>(L, pool, t, ntok, kout, vout, st)
                      : gather_t<uint16_t, 64>(L, pool, t, ntok, kout, vout, st);
  return gather_t<float, 64>(L, pool, t, ntok, kout, vout, st);
}

}  // namespace sr
