// KV-cache kernels: pool zeroing, chunk append (K rows + V transposed into pages), gather.
// These are HBM-bound copies; the append writes exactly the layout the attention kernel
// reads (StreamRender-H3 project page, "3.3 Inference Acceleration and End-to-End
// Deployment", persistent KV layout), so no repacking happens at attention time.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "mx_codec.hpp"

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

// One workgroup's share of an append (256 threads): half page `half` (64 tokens) of head h.
// Both K and V rows go through LDS (coalesced 16-byte reads along the features), then are
// written piece by piece in page order (coalesced 16-byte writes).  Tokens >= n are written as
// zeros.
template <typename T, int D>
__device__ __forceinline__ void append_half_page(const T* __restrict__ k, const T* __restrict__ v, int n, int H,
                                                 T* __restrict__ kpool, T* __restrict__ vpool, int total_pages,
                                                 int page0, int half, int h) {
  constexpr int E = 16 / int(sizeof(T));  // elements per 16-byte piece
  constexpr int CPR = D / E;              // pieces per token row
  constexpr int PITCH = D + E;            // LDS row pitch (elements), padded by one piece
  __shared__ __align__(16) T ktile[kAppendTokens * PITCH];
  __shared__ __align__(16) T vtile[kAppendTokens * PITCH];

  const int t0 = half * kAppendTokens;        // first token of this half page (slot-relative)
  const int tp = t0 % SR_PAGE_TOKENS;         // its position inside the page
  const size_t page = size_t(h) * total_pages + page0 + t0 / SR_PAGE_TOKENS;
  const u32x4_t z = {0, 0, 0, 0};

  // All IT row pieces of a thread (256 threads) are requested before the first is stored.
  static_assert((kAppendTokens * CPR) % 256 == 0, "whole rounds of 256 threads");
  constexpr int IT = kAppendTokens * CPR / 256;
  u32x4_t wk[IT], wv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int ci = threadIdx.x + it * 256, r = ci / CPR, x = ci % CPR, t = t0 + r;
    const size_t src = (size_t(t) * H + h) * D + x * E;
    wk[it] = t < n ? *reinterpret_cast<const u32x4_t*>(k + src) : z;
    wv[it] = t < n ? *reinterpret_cast<const u32x4_t*>(v + src) : z;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int ci = threadIdx.x + it * 256, r = ci / CPR, x = ci % CPR;
    *reinterpret_cast<u32x4_t*>(ktile + r * PITCH + x * E) = wk[it];
    *reinterpret_cast<u32x4_t*>(vtile + r * PITCH + x * E) = wv[it];
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

// Workgroup (64-token half page, head) of one contiguous run of tokens.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(const T* __restrict__ k, const T* __restrict__ v, int n, int H,
                                                     T* __restrict__ kpool, T* __restrict__ vpool, int total_pages,
                                                     int page0) {
  append_half_page<T, D>(k, v, n, H, kpool, vpool, total_pages, page0, blockIdx.x, blockIdx.y);
}

// Workgroup (window, 64-token half page of its pages, head) of a chunk packed window by window
// (WinView): window w's rows [row0[w], row0[w+1]) go to its pages page0 + w * pages ...
template <typename T, int D>
__global__ __launch_bounds__(256) void append_windows_kernel(const T* __restrict__ k, const T* __restrict__ v, int H,
                                                             T* __restrict__ kpool, T* __restrict__ vpool,
                                                             int total_pages, int page0, WinView win) {
  const int halves = win.pages * (SR_PAGE_TOKENS / kAppendTokens);
  const int w = blockIdx.x / halves, half = blockIdx.x % halves;
  const size_t off = size_t(win.row0[w]) * H * D;
  append_half_page<T, D>(k + off, v + off, win.row0[w + 1] - win.row0[w], H, kpool, vpool, total_pages,
                         page0 + w * win.pages, half, blockIdx.y);
}

// ---- fused qk-RMSNorm + rotary embedding + cache write ---------------------------------
// StreamRender-H3 project page, "3.2 Fast Causal H3 VAE": after the qkv projection, qk-norm,
// the rotary embedding and the K/V cache write run as one kernel (iteration 6); each token
// gets its rotary position once, when it is written (inference items), at its stream-absolute
// position (iteration 4).  Per (token, head): y = x / sqrt(mean(x^2) + eps) * gain, then
// rotation pair j = (y_2j, y_2j+1) turns by pos[axis_j] * theta_j.

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

// The E values of one 16-byte piece, widened to fp32, and back (round to nearest even).
__device__ __forceinline__ void widen_piece(const u32x4_t& w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen_piece(const u32x4_t& w, float (&f)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ unsigned bf16_rne(float x) {
  const unsigned u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN -> quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ u32x4_t narrow_piece(const float (&f)[8]) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_rne(f[2 * i]) | (bf16_rne(f[2 * i + 1]) << 16);
  return w;
}
__device__ __forceinline__ u32x4_t narrow_piece(const float (&f)[4]) {
  return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// RMS-normalises and rotates one piece (features x*E .. x*E+E-1) of one (token, head) row;
// the CPR lanes holding the pieces of the row are consecutive and reduce together.  gain holds
// the piece's E gains, cs the row's (cos, sin) per rotation pair.
template <int E, int CPR, int D>
__device__ __forceinline__ void prep_piece(float (&f)[E], int x, const float (&gain)[E], float eps,
                                           const float2* cs) {
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
#pragma unroll
  for (int m = CPR / 2; m >= 1; m /= 2) ss += __shfl_xor(ss, m, CPR);
  const float scale = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int e = 0; e < E; ++e) f[e] = f[e] * scale * gain[e];
#pragma unroll
  for (int e = 0; e < E; e += 2) {
    const float2 r = cs[(x * E + e) / 2];
    const float a = f[e], b = f[e + 1];
    f[e] = a * r.x - b * r.y;
    f[e + 1] = a * r.y + b * r.x;
  }
}

constexpr int kPrepHeads = 4;  // heads per workgroup of the fused append (they share the rotations)

// Workgroup (64-token half page, kPrepHeads heads); qkv [n][3][H][D], positions [n][3].  The
// (cos, sin) of every (token, rotation pair) of the tile is computed once, into LDS: the angle
// pos * theta in fp64, reduced to [-pi, pi], then the fp32 sine and cosine.  Per head, Q goes
// straight to q_out; normalised, rotated K and plain V go through LDS into the page, as in
// append_kernel.  A thread always holds the same feature piece x (256 is a multiple of the D / E
// pieces of a row), so its gains sit in registers for the whole kernel, and all IT of a head's
// row pieces it handles are requested before the first is used: one memory round trip per head
// instead of one (plus one for the gains) per piece.
template <typename T, int D>
__global__ __launch_bounds__(256) void prep_append_kernel(const T* __restrict__ qkv, const int32_t* __restrict__ pos,
                                                          int n, int H, const float* __restrict__ gq,
                                                          const float* __restrict__ gk, float eps, RopeTable rt,
                                                          T* __restrict__ qout, T* __restrict__ kpool,
                                                          T* __restrict__ vpool, int total_pages, int page0) {
  constexpr int E = 16 / int(sizeof(T));
  constexpr int CPR = D / E;
  constexpr int PITCH = D + E;
  constexpr int NP = D / 2;          // rotation pairs
  constexpr int CSP = NP + 1;        // LDS pitch of a token's rotation row (float2), padded
  static_assert(64 % CPR == 0, "the lanes of one row stay inside a wave");
  __shared__ __align__(16) T ktile[kAppendTokens * PITCH];
  __shared__ __align__(16) T vtile[kAppendTokens * PITCH];
  __shared__ float2 rot[kAppendTokens * CSP];

  static_assert(256 % CPR == 0 && (kAppendTokens * CPR) % 256 == 0, "a thread keeps its feature piece");
  constexpr int IT = kAppendTokens * CPR / 256;  // row pieces per thread and head
  const int t0 = blockIdx.x * kAppendTokens;
  const int tp = t0 % SR_PAGE_TOKENS;
  const u32x4_t z = {0, 0, 0, 0};
  const size_t hd = size_t(H) * D;
  const int x = threadIdx.x % CPR;
  float gqr[E], gkr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gqr[e] = gq[x * E + e];
    gkr[e] = gk[x * E + e];
  }

  for (int i = threadIdx.x; i < kAppendTokens * NP; i += blockDim.x) {
    const int r = i / NP, j = i % NP, t = t0 + r;
    const int p = t < n ? pos[size_t(t) * 3 + rt.axis[j]] : 0;
    const double ang = double(p) * rt.theta[j];
    const double red = ang - 6.283185307179586 * __builtin_rint(ang * 0.15915494309189535);
    float sn, cs;
    sincosf(float(red), &sn, &cs);
    rot[r * CSP + j] = make_float2(cs, sn);
  }
  __syncthreads();

  for (int hh = 0; hh < kPrepHeads; ++hh) {
    const int h = blockIdx.y * kPrepHeads + hh;
    if (h >= H) break;  // uniform
    const size_t page = size_t(h) * total_pages + page0 + t0 / SR_PAGE_TOKENS;
    // Every lane of a row group runs the reduction, also for rows past n (their values are
    // zero and their results are dropped).
    u32x4_t wq[IT], wk[IT], wv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (threadIdx.x + it * 256) / CPR, t = t0 + r;
      const bool ok = t < n;
      const size_t src = (size_t(ok ? t : 0) * 3 * H + h) * D + x * E;
      wq[it] = ok ? *reinterpret_cast<const u32x4_t*>(qkv + src) : z;
      wk[it] = ok ? *reinterpret_cast<const u32x4_t*>(qkv + src + hd) : z;
      wv[it] = ok ? *reinterpret_cast<const u32x4_t*>(qkv + src + 2 * hd) : z;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (threadIdx.x + it * 256) / CPR, t = t0 + r;
      const bool ok = t < n;
      float fq[E], fk[E];
      widen_piece(wq[it], fq);
      widen_piece(wk[it], fk);
      prep_piece<E, CPR, D>(fq, x, gqr, eps, rot + r * CSP);
      prep_piece<E, CPR, D>(fk, x, gkr, eps, rot + r * CSP);
      if (ok) *reinterpret_cast<u32x4_t*>(qout + (size_t(t) * H + h) * D + x * E) = narrow_piece(fq);
      *reinterpret_cast<u32x4_t*>(ktile + r * PITCH + x * E) = ok ? narrow_piece(fk) : z;
      *reinterpret_cast<u32x4_t*>(vtile + r * PITCH + x * E) = wv[it];
    }
    __syncthreads();
    T* kpage = kpool + page * SR_PAGE_TOKENS * D;
    for (int ci = threadIdx.x; ci < kAppendTokens * CPR; ci += blockDim.x) {
      const int x = ci / kAppendTokens, r = ci % kAppendTokens;
      *reinterpret_cast<u32x4_t*>(kpage + (size_t(x) * SR_PAGE_TOKENS + row_pos<T>(tp + r)) * E) =
          *reinterpret_cast<const u32x4_t*>(ktile + r * PITCH + x * E);
    }
    T* vpage = vpool + page * SR_PAGE_TOKENS * D;
    constexpr int GROUPS = kAppendTokens / E;
    for (int ci = threadIdx.x; ci < GROUPS * D; ci += blockDim.x) {
      const int g = ci / D, d = ci % D;
      *reinterpret_cast<u32x4_t*>(vpage + (size_t(tp / E + g) * D + d) * E) =
          column_piece(vtile + g * E * PITCH + d, PITCH);
    }
    __syncthreads();  // the tiles are refilled for the next head
  }
}

// Page (relative to the head's first page) and in-page token of token `off` of segment s; for a
// windowed chunk segment (s >= win.bank_segs in window mode) `off` is a packed row.
__device__ __forceinline__ int2 seg_token(const SegTable& tab, const WinView& win, int s, int off) {
  int page = tab.s[s].page;
  if (win.n > 0 && s >= win.bank_segs) {
    int w = 0;
    while (w + 1 < win.n && off >= win.row0[w + 1]) ++w;
    off -= win.row0[w];
    page += w * win.pages;
  }
  return make_int2(page + off / SR_PAGE_TOKENS, off % SR_PAGE_TOKENS);
}

// Thread per (token, feature).  Test/debug path; not tuned.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ kpool, const T* __restrict__ vpool,
                                                     SegTable tab, WinView win, int total_pages, int H, int ntok,
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
    const int2 pt = seg_token(tab, win, s, off);
    const size_t page = size_t(h) * total_pages + pt.x;
    const int tp = pt.y;
    const T* kpage = kpool + page * SR_PAGE_TOKENS * D;
    const T* vpage = vpool + page * SR_PAGE_TOKENS * D;
    kout[(size_t(t) * H + h) * D + d] = kpage[(size_t(d / E) * SR_PAGE_TOKENS + row_pos<T>(tp)) * E + d % E];
    vout[(size_t(t) * H + h) * D + d] = vpage[(size_t(tp / E) * D + d) * E + tp % E];
  }
}

// ---- reduced-precision (SR_MX) pages -------------------------------------------------
// "The road to the fastest, cheapest H3", Accelerating the denoiser, item 2: MXFP6 keys and
// FP8 values.  K page of one head (NB = D / 32 blocks per token): block b of token t packs 32
// E2M3 codes into 24 bytes, bytes 0-15 in the "lo" region at (b * 128 + t) * 16 and bytes
// 16-23 in the "hi" region at NB * 2048 + (b * 128 + t) * 8, so that one matrix operand
// (a key row's block) is a 16-byte and an 8-byte read and 32 lanes read contiguous memory;
// the scale bytes of token t follow at NB * 3072 + t * NB, block b at (b % 2) * NB / 2 + b / 2
// (the byte that lane half b % 2 selects in contraction step b / 2).  V page: byte
// (g * D + d) * 16 + i holds feature d of token t with r = t % 32,
// g = 4 * (t / 64) + 2 * ((t / 32) % 2) + (r / 4) % 2 and i = 4 * (r / 8) + r % 4: the 16
// tokens whose probabilities one lane half holds after the score instruction, in register
// order, so the P.V operand of a lane is two 16-byte reads.
template <int D>
struct MxPage {
  static constexpr int NB = D / 32;
  static constexpr int LO = 0;
  static constexpr int HI = NB * SR_PAGE_TOKENS * 16;
  static constexpr int SC = HI + NB * SR_PAGE_TOKENS * 8;
  static constexpr int KBYTES = int(mx_kpage_bytes(D));  // SC + NB * 128, padded to whole KiB
  static constexpr int VBYTES = D * SR_PAGE_TOKENS;
  static_assert(KBYTES >= SC + NB * SR_PAGE_TOKENS && VBYTES == int(mx_vpage_bytes(D)), "page sizes shared with the host");
  static constexpr int scale_pos(int b) { return (b % 2) * (NB / 2) + b / 2; }
};

// Byte of token tp (0..127) of feature d in a V page.
template <int D>
__host__ __device__ __forceinline__ int mx_v_offset(int tp, int d) {
  const int r = tp & 31;
  const int g = 4 * (tp >> 6) + 2 * ((tp >> 5) & 1) + ((r >> 2) & 1);
  return (g * D + d) * 16 + 4 * (r >> 3) + (r & 3);
}

// Workgroup (64-token half page, head).  K: one thread per (block, token) quantizes its 32
// features and writes its lo/hi pieces (a wave covers 64 consecutive rows of one block:
// contiguous writes); the scale bytes are collected in LDS and written as dwords.  V: staged
// in LDS like append_kernel, then one thread per 16-byte piece (group, feature) converts and
// packs 16 tokens.  Tokens >= n are written as zeros (codes 0, scale byte 0).
template <int D>
__global__ __launch_bounds__(256) void mx_append_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        int n, int H, char* __restrict__ kpool,
                                                        char* __restrict__ vpool, int total_pages, int page0) {
  using Pg = MxPage<D>;
  constexpr int NB = Pg::NB;
  constexpr int CPR = D / 8;     // 16-byte pieces per bf16 row
  constexpr int PITCH = D + 8;   // LDS row pitch (elements)
  __shared__ __align__(16) uint16_t vtile[kAppendTokens * PITCH];
  __shared__ __align__(4) uint8_t scales[kAppendTokens * NB];

  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kAppendTokens;
  const int tp = t0 % SR_PAGE_TOKENS;
  const size_t page = size_t(h) * total_pages + page0 + t0 / SR_PAGE_TOKENS;
  char* kp = kpool + page * Pg::KBYTES;
  char* vp = vpool + page * Pg::VBYTES;
  const u32x4_t z = {0, 0, 0, 0};

  for (int ci = threadIdx.x; ci < NB * kAppendTokens; ci += blockDim.x) {
    const int b = ci / kAppendTokens, r = ci % kAppendTokens, t = t0 + r;
    unsigned xs[32];
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(k + (size_t(t < n ? t : 0) * H + h) * D + b * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t w = t < n ? src[j] : z;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[8 * j + 2 * i] = w[i] & 0xFFFFu;
        xs[8 * j + 2 * i + 1] = w[i] >> 16;
      }
    }
    unsigned w[6];
    const int X = mx::quantize_block(xs, w);
    const int row = tp + r;
    *reinterpret_cast<u32x4_t*>(kp + Pg::LO + (b * SR_PAGE_TOKENS + row) * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<uint2*>(kp + Pg::HI + (b * SR_PAGE_TOKENS + row) * 8) = make_uint2(w[4], w[5]);
    scales[r * NB + Pg::scale_pos(b)] = uint8_t(X + 127);
  }
  for (int ci = threadIdx.x; ci < kAppendTokens * CPR; ci += blockDim.x) {
    const int r = ci / CPR, x = ci % CPR, t = t0 + r;
    *reinterpret_cast<u32x4_t*>(vtile + r * PITCH + x * 8) =
        t < n ? *reinterpret_cast<const u32x4_t*>(v + (size_t(t) * H + h) * D + x * 8) : z;
  }
  __syncthreads();
  for (int ci = threadIdx.x; ci < kAppendTokens * NB / 4; ci += blockDim.x)
    *reinterpret_cast<uint32_t*>(kp + Pg::SC + tp * NB + ci * 4) = reinterpret_cast<const uint32_t*>(scales)[ci];
  // V pieces of this half page: groups 4 * (tp / 64) + gl, gl = 2 * kb + hl.
  for (int ci = threadIdx.x; ci < 4 * D; ci += blockDim.x) {
    const int gl = ci / D, d = ci % D, kb = gl >> 1, hl = gl & 1;
    u32x4_t piece;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e;                                    // byte of the piece
        const int r = 8 * (i >> 2) + 4 * hl + (i & 3);              // token inside the 32-block
        word |= mx::e4m3_code(vtile[(kb * 32 + r) * PITCH + d]) << (8 * e);
      }
      piece[q] = word;
    }
    *reinterpret_cast<u32x4_t*>(vp + ((4 * (tp >> 6) + gl) * D + d) * 16) = piece;
  }
}

// Thread per (token, feature): the dequantized values as bf16.  Test/debug path; not tuned.
template <int D>
__global__ __launch_bounds__(256) void mx_gather_kernel(const char* __restrict__ kpool, const char* __restrict__ vpool,
                                                        SegTable tab, int total_pages, int H, int ntok,
                                                        uint16_t* __restrict__ kout, uint16_t* __restrict__ vout) {
  using Pg = MxPage<D>;
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
    const char* kp = kpool + page * Pg::KBYTES;
    const int b = d / 32, e = d % 32;
    const uint32_t* lo = reinterpret_cast<const uint32_t*>(kp + Pg::LO + (b * SR_PAGE_TOKENS + tp) * 16);
    const uint32_t* hi = reinterpret_cast<const uint32_t*>(kp + Pg::HI + (b * SR_PAGE_TOKENS + tp) * 8);
    const int bit = 6 * e, word = bit >> 5, sh = bit & 31;
    auto wd = [&](int i) { return i < 4 ? lo[i] : hi[i - 4]; };
    unsigned c = (wd(word) >> sh) & 63u;
    if (sh > 26) c |= (wd(word + 1) << (32 - sh)) & 63u;
    const int X = int(uint8_t(kp[Pg::SC + tp * Pg::NB + Pg::scale_pos(b)])) - 127;
    kout[(size_t(t) * H + h) * D + d] = uint16_t(mx::e2m3_to_bf16(c, X));
    const uint8_t vc = uint8_t(vpool[page * Pg::VBYTES + mx_v_offset<D>(tp, d)]);
    vout[(size_t(t) * H + h) * D + d] = uint16_t(mx::e4m3_to_bf16(vc));
  }
}

template <int D>
hipError_t mx_append_t(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0,
                       int32_t npages, hipStream_t st) {
  char* kpool = static_cast<char*>(pool);
  char* vpool = kpool + L.half_bytes;
  dim3 grid(npages * (SR_PAGE_TOKENS / kAppendTokens), L.H);
  hipLaunchKernelGGL((mx_append_kernel<D>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), n, L.H, kpool, vpool, L.total_pages, page0);
  return hipGetLastError();
}

template <int D>
hipError_t mx_gather_t(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                       hipStream_t st) {
  const char* kpool = static_cast<const char*>(pool);
  const char* vpool = kpool + L.half_bytes;
  dim3 grid((ntok + 63) / 64, L.H);
  hipLaunchKernelGGL((mx_gather_kernel<D>), grid, dim3(256), 0, st, kpool, vpool, t, L.total_pages, L.H, ntok,
                     static_cast<uint16_t*>(kout), static_cast<uint16_t*>(vout));
  return hipGetLastError();
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
hipError_t prep_append_t(const Layout& L, void* pool, const void* qkv, const int32_t* pos, int32_t n, const float* gq,
                         const float* gk, float eps, const RopeTable& rt, void* qout, int32_t page0, int32_t npages,
                         hipStream_t st) {
  T* kpool = static_cast<T*>(pool);
  T* vpool = reinterpret_cast<T*>(static_cast<char*>(pool) + L.half_bytes);
  dim3 grid(npages * (SR_PAGE_TOKENS / kAppendTokens), (L.H + kPrepHeads - 1) / kPrepHeads);
  hipLaunchKernelGGL((prep_append_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(qkv), pos, n, L.H,
                     gq, gk, eps, rt, static_cast<T*>(qout), kpool, vpool, L.total_pages, page0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t gather_t(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                    const WinView& win, hipStream_t st) {
  const T* kpool = static_cast<const T*>(pool);
  const T* vpool = reinterpret_cast<const T*>(static_cast<const char*>(pool) + L.half_bytes);
  dim3 grid((ntok + 63) / 64, L.H);
  hipLaunchKernelGGL((gather_kernel<T, D>), grid, dim3(256), 0, st, kpool, vpool, t, win, L.total_pages, L.H, ntok,
                     static_cast<T*>(kout), static_cast<T*>(vout));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t append_windows_t(const Layout& L, void* pool, const void* k, const void* v, const WinView& win,
                            int32_t page0, hipStream_t st) {
  T* kpool = static_cast<T*>(pool);
  T* vpool = reinterpret_cast<T*>(static_cast<char*>(pool) + L.half_bytes);
  dim3 grid(win.n * win.pages * (SR_PAGE_TOKENS / kAppendTokens), L.H);
  hipLaunchKernelGGL((append_windows_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(k),
                     static_cast<const T*>(v), L.H, kpool, vpool, L.total_pages, page0, win);
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
  if (L.dtype == SR_MX)
    return L.D == 128 ? mx_append_t<128>(L, pool, k, v, n, page0, npages, st)
                      : mx_append_t<64>(L, pool, k, v, n, page0, npages, st);
  if (L.dtype == SR_BF16)
    return L.D == 128 ? append_t<uint16_t, 128>(L, pool, k, v, n, page0, npages, st)
                      : append_t<uint16_t, 64>(L, pool, k, v, n, page0, npages, st);
  return append_t<float, 64>(L, pool, k, v, n, page0, npages, st);
}

hipError_t launch_prep_append(const Layout& L, void* pool, const void* qkv, const int32_t* pos, int32_t n,
                              const float* gq, const float* gk, float eps, const RopeTable& rt, void* qout,
                              int32_t page0, int32_t npages, hipStream_t st) {
  if (npages == 0) return hipSuccess;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? prep_append_t<uint16_t, 128>(L, pool, qkv, pos, n, gq, gk, eps, rt, qout, page0, npages, st)
                      : prep_append_t<uint16_t, 64>(L, pool, qkv, pos, n, gq, gk, eps, rt, qout, page0, npages, st);
  return prep_append_t<float, 64>(L, pool, qkv, pos, n, gq, gk, eps, rt, qout, page0, npages, st);
}

hipError_t launch_gather(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                         const WinView* win, hipStream_t st) {
  if (ntok == 0) return hipSuccess;
  if (L.dtype == SR_MX)  // windowed caches are bf16 / fp32 only (checked by the caller)
    return L.D == 128 ? mx_gather_t<128>(L, pool, t, ntok, kout, vout, st) : mx_gather_t<64>(L, pool, t, ntok, kout, vout, st);
  const WinView none{};
  const WinView& wv = win ? *win : none;
  if (L.dtype == SR_BF16)
    return L.D == 128 ? gather_t<uint16_t, 128>(L, pool, t, ntok, kout, vout, wv, st)
                      : gather_t<uint16_t, 64>(L, pool, t, ntok, kout, vout, wv, st);
  return gather_t<float, 64>(L, pool, t, ntok, kout, vout, wv, st);
}

hipError_t launch_append_windows(const Layout& L, void* pool, const void* k, const void* v, const WinView& win,
                                 int32_t page0, hipStream_t st) {
  if (L.dtype == SR_BF16)
    return L.D == 128 ? append_windows_t<uint16_t, 128>(L, pool, k, v, win, page0, st)
                      : append_windows_t<uint16_t, 64>(L, pool, k, v, win, page0, st);
  return append_windows_t<float, 64>(L, pool, k, v, win, page0, st);
}

}  // namespace sr
