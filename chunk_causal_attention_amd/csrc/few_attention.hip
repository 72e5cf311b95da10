// Split-K attention of a few query rows over the paged cache, for gfx950 (MI355X).
//
// The streaming decoder's global tokens (StreamRender-H3 project page, "3.2 Fast Causal H3
// VAE": four register tokens and a class token attend to the whole frame, iteration 4; their
// attention became a split-K kernel, iteration 6) are a handful of query rows per head over
// thousands of keys.  That is far too few rows for the chunk-attention kernel's 256-row query
// tiles, and the work is a single pass over the chunk's K and V: every byte is used by those
// few rows only, so the call is bound by HBM, not by the matrix units.
//
// Decomposition.  Wave w of workgroup (head h, piece p) takes half a cache page -- keys
// [64 (w % 2), 64 (w % 2) + 64) of page 4p + w / 2 of the head's key list -- with all the query
// rows (at most 32) as the columns of the 32x32 matrix instructions.  Its K and V operands are
// read straight from HBM into registers (each byte once, 32 lanes reading 512 contiguous
// bytes): the page layout is the one the chunk-attention kernel reads from LDS, K rows in
// operand order and V transposed, so the score registers of a lane are the P operand as they
// stand.  A wave computes S^T = K Q^T, the probabilities against its own row max, and
// O^T = V^T P^T; the eight waves (four pages) are merged in LDS into one record per workgroup
// (row max, row sum, unnormalised O of the valid rows): four pages per record rather than two
// halve the records that each head's merge loads, whose rate sets the kernel's tail.  The last workgroup of a head to arrive merges the
// head's records in piece order -- the result does not depend on the order of arrival -- and
// writes the output and the log-sum-exp.
//
// Records and arrival counters live in the attention workspace; they are stored and loaded
// with device-scope relaxed atomics, which gfx950 performs at the device's coherence point, and
// every wave waits for its record stores before the barrier that precedes the arrival.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMasked = -1.0e30f;  // score of a key past the segment; also the empty-wave max
constexpr int kWaves = 8;            // waves per workgroup: half a page each
constexpr int kPagesPerGroup = kWaves / 2;
constexpr int kPad = 33;             // LDS row pitch (floats) of the wave-merge buffer

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1])));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, unsigned(r[0])) + __builtin_bit_cast(float, unsigned(r[1]));
}

// Maximum and sum over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ void rec_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rec_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every vector memory operation of this wave (the record stores included) has completed.
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct FewArgs {
  const uint16_t* q;  // [n_q][H][D]
  uint16_t* o;        // [n_q][H][D]
  float* lse;         // [H][n_q] or null
  const char* kpool;
  const char* vpool;
  int32_t n_q, H, total_pages;
  int32_t npages;     // pages of the key list (segments in order)
  int32_t pieces;     // workgroups per head: ceil(npages / kPagesPerGroup)
  int32_t stride;     // floats per record: 64 + n_q * D
  float scale_log2;
  float* rec;         // H * pieces records
  int32_t* cnt;       // H arrival counters, zero between calls
  SegTable t;
};

template <int D>
__global__ __launch_bounds__(kWaves * 64) void few_attention_kernel(const FewArgs a) {
  constexpr int KS = D / 16;   // contraction slices of K Q^T
  constexpr int NDB = D / 32;  // 32-feature blocks of O^T
  constexpr int PAGE = SR_PAGE_TOKENS * D * 2;
  __shared__ float obuf[kWaves * D * kPad];  // wave merge; then the head merge's weights
  __shared__ float wm[kWaves][32], wl[kWaves][32];
  __shared__ float mq[32], lq[32];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int c = lane & 31, hl = lane >> 5;
  const int h = uniform(int(blockIdx.x) / a.pieces);
  const int piece = uniform(int(blockIdx.x) - h * a.pieces);
  const int pi = kPagesPerGroup * piece + (wave >> 1), half = wave & 1;

  // Page pi of the key list: its pool page and the valid keys of this wave's half.
  int page = 0, valid = 0;
  if (pi < a.npages) {
    int s = 0, first = 0;
    for (; s < a.t.n - 1; ++s) {
      const int np = (a.t.s[s].len + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
      if (pi < first + np) break;
      first += np;
    }
    const int off = pi - first;
    page = a.t.s[s].page + off;
    valid = min(a.t.s[s].len - off * SR_PAGE_TOKENS - 64 * half, 64);
  }
  page = uniform(page);
  valid = uniform(max(valid, 0));

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
  float m = kMasked, l = 0.0f;
  if (valid > 0) {
    const size_t base = (size_t(h) * a.total_pages + page) * PAGE;
    const char* kp = a.kpool + base;
    const char* vp = a.vpool + base;
    // Operands: K rows 64 half + 32 kb + c, feature piece 2 ks + hl; V^T rows 32 db + c, key
    // piece 8 half + 2 sl + hl; query row c (zero past n_q), features 16 ks + 8 hl ...
    bf16x8_t ka[2][KS], va[4][NDB], qo[KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[kb][ks] = *reinterpret_cast<const bf16x8_t*>(
            kp + size_t((2 * ks + hl) * SR_PAGE_TOKENS + 64 * half + 32 * kb + c) * 16);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        va[sl][db] = *reinterpret_cast<const bf16x8_t*>(vp + size_t((8 * half + 2 * sl + hl) * D + 32 * db + c) * 16);
    const bool qok = c < a.n_q;
    const uint16_t* qs = a.q + (size_t(qok ? c : 0) * a.H + h) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qo[ks] = qok ? *reinterpret_cast<const bf16x8_t*>(qs + 16 * ks) : bf16x8_t{};

    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], qo[ks], s[kb], 0, 0, 0);
    }
    // Register i of lane half hl in block kb holds key 32 kb + 16 (i / 8) + 8 hl + i % 8 (the
    // cache's row order); keys from `valid` on are masked.
    float mx = kMasked;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 16 * (i / 8) + 8 * hl + (i % 8);
        const float x = key < valid ? s[kb][i] * a.scale_log2 : kMasked;
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    m = pair_max(mx);  // key 0 is valid: m is a score
    bf16x8_t p[4];
    float ls = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      f32x8_t t;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * sl + 8 * hl + e;
        t[e] = key < valid ? __builtin_amdgcn_exp2f(s[sl >> 1][8 * (sl & 1) + e] - m) : 0.0f;
      }
      p[sl] = __builtin_convertvector(t, bf16x8_t);  // round to nearest even
#pragma unroll
      for (int e = 0; e < 8; ++e) ls += float(p[sl][e]);  // the sum of what P.V multiplies
    }
    l = pair_sum(ls);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[sl][db], p[sl], o[db], 0, 0, 0);
  }

  // Merge the eight waves: rescale to the workgroup's row max, sum in LDS.
  if (hl == 0) {
    wm[wave][c] = m;
    wl[wave][c] = l;
  }
  __syncthreads();
  float mw = wm[0][c];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mw = fmaxf(mw, wm[w][c]);
  const float f = __builtin_amdgcn_exp2f(m - mw);  // 0 for a wave without keys
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      obuf[(wave * D + 32 * db + 8 * (i / 4) + 4 * hl + (i % 4)) * kPad + c] = o[db][i] * f;
  __syncthreads();
  const int n_q = a.n_q;
  float* rec = a.rec + size_t(h * a.pieces + piece) * a.stride;
  if (tid < n_q) {
    float mm = wm[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, wm[w][tid]);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ll += wl[w][tid] * __builtin_amdgcn_exp2f(wm[w][tid] - mm);
    rec_store(rec + tid, mm);
    rec_store(rec + 32 + tid, ll);
  }
  for (int j = tid; j < n_q * D; j += kWaves * 64) {
    const int q = j / D, d = j - q * D;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += obuf[(w * D + d) * kPad + q];
    rec_store(rec + 64 + j, acc);
  }
  wait_memory();
  __syncthreads();
  if (tid == 0) {
    int32_t* cnt = a.cnt + h;
    const int arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = arrived == a.pieces - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag = last ? 1 : 0;
  }
  __syncthreads();
  if (flag == 0) return;

  // The head's last workgroup: weights 2^(m_p - M) / L of every (piece, row), then O.
  const float* head_rec = a.rec + size_t(h) * a.pieces * a.stride;
  const int np = a.pieces * n_q;  // the host keeps 2 np within obuf
  float* wmax = obuf;
  float* wsum = obuf + np;
  for (int j = tid; j < np; j += kWaves * 64) {
    const int p = j / n_q, q = j - p * n_q;
    wmax[j] = rec_load(head_rec + size_t(p) * a.stride + q);
    wsum[j] = rec_load(head_rec + size_t(p) * a.stride + 32 + q);
  }
  __syncthreads();
  // Row q's maximum and sum over the pieces by wave q % 4, its lanes taking the pieces; then
  // the weights of the row's pieces.
  for (int q = wave; q < n_q; q += kWaves) {
    float mm = kMasked;
    for (int p = lane; p < a.pieces; p += 64) mm = fmaxf(mm, wmax[p * n_q + q]);
    mm = wave_max(mm);
    float ll = 0.0f;
    for (int p = lane; p < a.pieces; p += 64) ll += wsum[p * n_q + q] * __builtin_amdgcn_exp2f(wmax[p * n_q + q] - mm);
    ll = wave_sum(ll);
    for (int p = lane; p < a.pieces; p += 64) wmax[p * n_q + q] = __builtin_amdgcn_exp2f(wmax[p * n_q + q] - mm) / ll;
    if (lane == 0) {
      mq[q] = mm;
      lq[q] = ll;
    }
  }
  __syncthreads();
  // Up to 32 records' loads in flight at a time, so a head of up to 64 pages takes one round
  // trip per output element (pieces past the last: weight 0, last record reread).
  constexpr int U = 32;
  for (int j = tid; j < n_q * D; j += kWaves * 64) {
    const int q = j / D, d = j - q * D;
    float acc = 0.0f;
    for (int p0 = 0; p0 < a.pieces; p0 += U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = rec_load(head_rec + size_t(min(p0 + u, a.pieces - 1)) * a.stride + 64 + j);
#pragma unroll
      for (int u = 0; u < U; ++u) acc += (p0 + u < a.pieces ? wmax[(p0 + u) * n_q + q] : 0.0f) * x[u];
    }
    const __bf16 r = __bf16(acc);
    a.o[(size_t(q) * a.H + h) * D + d] = __builtin_bit_cast(uint16_t, r);
  }
  if (a.lse && tid < n_q) a.lse[size_t(h) * n_q + tid] = (mq[tid] + __log2f(lq[tid])) * kLn2;
}

}  // namespace

int64_t few_attention_record_floats(const Layout& L, const SegTable& t, int32_t n_q) {
  int64_t npages = 0;
  for (int s = 0; s < t.n; ++s) npages += (t.s[s].len + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
  const int64_t pieces = (npages + kPagesPerGroup - 1) / kPagesPerGroup;
  return int64_t(L.H) * pieces * (64 + int64_t(n_q) * L.D);
}

bool few_attention_shape_ok(const Layout& L, const SegTable& t, int32_t n_q) {
  if (L.dtype != SR_BF16 || (L.D != 64 && L.D != 128) || n_q < 1 || n_q > kFewRows) return false;
  int64_t npages = 0;
  for (int s = 0; s < t.n; ++s) npages += (t.s[s].len + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
  const int64_t pieces = (npages + kPagesPerGroup - 1) / kPagesPerGroup;
  return npages > 0 && 2 * pieces * n_q <= int64_t(kWaves) * L.D * kPad;
}

bool few_attention_fits(const Layout& L, const SegTable& t, int32_t n_q, const SplitWorkspace& ws) {
  if (ws.cus_per_xcd <= 0 || !few_attention_shape_ok(L, t, n_q)) return false;
  const int64_t have = int64_t(8) * kMaxPieces * ws.cus_per_xcd * attn_record_floats(L.D);  // the records area
  return L.H <= 8 * ws.cus_per_xcd && few_attention_record_floats(L, t, n_q) <= have;
}

hipError_t launch_few_attention(const Layout& L, const void* pool, const SegTable& t, int32_t n_q, const void* q,
                                void* o, float* lse, float softmax_scale, const SplitWorkspace& ws, hipStream_t st) {
  FewArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.kpool = static_cast<const char*>(pool);
  a.vpool = static_cast<const char*>(pool) + L.half_bytes;
  a.n_q = n_q;
  a.H = L.H;
  a.total_pages = L.total_pages;
  a.npages = 0;
  for (int s = 0; s < t.n; ++s) a.npages += (t.s[s].len + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
  a.pieces = (a.npages + kPagesPerGroup - 1) / kPagesPerGroup;
  a.stride = 64 + n_q * L.D;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.rec = ws.records;
  a.cnt = ws.counters;
  a.t = t;
  const dim3 grid(L.H * a.pieces), block(kWaves * 64);
  if (L.D == 128)
    hipLaunchKernelGGL(few_attention_kernel<128>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(few_attention_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace sr
