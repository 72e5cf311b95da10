// Chunk-causal attention over the paged KV cache, for gfx950 (MI355X).
//
// Computes, per head and current-chunk query i, softmax attention over the keys of the
// persistent bank, the history chunks in the window and the current chunk up to i's causal
// block (StreamRender-H3 project page, "3.1.2 Historical Context and Temporal Consistency",
// prefix cache; "3.3 Inference Acceleration and End-to-End Deployment", static-context KV
// caching and persistent KV layout).
//
// Work decomposition.  One workgroup per (head, tile of BM = NW*QB*32 queries); each wave
// owns QB blocks of 32 queries for the whole key sequence.  The workgroup walks the key
// tiles of its segments in visiting order; tiles past the last visible causal block are
// never loaded.  Each tile (BN keys) is staged through LDS, double buffered: the next tile's
// global loads are issued before the current tile's math.
//
// Matrix instructions (32x32 output tile).  Scores are computed transposed, S^T = K . Q^T:
// the key block is the A operand, the queries are the B operand held in registers for the
// whole kernel, so lane (c, hl) of a wave owns query column c and row-wise reductions are
// in-lane plus one exchange with the other lane half.  The output P.V is also computed
// transposed, O^T += V^T . P^T, so the probabilities never leave the registers: K rows are
// written to LDS in a permuted row order chosen so that the score registers of a lane come
// out exactly in the operand order the P.V instruction expects, and V is stored transposed
// in the cache pages, so its operand is one contiguous LDS read per lane.
//
// Softmax in the exp2 domain with a lazily updated running max: O and l are rescaled only
// when some row's max grows by more than 2^8, otherwise the stale max is kept (exact in real
// arithmetic; probabilities stay below 2^8, far from fp32/bf16 overflow).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace sr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte piece

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kMaxInit = -1.0e30f;       // finite: keeps exp2(x - max) defined on masked rows

// Accumulator layout shared by the 32x32 instructions: lane 32*hl + c holds column c and,
// in register i, row 8*(i/4) + 4*hl + (i%4).
template <typename T>
struct Mma;

// bf16 inputs, fp32 accumulation: v_mfma_f32_32x32x16_bf16.  Operand lane (c, hl) holds
// row/column c and contraction indices 8*hl .. 8*hl+7.
template <>
struct Mma<uint16_t> {
  static constexpr int K = 16;
  static constexpr int EPL = 8;
  using Op = bf16x8_t;
  __device__ static f32x16_t mma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Key (inside a 32-key block) whose score lands in register i of lane half hl: the
  // registers 8*kq .. 8*kq+7 of a lane half are then the keys 16*kq + 8*hl + (0..7), which
  // is the P operand of contraction slice kq.
  __device__ static constexpr int key_of_reg(int i, int hl) { return 16 * (i / 8) + 8 * hl + (i % 8); }
  // LDS row that holds key r so that key_of_reg holds: swap bits 2 and 3 of r.
  __device__ static constexpr int row_of_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
  __device__ static Op load(const char* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static Op pack(const f32x16_t& s, int kq) {
    f32x8_t t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = s[8 * kq + e];
    return __builtin_convertvector(t, bf16x8_t);  // round to nearest even
  }
  __device__ static void store4(uint16_t* dst, f32x4_t v) {
    *reinterpret_cast<bf16x4_t*>(dst) = __builtin_convertvector(v, bf16x4_t);
  }
};

// fp32 inputs: v_mfma_f32_32x32x2_f32.  Operand lane (c, hl) holds row/column c and
// contraction index hl.
template <>
struct Mma<float> {
  static constexpr int K = 2;
  static constexpr int EPL = 1;
  using Op = float;
  __device__ static f32x16_t mma(Op a, Op b, f32x16_t c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
  // Register i of lane half hl holds key 2*i + hl: the P operand of slice kq is register kq.
  __device__ static constexpr int key_of_reg(int i, int hl) { return 2 * i + hl; }
  __device__ static constexpr int row_of_key(int r) { return 8 * (r / 8) + 4 * (r % 2) + (r / 2) % 4; }
  __device__ static Op load(const char* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static Op pack(const f32x16_t& s, int kq) { return s[kq]; }
  __device__ static void store4(float* dst, f32x4_t v) { *reinterpret_cast<f32x4_t*>(dst) = v; }
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  const char* kpool;
  const char* vpool;
  int32_t n_q, H, total_pages, causal_block;
  int32_t q_tiles, num_wg;
  float scale_log2;
  SegTable t;
};

// Registers holding one K/V tile between its global loads and its LDS stores.
template <int KCH, int VCH>
struct Stage {
  u32x4_t k[KCH];
  u32x4_t v[VCH];
};

// Issues the global loads of key tile (segment s, first key k0): BN key rows of K (contiguous
// in the page) and the BN-key slice of each of the D rows of the transposed V page.
template <typename T, int D, int BN, int NT, int KCH, int VCH>
__device__ __forceinline__ void load_tile(Stage<KCH, VCH>& st, const AttnArgs& a, size_t head_page, int s, int k0,
                                          int tid) {
  constexpr int ES = int(sizeof(T));
  constexpr int KPR = D * ES / 16;
  constexpr int VPR = BN * ES / 16;
  const size_t page = head_page + a.t.s[s].page + k0 / SR_PAGE_TOKENS;
  const char* kb = a.kpool + (page * SR_PAGE_TOKENS + k0 % SR_PAGE_TOKENS) * (D * ES);
  const char* vb = a.vpool + page * (D * SR_PAGE_TOKENS * ES) + (k0 % SR_PAGE_TOKENS) * ES;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int ci = j * NT + tid;
    st.k[j] = *reinterpret_cast<const u32x4_t*>(kb + (ci / KPR) * (D * ES) + (ci % KPR) * 16);
  }
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int ci = j * NT + tid;
    st.v[j] = *reinterpret_cast<const u32x4_t*>(vb + (ci / VPR) * (SR_PAGE_TOKENS * ES) + (ci % VPR) * 16);
  }
}

// Writes a staged tile into one LDS stage: K rows at their permuted positions (see
// Mma::row_of_key), V^T rows as they are.
template <typename M, int D, int BN, int NT, int KCH, int VCH, int KPITCH, int VPITCH>
__device__ __forceinline__ void store_tile(const Stage<KCH, VCH>& st, char* stage, int tid) {
  constexpr int ES = int(sizeof(typename M::Op)) / M::EPL;
  constexpr int KPR = D * ES / 16;
  constexpr int VPR = BN * ES / 16;
  char* sv = stage + BN * KPITCH;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int ci = j * NT + tid;
    const int r = ci / KPR;
    const int lr = (r & ~31) | M::row_of_key(r & 31);
    *reinterpret_cast<u32x4_t*>(stage + lr * KPITCH + (ci % KPR) * 16) = st.k[j];
  }
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int ci = j * NT + tid;
    *reinterpret_cast<u32x4_t*>(sv + (ci / VPR) * VPITCH + (ci % VPR) * 16) = st.v[j];
  }
}

template <typename T, int D, int QB, int NW, int BN>
__global__ __launch_bounds__(NW * 64, NW / 4) void chunk_attention_kernel(const AttnArgs a) {
  using M = Mma<T>;
  using Op = typename M::Op;
  constexpr int ES = int(sizeof(T));
  constexpr int BM = NW * QB * 32;
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;           // 32-feature blocks of the output
  constexpr int KSTEPS = D / M::K;      // contraction steps of K.Q^T
  constexpr int PSTEPS = 32 / M::K;     // contraction steps of V^T.P^T per 32-key block
  constexpr int KPITCH = D * ES + 16;   // LDS bytes per key row (16-byte pad: bank spread)
  constexpr int VPITCH = BN * ES + 16;  // LDS bytes per feature row of V^T
  constexpr int KTILE = BN * KPITCH;
  constexpr int STAGE = KTILE + D * VPITCH;
  constexpr int NT = NW * 64;
  constexpr int KPR = D * ES / 16;      // 16-byte pieces per key row
  constexpr int VPR = BN * ES / 16;     // 16-byte pieces per V^T row of the tile
  constexpr int KCH = BN * KPR / NT;
  constexpr int VCH = D * VPR / NT;
  static_assert(KCH * NT == BN * KPR && VCH * NT == D * VPR, "tile pieces must split evenly");
  static_assert(BN % 32 == 0 && SR_PAGE_TOKENS % BN == 0, "tiles must not straddle pages");
  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, hl = lane >> 5;

  // Workgroups are dispatched round-robin over the 8 XCDs (hardware id i runs on XCD i % 8).
  // Renumber so each XCD gets a contiguous range of (head, query tile): the query tiles of a
  // head then share that XCD's L2 while they stream the same keys.
  const int G = a.num_wg, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3, per = G >> 3, rem = G & 7;
  const int wg = local + xcd * per + (xcd < rem ? xcd : rem);
  // Integer divisions are expanded on the vector ALU; readfirstlane tells the compiler the
  // results are wave-uniform so the tile loop stays a scalar loop.
  const int h = uniform(wg / a.q_tiles);
  const int q0 = uniform((wg - h * a.q_tiles) * BM);
  const int n_q = a.n_q, H = a.H, cb = a.causal_block;
  const int cur = a.t.n - 1;
  const int cur_len = a.t.s[cur].len;

  // Query operands (B operand of K.Q^T), resident for the whole kernel.
  Op qop[QB][KSTEPS];
  int lim_cur[QB];
  const T* __restrict__ qg = static_cast<const T*>(a.q);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = q0 + (wave * QB + qb) * 32 + c;
    const bool ok = qrow < n_q;
    const T* src = qg + (size_t(ok ? qrow : 0) * H + h) * D + hl * M::EPL;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      Op v = M::load(reinterpret_cast<const char*>(src + ks * M::K));
      qop[qb][ks] = ok ? v : Op{};
    }
    lim_cur[qb] = ok ? min(cur_len, (qrow / cb + 1) * cb) : cur_len;
  }

  // Keys of the current chunk visible to every / to some query of this workgroup.
  const int qlast = min(q0 + BM, n_q) - 1;
  const int cur_all = uniform(min(cur_len, (q0 / cb + 1) * cb));
  const int cur_any = uniform(min(cur_len, (qlast / cb + 1) * cb));
  int ntiles = (cur_any + BN - 1) / BN;
  for (int s = 0; s < cur; ++s) ntiles += (a.t.s[s].len + BN - 1) / BN;
  ntiles = uniform(ntiles);

  float m_run[QB], l_run[QB];
  f32x16_t acc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kMaxInit;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16_t{};
  }

  const size_t head_page = size_t(h) * a.total_pages;
  Stage<KCH, VCH> stg;
  auto seg_end = [&](int s) { return s == cur ? cur_any : a.t.s[s].len; };
  auto advance = [&](int& s, int& k0) {
    k0 += BN;
    if (k0 >= seg_end(s)) {
      ++s;
      k0 = 0;
    }
  };
  int ls = 0, lk = 0;  // next tile to load
  int cs = 0, ck = 0;  // tile to compute
  load_tile<T, D, BN, NT, KCH, VCH>(stg, a, head_page, ls, lk, tid);
  store_tile<M, D, BN, NT, KCH, VCH, KPITCH, VPITCH>(stg, smem, tid);
  advance(ls, lk);
  __syncthreads();

  const float sl2 = a.scale_log2;
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile<T, D, BN, NT, KCH, VCH>(stg, a, head_page, ls, lk, tid);

    const bool is_cur = cs == cur;
    const int seg_len = a.t.s[cs].len;
    const bool partial = ck + BN > (is_cur ? cur_all : seg_len);

    const char* sk = smem + buf * STAGE;
    const char* sv = sk + KTILE;

    // S^T = K . Q^T for the BN keys of the tile.
    f32x16_t sc[NKB][QB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[kb][qb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const Op ka = M::load(sk + (kb * 32 + c) * KPITCH + (ks * M::K + hl * M::EPL) * ES);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[kb][qb] = M::mma(ka, qop[qb][ks], sc[kb][qb]);
      }
    }

    // Keys past the segment's valid length, or in a later causal block than the query's.
    if (partial) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lim = (is_cur ? lim_cur[qb] : seg_len) - ck;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + M::key_of_reg(i, hl) >= lim) sc[kb][qb][i] = -INFINITY;
      }
    }

    // Online softmax (exp2 domain), lazily rescaled.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][qb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run[qb], mx * sl2);
      if (__any(mnew > m_run[qb] + kRescaleThreshold)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
        m_run[qb] = mnew;
      }
      const float mneg = -m_run[qb];
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][i], sl2, mneg));
          lsum += p;
          sc[kb][qb][i] = p;
        }
      l_run[qb] += lsum;
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      Op pop[QB][PSTEPS];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kq = 0; kq < PSTEPS; ++kq) pop[qb][kq] = M::pack(sc[kb][qb], kq);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kq = 0; kq < PSTEPS; ++kq) {
          const Op va = M::load(sv + (db * 32 + c) * VPITCH + (kb * 32 + kq * M::K + hl * M::EPL) * ES);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = M::mma(va, pop[qb][kq], acc[qb][db]);
        }
      }
    }

    if (more) {
      store_tile<M, D, BN, NT, KCH, VCH, KPITCH, VPITCH>(stg, smem + (buf ^ 1) * STAGE, tid);
      advance(ls, lk);
    }
    advance(cs, ck);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, written token-major; lse = (max + log2 l) * ln 2.
  T* __restrict__ og = static_cast<T*>(a.o);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = q0 + (wave * QB + qb) * 32 + c;
    const float l = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.0f / l;
    if (qrow < n_q) {
      T* orow = og + (size_t(qrow) * H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          f32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[qb][db][4 * ig + e] * inv;
          M::store4(orow + db * 32 + 8 * ig + 4 * hl, v);
        }
      if (a.lse && hl == 0) a.lse[size_t(h) * n_q + qrow] = (m_run[qb] + __log2f(l)) * kLn2;
    }
  }
}

template <typename T, int D, int QB, int NW, int BN>
hipError_t launch_t(const Layout& L, const void* pool, const SegTable& t, const void* q, void* o, float* lse,
                    float scale, hipStream_t st) {
  constexpr int BM = NW * QB * 32;
  AttnArgs a;
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.kpool = static_cast<const char*>(pool);
  a.vpool = static_cast<const char*>(pool) + L.half_bytes;
  a.n_q = t.s[t.n - 1].len;
  a.H = L.H;
  a.total_pages = L.total_pages;
  a.causal_block = L.cb;
  a.q_tiles = (a.n_q + BM - 1) / BM;
  a.num_wg = a.q_tiles * L.H;
  a.scale_log2 = scale * kLog2e;
  a.t = t;
  hipLaunchKernelGGL((chunk_attention_kernel<T, D, QB, NW, BN>), dim3(a.num_wg), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Layout& L, const void* pool, const SegTable& t, const void* q, void* o, float* lse,
                            float softmax_scale, hipStream_t st) {
  if (L.dtype == SR_BF16)
    return L.D == 128 ? launch_t<uint16_t, 128, 1, 8, 64>(L, pool, t, q, o, lse, softmax_scale, st)
                      : launch_t<uint16_t, 64, 1, 8, 64>(L, pool, t, q, o, lse, softmax_scale, st);
  return L.D == 128 ? launch_t<float, 128, 1, 4, 32>(L, pool, t, q, o, lse, softmax_scale, st)
                    : launch_t<float, 64, 1, 4, 32>(L, pool, t, q, o, lse, softmax_scale, st);
}

}  // namespace sr
