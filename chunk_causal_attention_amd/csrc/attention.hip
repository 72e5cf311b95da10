// Chunk-causal attention over the paged KV cache, for gfx950 (MI355X).
//
// Computes, per head and current-chunk query i, softmax attention over the keys of the
// persistent bank, the history chunks in the window and the current chunk up to i's causal
// block (StreamRender-H3 project page, "3.1.2 Historical Context and Temporal Consistency",
// prefix cache; "3.3 Inference Acceleration and End-to-End Deployment", static-context KV
// caching and persistent KV layout).
//
// Work decomposition.  An item is (head, tile of BM = NW*QB*32 = 256 queries); each wave
// owns QB blocks of 32 queries.  A piece of work is an item's query tile over a range of
// its key tiles: the whole range, or, in the split schedule (kernels.hpp: queues of units), part
// of it, with the partial results merged by the item's last piece.  A piece walks the key
// tiles of its segments in visiting order; tiles past the last visible causal block are
// never loaded.  Each tile (BN = 128 keys, one cache page) is copied unchanged from HBM
// into LDS by gfx950's global-to-LDS loads (no staging registers), double buffered.  The
// cache pages are stored in the order the matrix instructions consume them, so every
// operand read is one 16-byte piece per lane at a lane base plus a constant offset, and
// 32 lanes read 512 contiguous bytes (no bank conflicts).
//
// Schedule.  Iteration i of the key loop works on 64-key sub-tiles of the cache pages:
//   [mask sub-tile i if partial]
//   { O^T += V^T P^T for sub-tile i-1  ||  exp2, rounding and row sums of half of sub-tile i }
//   { S^T = K Q^T for sub-tile i+1     ||  the other half }
//   [rare: sub-tile i's row max, rescale of O and l, its probabilities again]
// Each {..} block mixes MFMAs, their LDS operand reads and vector-ALU work (one probability
// per MFMA), and is scheduled to keep several LDS reads in flight and to slot the vector work
// between the MFMAs; two waves per SIMD run the same stream.  A sub-tile past every query's
// visible keys is simply fully masked (its probabilities are zero), so the loop has no other
// branches.  The loop runs one page (two iterations) per trip, the two sub-tiles' score
// registers alternating; a closing step adds the last sub-tile's P.V.  K and V pages have
// separate double buffers in LDS; the pages of tile t+2 (K) and t+1 (V) are requested at
// iteration 2t+1, two iterations before their first use, and a barrier ends every even
// iteration (one per page).
//
// Matrix instructions (32x32 output tile).  Scores are computed transposed, S^T = K . Q^T:
// the key block is the A operand, the queries are the B operand held in registers for the
// whole kernel, so lane (c, hl) of a wave owns query column c and row-wise reductions are
// in-lane plus one exchange with the other lane half (v_permlane32_swap).  The output P.V
// is also computed transposed, O^T += V^T . P^T, so the probabilities never leave the
// registers: the cache pages hold K rows in a permuted order chosen so that the score
// registers of a lane come out exactly in the operand order the P.V instruction expects,
// and V transposed, so its operand is one contiguous LDS read per lane.
//
// Softmax in the exp2 domain with a lazily updated running max (exact in real arithmetic): a
// sub-tile's probabilities are taken against the running max as it stands, and the sub-tile's
// own row max is computed only when some lane's sum of its 32 probabilities exceeds 2^12 (a
// probability may be that large or have overflowed); then the running max moves, O and l are
// rescaled and the probabilities are taken again.  So every probability that reaches the P.V
// product is at most 2^12, far from fp32/bf16 overflow, and the row max costs nothing on the
// common path.  The row sums are plain fp32 adds of the probabilities before their bf16
// rounding (two chains per lane): a dot-product instruction on the rounded pairs stalls the
// matrix unit when it sits between MFMAs (measured), and the rounding of P is one relative
// 2^-9 error per weight either way.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "mx_codec.hpp"

namespace sr {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte piece
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));  // operand of the scaled MX instruction

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units (generic path: fp32, head_dim 64 with QB > 1)
constexpr float kMaxInit = -1.0e30f;       // finite: keeps exp2(x - max) defined on masked rows
constexpr int kMaxTiles = SR_MAX_VISIBLE_PAGES;  // tile-table capacity (pages of visible keys)

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lanes l and l^32 each get f(x_l, x_{l^32}).
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
  static constexpr int SUB = 64;  // keys per compute sub-tile
  using Op = bf16x8_t;
  __device__ static f32x16_t mma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Key (inside a 32-key block) whose score lands in register i of lane half hl: the
  // registers 8*kq .. 8*kq+7 of a lane half are then the keys 16*kq + 8*hl + (0..7), which
  // is the P operand of contraction slice kq.  This holds because the cache stores key r of
  // each 32-row block at page row r with bits 2 and 3 swapped (row_pos in kv_kernels.hip):
  // output row 8*(i/4) + 4*hl + (i%4) then holds exactly that key.
  __device__ static constexpr int key_of_reg(int i, int hl) { return 16 * (i / 8) + 8 * hl + (i % 8); }
  __device__ static Op load(const char* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static Op pack(const f32x16_t& s, int kq) {
    f32x8_t t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = s[8 * kq + e];
    return __builtin_convertvector(t, bf16x8_t);  // round to nearest even
  }
  // acc + sum of the 8 bf16 values of p
  __device__ static float row_sum(Op p, float acc) {
    const bf16x2_t one = {__bf16(1.0f), __bf16(1.0f)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2_t pr = {p[2 * e], p[2 * e + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
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
  static constexpr int SUB = 64;
  using Op = float;
  __device__ static f32x16_t mma(Op a, Op b, f32x16_t c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
  // Register i of lane half hl holds key 2*i + hl, so the P operand of slice kq is register
  // kq (the cache stores key r at row 8*(r/8) + 4*(r%2) + (r/2)%4 of each 32-row block).
  __device__ static constexpr int key_of_reg(int i, int hl) { return 2 * i + hl; }
  __device__ static Op load(const char* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static Op pack(const f32x16_t& s, int kq) { return s[kq]; }
  __device__ static float row_sum(Op p, float acc) { return acc + p; }
  __device__ static void store4(float* dst, f32x4_t v) { *reinterpret_cast<f32x4_t*>(dst) = v; }
};

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  const char* kpool;
  const char* vpool;
  int32_t n_q, H, total_pages, causal_block;
  int32_t q_tiles, num_wg;
  float scale_log2;
  int32_t split;           // 0: one workgroup per item; 1: the split schedule (queues of units)
  int32_t fan;             // > 1: the fan split (fan_pieces), used instead of the queues
  int32_t fixed_tiles;     // pages of the bank and history segments
  int32_t n_items;         // H * q_tiles (head, query tile) items, head-major
  int32_t cus_per_xcd;     // split: C, compute units per XCD
  float* rec;              // split: 4C partial records per XCD
  int32_t* cnt;            // split: C arrival counters per XCD (zero between calls)
  int32_t* qctr;           // split: queue counter of each XCD, then the exit counter (zero between calls)
  SegTable t;
  WinView win;                              // window mode (win.n > 0): see WinView
  int32_t q_first[8], q_whole[8], q_left[8];  // split: each XCD's first item, whole items, split items
  int32_t q_share[8];                         // split: each XCD's split tiles per compute unit
  int32_t q_split0[9];                        // split: split items of the XCDs before x (q_split0[8]: all)
  int32_t q_levels;                           // split: most pieces of a split item
  alignas(4) int16_t left_tiles[8][kMaxCusPerXcd];  // split: key tiles of each XCD's split items
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Geometry of one kernel instantiation: one LDS tile = one cache page = 2 sub-tiles.
template <typename T, int D_, int QB_, int NW_>
struct Geo {
  using M = Mma<T>;
  using Op = typename M::Op;
  using Elem = T;
  static constexpr bool MX = false;
  static constexpr int D = D_, QB = QB_, NW = NW_;
  static constexpr int ES = int(sizeof(T));
  static constexpr int SUB = M::SUB;           // keys per compute sub-tile
  static constexpr int BN = SR_PAGE_TOKENS;    // keys per LDS tile
  static constexpr int BM = NW * QB * 32;
  static constexpr int NKB = SUB / 32;         // 32-key blocks per sub-tile
  static constexpr int NDB = D / 32;           // 32-feature blocks of the output
  static constexpr int KSTEPS = D / M::K;      // contraction steps of K.Q^T
  static constexpr int PSTEPS = 32 / M::K;     // contraction steps of V^T.P^T per 32-key block
  static constexpr int KTILE = BN * D * ES;    // bytes of the K page (and of the V page)
  static constexpr int KPAGE = KTILE, VPAGE = KTILE;
  static constexpr int VBASE = 2 * KTILE;      // LDS: K page buffers 0, 1, then V page buffers 0, 1
  static constexpr int TABLE = 4 * KTILE;      // then the tile table (16 bytes per tile)
  static constexpr int LDS_BYTES = TABLE + kMaxTiles * 16;
  __device__ static constexpr int key_of_reg(int i, int hl) { return M::key_of_reg(i, hl); }
  struct QOps {
    Op op[QB][KSTEPS];  // query operands, resident for the whole piece
  };
  static_assert(BN == 2 * SUB && SUB % 32 == 0, "a tile is two sub-tiles");
  static constexpr bool REC16 = ES == 2;           // O^T kept as bf16 in the record (bf16 caches)
  static constexpr int RPL = 2 * kRecordWordsPerLane;  // record floats per lane: O^T, (max, sum)
  static constexpr int REC = NW * 64 * RPL;            // record floats per workgroup
  static_assert(QB * (NDB * (REC16 ? 4 : 8) + 1) <= kRecordWordsPerLane, "record fits its slot");
  static_assert(BM == kQueryTile && REC == attn_record_floats(D), "record layout shared with the host");
};

// Geometry of the reduced-precision kernel (SR_MX caches): K pages of MXFP6 codes and
// scales, V pages of FP8 codes (layout in kv_kernels.hip, MxPage), bf16 queries quantized to
// MXFP6 in the prologue, bf16 output.  One LDS tile = one page = 2 sub-tiles of 64 keys, as in
// Geo, with one wave per 32 queries.
template <int D_>
struct GeoMx {
  using M = Mma<uint16_t>;  // bf16 output stores
  using Elem = uint16_t;
  using Op = i32x8_t;
  static constexpr bool MX = true;
  static constexpr int D = D_, QB = 1, NW = 8;
  static constexpr int SUB = 64, BN = SR_PAGE_TOKENS, BM = NW * 32;
  static constexpr int NKB = SUB / 32, NDB = D / 32, NB = D / 32;
  static constexpr int KSTEPS = D / 64;  // contraction steps of K.Q^T (64 features each)
  static constexpr int KPAGE = int(mx_kpage_bytes(D)), VPAGE = int(mx_vpage_bytes(D));
  static constexpr int LO = 0, HI = NB * BN * 16, SC = HI + NB * BN * 8;  // K page regions
  static constexpr int VBASE = 2 * KPAGE;  // LDS: K page buffers 0, 1, then V page buffers 0, 1
  static constexpr int TABLE = VBASE + 2 * VPAGE;
  static constexpr int LIMS = TABLE + kMaxTiles * 16;  // per-lane causal limits (int), read on partial tiles
  static constexpr int LDS_BYTES = LIMS + NW * 64 * 4;
  static constexpr int RPL = 2 * kRecordWordsPerLane;
  static constexpr int REC = NW * 64 * RPL;
  static constexpr bool REC16 = true;
  static_assert(BM == kQueryTile && REC == attn_record_floats(D), "record layout shared with the host");
  static_assert(SC + NB * BN <= KPAGE && KPAGE % 1024 == 0 && VPAGE % 1024 == 0, "page layout");
  // Score register i of lane half hl holds key 8*(i/4) + 4*hl + i%4 of its 32-key block (the
  // accumulator layout; MX pages keep the keys in order).
  __device__ static constexpr int key_of_reg(int i, int hl) { return 8 * (i / 4) + 4 * hl + (i % 4); }
  struct QOps {
    i32x8_t op[KSTEPS];  // MXFP6 codes of the lane's query block in each contraction step
    int sc;              // their E8M0 scale bytes: byte ks for step ks
  };
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 16-byte global-to-LDS load per lane: lane i's 16 bytes at `block` + lane_off land at
// LDS byte lds_base + 16 * i (lane_off = 16 i).  The block address is uniform and goes in a
// scalar register pair, the lane's offset in one vector register, so a page's loads hold no
// 64-bit vector addresses across the key loop.  Issued as inline asm so the compiler's
// wait-count insertion does not treat every later LDS read as dependent on it (it cannot tell
// the page buffers apart); the kernel orders these loads itself with explicit vmcnt waits and
// barriers.  M0 is written here and used by nothing else in this kernel (it is a reserved
// register that the compiler only sets right before instructions that read it).  The LDS-DMA
// load reads M0, and a scalar write of M0 needs one wait state before such a read (the
// compiler cannot insert it inside the asm block), hence the s_nop.
__device__ __forceinline__ void lds_load16(const char* block, int lane_off, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(lane_off),
               "s"(block)
               : "memory");
}

// Issues the global-to-LDS loads of one page of BYTES bytes (`src` = its first byte) into
// `dst`: a contiguous copy by the first NI = NW / 2 waves; load j of wave w < NI moves 1 KiB
// block (j*NI + w), lane i its piece i.  BYTES is a whole number of KiB, so a wave loads
// whole blocks or none (the last round may leave waves out).  Waves w and w + NW/2 share a
// SIMD, and the first (older) one wins the matrix unit's arbitration and reaches the page
// barrier first; giving it the loads evens out the time the two need per page (measured 0.7%
// faster than spreading them over all waves, 0.5% slower when the other half issues them).
template <int BYTES, int NW>
__device__ __forceinline__ void issue_bytes(const char* src, char* dst, int wave, int lane) {
  static_assert(BYTES % 1024 == 0, "pages are copied in 1 KiB blocks");
  constexpr int BLOCKS = BYTES / 1024;
  constexpr int NI = NW / 2;
  if (wave >= NI) return;
  const unsigned base = unsigned(size_t((lds_ptr_t)dst));
#pragma unroll
  for (int j = 0; j < (BLOCKS + NI - 1) / NI; ++j) {
    const int b = j * NI + wave;
    if ((j + 1) * NI <= BLOCKS || b < BLOCKS) lds_load16(src + b * 1024, lane * 16, uniform(int(base) + b * 1024));
  }
}
template <class G>
__device__ __forceinline__ void issue_k(const char* src, char* dst, int wave, int lane) {
  issue_bytes<G::KPAGE, G::NW>(src, dst, wave, lane);
}
template <class G>
__device__ __forceinline__ void issue_v(const char* src, char* dst, int wave, int lane) {
  issue_bytes<G::VPAGE, G::NW>(src, dst, wave, lane);
}

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations (global loads,
// global-to-LDS loads, stores) still outstanding.
// Inline asm as well: the compiler does not see the page loads and would drop a builtin
// wait that it considers redundant.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Operand addresses in a page buffer (byte offsets).  K: page row lr (rows are stored in
// operand order), element e of the row; piece x of every row is stored contiguously.
template <class G>
__device__ __forceinline__ int k_addr(int lr, int e) {
  const int bo = e * G::ES;
  return ((bo >> 4) * G::BN + lr) * 16 + (bo & 15);
}
// V: feature row d, key k of the page; piece y (keys 16/ES*y ..) of every feature row is
// stored contiguously.
template <class G>
__device__ __forceinline__ int v_addr(int d, int k) {
  const int bo = k * G::ES;
  return ((bo >> 4) * G::D + d) * 16 + (bo & 15);
}

// Per-lane running state of the online softmax for the wave's QB query blocks.
template <class G>
struct RowState {
  float m[G::QB];               // running max (log2 domain, scaled)
  float l[G::QB];               // running sum of probabilities (relative to m)
  f32x16_t acc[G::QB][G::NDB];  // O^T accumulators
};

template <class G>
using Scores = f32x16_t[G::NKB][G::QB];
template <class G>
using Probs = typename G::Op[G::NKB][G::QB][G::PSTEPS];

// S^T = K . Q^T for sub-tile `sub` of the K page in `kpage`.
template <class G>
__device__ __forceinline__ void scores(Scores<G>& sc, const typename G::Op (&qop)[G::QB][G::KSTEPS], const char* kpage,
                                       int sub, int c, int hl) {
  using M = typename G::M;
#pragma unroll
  for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
    for (int qb = 0; qb < G::QB; ++qb) sc[kb][qb] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < G::KSTEPS; ++ks)
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
      const typename G::Op ka = M::load(kpage + k_addr<G>(sub * G::SUB + kb * 32 + c, ks * M::K + hl * M::EPL));
#pragma unroll
      for (int qb = 0; qb < G::QB; ++qb) sc[kb][qb] = M::mma(ka, qop[qb][ks], sc[kb][qb]);
    }
}

// Key r of the sub-tile is visible to query block qb iff r < lim[qb]; the others get -inf.
template <class G>
__device__ __forceinline__ void mask_sub(Scores<G>& sc, const int (&lim)[G::QB], int hl) {
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + G::key_of_reg(i, hl) >= lim[qb]) sc[kb][qb][i] = -INFINITY;
}

// Row max of the raw scores (both lane halves hold the same value).
template <class G>
__device__ __forceinline__ void row_max(const Scores<G>& sc, float (&rmax)[G::QB]) {
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][qb][i]);
    rmax[qb] = pair_max(mx);
  }
}

// Lazy rescale: move the running max only when some row's max grew by more than 2^8.
template <class G>
__device__ __forceinline__ void rescale(RowState<G>& st, const float (&rmax)[G::QB], float sl2) {
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const float mnew = fmaxf(st.m[qb], rmax[qb] * sl2);
    if (__any(mnew > st.m[qb] + kRescaleThreshold)) {
      const float alpha = __builtin_amdgcn_exp2f(st.m[qb] - mnew);
      st.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) st.acc[qb][db] *= alpha;
      st.m[qb] = mnew;
    }
  }
}

// Probabilities exp2(s * scale_log2 - m), rounded to the operand type, and their row sums.
template <class G>
__device__ __forceinline__ void softmax_exp(RowState<G>& st, Scores<G>& sc, Probs<G>& pop, float sl2) {
  using M = typename G::M;
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const float mneg = -st.m[qb];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][qb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][i], sl2, mneg));
#pragma unroll
      for (int kq = 0; kq < G::PSTEPS; ++kq) {
        pop[kb][qb][kq] = M::pack(sc[kb][qb], kq);
        lsum = M::row_sum(pop[kb][qb][kq], lsum);
      }
    }
    st.l[qb] += lsum;
  }
}

// O^T += V^T . P^T for sub-tile `sub` of the V page in `vpage`.
template <class G>
__device__ __forceinline__ void accumulate(RowState<G>& st, const Probs<G>& pop, const char* vpage, int sub, int c,
                                           int hl) {
  using M = typename G::M;
#pragma unroll
  for (int db = 0; db < G::NDB; ++db)
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int kq = 0; kq < G::PSTEPS; ++kq) {
        const typename G::Op va =
            M::load(vpage + v_addr<G>(db * 32 + c, sub * G::SUB + kb * 32 + kq * M::K + hl * M::EPL));
#pragma unroll
        for (int qb = 0; qb < G::QB; ++qb) st.acc[qb][db] = M::mma(va, pop[kb][qb][kq], st.acc[qb][db]);
      }
}

// ---- bf16 path: explicitly pipelined blocks ------------------------------------------
// Each MFMA sits in its own scheduling region (sched_barrier), with the LDS read of the
// operand AH MFMAs ahead and a slice of the vector work, so the order below is the order
// the hardware sees.  The A operands of all MFMAs (V^T rows in block A, K rows in block B)
// stream through one ring of AH registers: MFMA j of a block reads slot j % AH and refills it
// with the operand AH MFMAs later, which near the end of a block is an operand of the next
// block.  So the reads run AH ahead across block boundaries too, except where the next
// block's page is published by the barrier in between.
constexpr int AH = 8;

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// An empty asm "use": the value must be computed before this point.  Keeps the compiler from
// sinking the exponentials (consumed only in the next iteration) out of the region where they
// fill the gap between two MFMAs.
template <typename V>
__device__ __forceinline__ void pin(const V& v) {
  asm volatile("" ::"v"(v));
}

// P.V operand r of sub-tile `sub`: r -> (db = r % NDB, kb, kq), so consecutive MFMAs
// accumulate into different output blocks.
template <class G>
__device__ __forceinline__ typename G::Op pv_operand(const char* vpage, int sub, int r, int c, int hl) {
  constexpr int NDB = G::NDB;
  const int db = r % NDB, kk = r / NDB, kb = kk / G::PSTEPS, kq = kk % G::PSTEPS;
  return G::M::load(vpage + v_addr<G>(db * 32 + c, sub * G::SUB + kb * 32 + kq * 16 + hl * 8));
}
// Score operand r of sub-tile `sub`: r -> (ks = r / NKB, kb = r % NKB), alternating the two
// score chains.
template <class G>
__device__ __forceinline__ typename G::Op qk_operand(const char* kpage, int sub, int r, int c, int hl) {
  const int ks = r / G::NKB, kb = r % G::NKB;
  return G::M::load(kpage + k_addr<G>(sub * G::SUB + kb * 32 + c, ks * 16 + hl * 8));
}

// Probabilities of a sub-tile are computed against the running max as it stands, without the
// sub-tile's own row max: a lane's 32 probabilities and their sum are taken first, and only if
// that sum exceeds 2^kSumLimit in some lane (some probability may be that large, or have
// overflowed) does the wave take the slow path (rescale_and_redo): the sub-tile's row max,
// the rescale of O and l to the new running max, and the probabilities again.  Every
// probability of the fast path is at most 2^kSumLimit, far from fp32/bf16 overflow.  The
// running max starts at kMaxInit, so a piece's first sub-tile always takes the slow path.
constexpr float kSumLimit = 4096.0f;  // 2^12

// Probability e of sub-tile `sc` (score register e % 16 of key block e / 16): exp2(s * sl2 - m)
// into grp[e % 8] and the row sum (two chains, by parity of e); a complete group of 8 is
// rounded to bf16 into its P.V operand.  The raw score stays in sc for the slow path.
template <class G>
__device__ __forceinline__ void prob(const Scores<G>& sc, Probs<G>& pop, float (&grp)[8], float (&lpart)[2], int e,
                                     float sl2, float mneg) {
  using M = typename G::M;
  const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e / 16][0][e % 16], sl2, mneg));
  grp[e % 8] = p;
  pin(grp[e % 8]);
  lpart[e & 1] += p;
  if ((e & 7) == 7) {
    f32x16_t t{};
#pragma unroll
    for (int x = 0; x < 8; ++x) t[8 * ((e % 16) / 8) + x] = grp[x];
    pop[e / 16][0][(e % 16) / 8] = M::pack(t, (e % 16) / 8);
    pin(pop[e / 16][0][(e % 16) / 8]);
  }
}

// Block A: O^T += V^T P^T of sub-tile i-1, with the first half of sub-tile i's probabilities
// (one per MFMA) in the shadow of its MFMAs.  LOADED: the ring already holds the first AH V
// operands (read during the previous block B); else they are read here.  SOFTMAX: false for
// the closing step (no sub-tile i).  With SOFTMAX, the last AH regions also read the first AH
// score operands of sub-tile i+1 (block B) into the ring, unless LAST (i is the piece's last
// sub-tile: there is no sub-tile i+1).
template <class G, bool LOADED, bool SOFTMAX, bool LAST = false>
__device__ __forceinline__ void block_a(RowState<G>& st, const Scores<G>& sc, Probs<G>& pop, float (&lpart)[2],
                                        float sl2, float mneg, const char* vpage, int vsub, const char* kpage,
                                        int ksub, typename G::Op (&ring)[AH], int c, int hl) {
  using M = typename G::M;
  constexpr int NP = G::NDB * G::NKB * G::PSTEPS;
  constexpr int NE = 16 * G::NKB;  // probabilities per lane
  static_assert(NP % AH == 0, "ring slots must line up across blocks");
  static_assert(NE % 2 == 0 && (NE / 2) % 8 == 0, "whole operand groups per block");
  constexpr int EA = NE / 2;  // probabilities computed here
  if constexpr (!LOADED) {
#pragma unroll
    for (int r = 0; r < AH; ++r) ring[r] = pv_operand<G>(vpage, vsub, r, c, hl);
  }
  float grp[8];
  fence();
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int db = r % G::NDB, kk = r / G::NDB, kb = kk / G::PSTEPS, kq = kk % G::PSTEPS;
    st.acc[0][db] = M::mma(ring[r % AH], pop[kb][0][kq], st.acc[0][db]);
    if (r + AH < NP)
      ring[r % AH] = pv_operand<G>(vpage, vsub, r + AH, c, hl);
    else if (SOFTMAX && !LAST)
      ring[r % AH] = qk_operand<G>(kpage, ksub, r + AH - NP, c, hl);
    if constexpr (SOFTMAX) {
#pragma unroll
      for (int e = r * EA / NP; e < (r + 1) * EA / NP; ++e) prob<G>(sc, pop, grp, lpart, e, sl2, mneg);
    }
    fence();
  }
}

// Block B: S^T = K Q^T of sub-tile i+1 alongside the second half of sub-tile i's
// probabilities.  The ring holds the first AH score operands on entry.  NEXT_V: the last AH
// regions read the first AH V operands of the next block A (half `vsub_next` of the V page at
// `vnext`) into the ring.  LAST: sub-tile i is the piece's last, so there are no scores to
// compute (and no score operands in the ring), only the probabilities and the V operands.
template <class G, bool NEXT_V, bool LAST = false>
__device__ __forceinline__ void block_b(const Scores<G>& sc, Probs<G>& pop, float (&lpart)[2], Scores<G>& sn,
                                        const typename G::Op (&qop)[1][G::KSTEPS], const char* kpage, int ksub,
                                        const char* vnext, int vsub_next, typename G::Op (&ring)[AH], float sl2,
                                        float mneg, int c, int hl) {
  using M = typename G::M;
  constexpr int NS = G::KSTEPS * G::NKB;
  static_assert(NS % AH == 0, "ring slots must line up across blocks");
  constexpr int NE = 16 * G::NKB, EA = NE / 2, NB = NE - EA;
  if constexpr (!LAST) {
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) sn[kb][0] = f32x16_t{};
  }
  float grp[8];
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    [[maybe_unused]] const int ks = r / G::NKB, kb = r % G::NKB;
    if constexpr (!LAST) sn[kb][0] = M::mma(ring[r % AH], qop[0][ks], sn[kb][0]);
    if (r + AH < NS) {
      if constexpr (!LAST) ring[r % AH] = qk_operand<G>(kpage, ksub, r + AH, c, hl);
    }
    else if (NEXT_V)
      ring[r % AH] = pv_operand<G>(vnext, vsub_next, r + AH - NS, c, hl);
#pragma unroll
    for (int e = EA + r * NB / NS; e < EA + (r + 1) * NB / NS; ++e) prob<G>(sc, pop, grp, lpart, e, sl2, mneg);
    fence();
  }
}

// The slow path of a sub-tile whose probabilities may exceed 2^kSumLimit: its row max moves the
// running max (where it is larger), O and l are rescaled to the new max, and the sub-tile's
// probabilities and row sum are computed again.  Exact in real arithmetic, like the fast path.
template <class G>
__device__ __forceinline__ float rescale_and_redo(RowState<G>& st, const Scores<G>& sc, Probs<G>& pop, float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16 * G::NKB; ++e) mx = fmaxf(mx, sc[e / 16][0][e % 16]);
  const float m_old = st.m[0];
  const float mnew = fmaxf(m_old, pair_max(mx) * sl2);
  const float alpha = __builtin_amdgcn_exp2f(m_old - mnew);
  st.l[0] *= alpha;
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) st.acc[0][db] *= alpha;
  st.m[0] = mnew;
  float grp[8], lpart[2] = {0.0f, 0.0f};
#pragma unroll
  for (int e = 0; e < 16 * G::NKB; ++e) prob<G>(sc, pop, grp, lpart, e, sl2, -mnew);
  return lpart[0] + lpart[1];
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = uint64_t(x);
  return int64_t((uint64_t(uint32_t(uniform(int(u >> 32)))) << 32) | uint32_t(uniform(int(uint32_t(u)))));
}

// A split item as the merge sees it: XCD x, index r among the XCD's split items and its tile
// count (queue split), or its pieces, first record slot and arrival counter (fan split).
struct SplitItem {
  int x = 0, r = 0, tiles = 0, share = 0;
  int fan = 0;    // fan split: pieces of the item (0: queue split)
  int slot0 = 0;  // fan split: the item's first record slot
  int ctr = 0;    // fan split: the item's arrival counter
};

// Calls f(slot) for every piece of split item `it` in slot order; returns their count.
template <class F>
__device__ __forceinline__ int for_each_subpiece(const AttnArgs& a, const SplitItem& it, int C, F&& f) {
  if (it.fan > 0) {
    for (int q = 0; q < it.fan; ++q) f(it.slot0 + q);
    return it.fan;
  }
  const int base = (it.x * C + it.r) * kMaxPieces;
  int n = 0;
  for (int k = 0; k < kMaxPieces; ++k) {
    if (piece_begin(it.tiles, it.share, k + 1) > piece_begin(it.tiles, it.share, k)) {
      f(base + k);
      ++n;
    }
  }
  return n;
}

// Records are written and read with relaxed 8-byte atomic stores and loads at device (agent)
// scope, which gfx950 performs at the device's coherence point (the sc1 cache policy) without
// touching other data in the XCD's L2.  Ordering: every wave waits for its record stores to
// complete (vmcnt 0) before the workgroup barrier that precedes the arrival counter update,
// and the merging workgroup loads records only after its counter update returned.
// Release/acquire fences at device scope would instead write back and invalidate the whole L2
// of the XCD, dropping the key pages every other workgroup there is streaming.
__device__ __forceinline__ void rec_put(float* rec, int word, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(rec) + word, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t rec_get(const float* rec, int word) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(rec)) + word, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), bf16x2_t));
}
__device__ __forceinline__ float bf16_low(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_high(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
__device__ __forceinline__ uint64_t pair64(uint32_t lo, uint32_t hi) { return uint64_t(lo) | (uint64_t(hi) << 32); }
// The bits of a float, taken by value: __builtin_bit_cast applied directly to an element of an
// ext_vector_type vector reads the wrong value with this toolchain (every element of the
// vector came out as element 0), a scalar argument does not.
__device__ __forceinline__ uint32_t float_bits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Record layout: 8-byte words, lane-major: word w of lane (wave, lane) at word index
// (wave * RPL / 2 + w) * 64 + lane, so every store and load of a record is a coalesced 512-byte
// row per wave.  Per query block, fp32 records (fp32 caches): O^T in words 8 db + k (registers
// 2k, 2k+1 of output block db), then one word (max, sum).  bf16 records (bf16 and reduced-
// precision caches, whose outputs are bf16): O^T rounded to bf16 in words 4 db + k (registers
// 4k .. 4k+3 of block db), then (max, sum) in fp32.
template <class G>
constexpr int record_words() {
  return G::REC16 ? 4 : 8;  // words per 32-feature output block
}
template <class G>
__device__ __forceinline__ uint64_t record_word(const RowState<G>& st, int qb, int db, int k) {
  const f32x16_t& o = st.acc[qb][db];
  if constexpr (G::REC16)
    return pair64(pack_bf16x2(o[4 * k], o[4 * k + 1]), pack_bf16x2(o[4 * k + 2], o[4 * k + 3]));
  else
    return pair64(float_bits(o[2 * k]), float_bits(o[2 * k + 1]));
}

template <class G>
__device__ __forceinline__ void store_record(float* rec, const RowState<G>& st, int wave, int lane) {
  static_assert(G::RPL % 2 == 0, "records in 8-byte words");
  constexpr int NK = record_words<G>();
  static_assert(G::QB * (G::NDB * NK + 1) <= G::RPL / 2, "record fits its slot");
  const int base = wave * (G::RPL / 2) * 64 + lane;
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const int w0 = qb * (G::NDB * NK + 1);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int k = 0; k < NK; ++k) rec_put(rec, base + (w0 + NK * db + k) * 64, record_word<G>(st, qb, db, k));
    rec_put(rec, base + (w0 + NK * G::NDB) * 64,
            pair64(float_bits(st.m[qb]), float_bits(st.l[qb])));
  }
}

// Merges the pieces of a split item in slot order, rescaling to the running max as it goes
// (O^T and l of each piece times 2^(m_piece - m)).  Every piece, the merging workgroup's own
// included, is read back from its record (the own one was completed before the arrival
// counter moved), so all pieces pass through the same rounding whichever piece merges.
template <class G>
__device__ __forceinline__ void merge_records(const AttnArgs& a, RowState<G>& st, const SplitItem& it, int wave,
                                              int lane) {
  constexpr int NK = record_words<G>();
  const int base = wave * (G::RPL / 2) * 64 + lane;
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    st.m[qb] = kMaxInit;
    st.l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) st.acc[qb][db] = f32x16_t{};
  }
  for_each_subpiece(a, it, a.cus_per_xcd, [&](int slot) {
    const float* rec = a.rec + size_t(slot) * G::REC;
#pragma unroll
    for (int qb = 0; qb < G::QB; ++qb) {
      const int w0 = qb * (G::NDB * NK + 1);
      const uint64_t ml = rec_get(rec, base + (w0 + NK * G::NDB) * 64);
      const float mk = __builtin_bit_cast(float, uint32_t(ml)), lk = __builtin_bit_cast(float, uint32_t(ml >> 32));
      const float mn = fmaxf(st.m[qb], mk);
      const float a0 = __builtin_amdgcn_exp2f(st.m[qb] - mn), a1 = __builtin_amdgcn_exp2f(mk - mn);
      st.m[qb] = mn;
      st.l[qb] = st.l[qb] * a0 + lk * a1;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const uint64_t wv = rec_get(rec, base + (w0 + NK * db + k) * 64);
          const uint32_t lo = uint32_t(wv), hi = uint32_t(wv >> 32);
          f32x16_t& o = st.acc[qb][db];
          if constexpr (G::REC16) {
            o[4 * k] = o[4 * k] * a0 + bf16_low(lo) * a1;
            o[4 * k + 1] = o[4 * k + 1] * a0 + bf16_high(lo) * a1;
            o[4 * k + 2] = o[4 * k + 2] * a0 + bf16_low(hi) * a1;
            o[4 * k + 3] = o[4 * k + 3] * a0 + bf16_high(hi) * a1;
          } else {
            o[2 * k] = o[2 * k] * a0 + __builtin_bit_cast(float, lo) * a1;
            o[2 * k + 1] = o[2 * k + 1] * a0 + __builtin_bit_cast(float, hi) * a1;
          }
        }
    }
  });
}

// Iteration i of the key loop (ODD: i odd): mask sub-tile i if partial; P.V of sub-tile i-1
// alongside the row max of sub-tile i; the lazy rescale; scores of sub-tile i+1 (into sn)
// alongside the probabilities of sub-tile i.  `ent` is the table entry of tile i / 2.  The
// closing step (CLOSING, i == nsub) only adds the P.V of sub-tile nsub-1.  `mid` runs
// between the P.V and the scores (the page requests placed there).  `ring` carries
// operands between the blocks: an odd iteration leaves in it the first V operands of the
// even iteration that follows (the even iteration's V page was published before the odd
// one began); an odd iteration reads its own after the barrier that precedes it.
struct NoWork {
  __device__ void operator()() const {}
};
template <class G, int ODD, bool CLOSING = false, bool LAST = false, class Mid = NoWork>
__device__ __forceinline__ void key_step(int i, const int4& ent, int nsub, const int (&lim_cur)[G::QB], char* smem,
                                         RowState<G>& st, Scores<G>& sc, Scores<G>& sn, Probs<G>& pop,
                                         const typename G::Op (&qop)[G::QB][G::KSTEPS], typename G::Op (&ring)[AH],
                                         float sl2, int c, int hl, Mid mid = Mid{}) {
  constexpr int SUB = G::SUB;
  constexpr int NEXT = ODD ? 0 : 1;  // half of the page holding sub-tiles i-1 and i+1
  const int sub0 = ODD * SUB;
  const bool in_seq = i < nsub;
  const int any_rel = in_seq ? uniform(ent.z) - sub0 : 0;
  const int all_rel = in_seq ? uniform(ent.w) - sub0 : 0;
  const int cur_k0 = uniform(ent.y);
  int lim[G::QB];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb)
    lim[qb] = any_rel <= 0 ? 0 : (cur_k0 >= 0 ? lim_cur[qb] - cur_k0 - sub0 : all_rel);
  if (!CLOSING && all_rel < SUB) mask_sub<G>(sc, lim, hl);
  const char* vpage = smem + G::VBASE + (((i - 1) >> 1) & 1) * G::VPAGE;  // sub-tile i-1
  const char* kpage = smem + (((i + 1) >> 1) & 1) * G::KPAGE;             // sub-tile i+1
  float rmax[G::QB];
  if constexpr (G::ES == 2 && G::QB == 1) {
    float lpart[2] = {0.0f, 0.0f};
    const float mneg = -st.m[0];
    block_a<G, !ODD, !CLOSING, LAST>(st, sc, pop, lpart, sl2, mneg, vpage, NEXT, kpage, NEXT, ring, c, hl);
    if (CLOSING) return;  // nothing follows the last sub-tile's P.V
    mid();
    // Odd i: the next iteration's P.V reads sub-tile i, the second half of V page i / 2.
    const char* vnext = smem + G::VBASE + ((i >> 1) & 1) * G::VPAGE;
    block_b<G, ODD == 1, LAST>(sc, pop, lpart, sn, qop, kpage, NEXT, vnext, 1, ring, sl2, mneg, c, hl);
    float lsum = lpart[0] + lpart[1];
    // Some probability of the sub-tile may exceed 2^kSumLimit: take its row max (rare).
    if (__any(!(lsum <= kSumLimit))) lsum = rescale_and_redo<G>(st, sc, pop, sl2);
    st.l[0] += lsum;
  } else {
    accumulate<G>(st, pop, vpage, NEXT, c, hl);
    if (CLOSING) return;
    row_max<G>(sc, rmax);
    rescale<G>(st, rmax, sl2);
    mid();
    if constexpr (!LAST) scores<G>(sn, qop, kpage, NEXT, c, hl);
    softmax_exp<G>(st, sc, pop, sl2);
  }
}

// ---- reduced-precision path (SR_MX) -------------------------------------------------
// "The road to the fastest, cheapest H3", Accelerating the denoiser, item 2: MXFP6 queries
// and keys, FP8 values.  Scores: v_mfma_scale_f32_32x32x64_f8f6f4 with FP6 E2M3 operands,
// each lane holding one 32-feature block of a key (A) or query (B) row, 24 bytes of codes,
// with its own E8M0 scale byte.  P.V: the same instruction with FP8 E4M3 operands; the
// probabilities are converted to FP8 as p * 2^kPShift (round to nearest even) and the
// instruction's B scale 2^-kPShift takes the factor out again, so that probabilities down to
// 2^-15 of the running max stay representable.  The lazy rescale threshold is
// kMxRescale = 2 (log2), so p * 2^kPShift <= 2^8 stays below FP8's largest value 448.  The
// row sums are those of the rounded probabilities, taken by one more instruction with an
// all-ones A operand (every output row is then the row sum), which keeps the vector ALU free
// for the exponentials.
constexpr int kFmtFp8 = 0, kFmtFp6 = 2;  // format codes of the scaled MX instruction
constexpr int kPShift = 6;
constexpr float kMxRescale = 2.0f;
constexpr int kScaleOne = 127;  // E8M0 byte of 1.0

template <int FA, int FB, int OA, int OB>
__device__ __forceinline__ f32x16_t mma_mx(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OA, sa, OB, sb);
}

// Quantizes the lane's query row (bf16, `row` = its first feature) for the B operand of the
// score instruction: contraction step ks uses block 2*ks + hl.  Same codes as the cache's
// keys (mx_codec.hpp).  Rows past n_q get zero codes.
template <class G>
__device__ __forceinline__ void mx_queries(typename G::QOps& qo, const uint16_t* row, bool ok, int hl) {
  qo.sc = 0;
#pragma unroll
  for (int ks = 0; ks < G::KSTEPS; ++ks) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(row + (2 * ks + hl) * 32);
    unsigned xs[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t w = ok ? src[j] : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[8 * j + 2 * i] = w[i] & 0xFFFFu;
        xs[8 * j + 2 * i + 1] = w[i] >> 16;
      }
    }
    unsigned w[6];
    const int X = mx::quantize_block(xs, w);
    qo.op[ks] = i32x8_t{int(w[0]), int(w[1]), int(w[2]), int(w[3]), int(w[4]), int(w[5]), 0, 0};
    qo.sc |= (X + 127) << (8 * ks);
  }
}

// Byte offsets, inside a page buffer, of what lane (c, hl) reads at the start of each region
// (block hl of key row c, its scale bytes, feature row c of lane half hl's V keys); every
// operand read is one of them plus a constant.  Each page adds an opaque scalar zero to them
// (mx_page), so that the operand addresses are formed next to their reads (an immediate offset
// each) instead of being hoisted out of the loop into registers of their own.
struct MxLane {
  int kl, kh, ks, v;
};
template <class G>
__device__ __forceinline__ MxLane mx_lane(int c, int hl) {
  return MxLane{G::LO + (hl * G::BN + c) * 16, G::HI + (hl * G::BN + c) * 8, G::SC + c * G::NB + hl * (G::NB / 2),
                (hl * G::D + c) * 16};
}

// A operand of the score instruction: block 2*ks + hl of key row r0 + c of the K page (16 + 8
// bytes; the last two dwords are not read for FP6).
template <class G>
__device__ __forceinline__ i32x8_t mx_k_operand(const char* kpage, const MxLane& ln, int r0, int ks) {
  const int cst = 2 * ks * G::BN + r0;  // rows past the lane's own
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kpage + ln.kl + cst * 16);
  const i32x2_t hi = *reinterpret_cast<const i32x2_t*>(kpage + ln.kh + cst * 8);
  const i32x4_t hi4 = __builtin_shufflevector(hi, hi, 0, 1, -1, -1);
  return __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, -1, -1);
}
// Scale bytes of key row r0 + c for the lane half: byte ks is block 2*ks + hl.
template <class G>
__device__ __forceinline__ int mx_k_scales(const char* kpage, const MxLane& ln, int r0) {
  if constexpr (G::NB == 4) return *reinterpret_cast<const uint16_t*>(kpage + ln.ks + r0 * 4);
  return *reinterpret_cast<const uint8_t*>(kpage + ln.ks + r0 * 2);
}
// A operand of the P.V instruction for output block db, sub-tile `sub`: feature row
// db*32 + c, the 16 keys of each 32-key block that lane half hl's probabilities cover
// (groups 4*sub + hl and 4*sub + 2 + hl of the V page).
template <class G>
__device__ __forceinline__ i32x8_t mx_v_operand(const char* vpage, const MxLane& ln, int sub, int db) {
  const int cst = (4 * sub * G::D + db * 32) * 16;
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(vpage + ln.v + cst);
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(vpage + ln.v + cst + 2 * G::D * 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// S^T = K Q^T for sub-tile `sub` of the K page.
template <class G>
__device__ __forceinline__ void mx_scores(f32x16_t (&sn)[2], const typename G::QOps& qo, const char* kpage,
                                          const MxLane& ln, int sub) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r0 = sub * G::SUB + kb * 32;
    const int ksc = mx_k_scales<G>(kpage, ln, r0);
    sn[kb] = mma_mx<kFmtFp6, kFmtFp6, 0, 0>(mx_k_operand<G>(kpage, ln, r0, 0), qo.op[0], f32x16_t{}, ksc, qo.sc);
    if constexpr (G::KSTEPS > 1)
      sn[kb] = mma_mx<kFmtFp6, kFmtFp6, 1, 1>(mx_k_operand<G>(kpage, ln, r0, 1), qo.op[1], sn[kb], ksc, qo.sc);
  }
}

// ---- reduced-precision key loop: explicitly pipelined blocks --------------------------
// As in the bf16 path, each MFMA sits in its own scheduling region with a slice of the
// vector work, and the LDS operands of a block are read in the regions of the block before:
// block A reads the K operands of block B, block B those of the next block A (when that
// V page is already published).  Per 64-key sub-tile and wave the vector work is 32
// exponentials with their scaling, 16 conversions to FP8 and 16 max3 against 4 + 1 P.V and
// 4 score MFMAs (head_dim 128).  An exponential costs about 3.4 FMA issue slots and does not
// overlap other vector work, and the two waves of a SIMD (one workgroup, one barrier per
// page) run in phase, so each block carries vector work in proportion to its MFMA time: the
// whole row max in the first region of block A, the rescale decision in the second, most
// exponentials in the rest of block A (whose P.V MFMAs are the long ones), the remainder in
// block B.
template <class G>
constexpr int mx_early() { return G::NDB == 4 ? 24 : 12; }  // probabilities computed in block A
constexpr int kOnesFp4 = 0x22222222;      // eight FP4 (E2M1) 1.0
constexpr int kFmtFp4 = 4;

// Score operand j of a sub-tile: key block j % 2, contraction step j / 2 (consecutive
// instructions accumulate into different score blocks).
template <class G>
__device__ __forceinline__ i32x8_t mx_qk_operand(const char* kpage, const MxLane& ln, int sub, int j) {
  return mx_k_operand<G>(kpage, ln, sub * G::SUB + (j % 2) * 32, j / 2);
}
// Score instruction j (j is a constant once the callers' loops are unrolled).
template <class G>
__device__ __forceinline__ void mx_score_mma(f32x16_t (&sn)[2], int j, const i32x8_t& kop, const typename G::QOps& qo,
                                             const int (&ksc)[2]) {
  if (j < 2) {
    sn[j] = mma_mx<kFmtFp6, kFmtFp6, 0, 0>(kop, qo.op[0], f32x16_t{}, ksc[j], qo.sc);
  } else if constexpr (G::KSTEPS > 1) {
    sn[j - 2] = mma_mx<kFmtFp6, kFmtFp6, 1, 1>(kop, qo.op[1], sn[j - 2], ksc[j - 2], qo.sc);
  }
}
// Probability e of the sub-tile (score register e % 16 of key block e / 16) into sc; when a
// group of four is complete, its FP8 codes go to dword e / 4 of pnew.
__device__ __forceinline__ void mx_prob(f32x16_t (&sc)[2], i32x8_t& pnew, int e, float sl2, float mneg) {
  sc[e / 16][e % 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e / 16][e % 16], sl2, mneg));
  pin(sc[e / 16][e % 16]);
  if ((e & 3) == 3) {
    const f32x16_t& s = sc[e / 16];
    const int b = (e % 16) - 3;
    // The first conversion fills bytes 0-1 and the second bytes 2-3, so the register's prior
    // contents (the probabilities of two sub-tiles ago) do not matter; converting into it in
    // place spares zeroing or copying.
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[b], s[b + 1], pnew[e / 4], false);
    pnew[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(s[b + 2], s[b + 3], lo, true);
    pin(pnew[e / 4]);
  }
}

// Block A: O^T += V^T P^T of sub-tile i-1 (NDB instructions) and the row sums (one
// instruction with all-ones A), with, between them, the row max of sub-tile i (region 0),
// the rescale decision (region 1), the first mx_early probabilities of sub-tile i (regions 1
// on) and the K operands and scales of block B.  LOADED: vop already holds the V operands.
// SOFTMAX false: the closing step (P.V only).
template <class G, bool LOADED, bool SOFTMAX>
__device__ __forceinline__ void mx_block_a(RowState<G>& st, f32x16_t& lacc, f32x16_t (&sc)[2], const i32x8_t& pop,
                                           i32x8_t& pnew, bool& grow, float& mnew, float& mneg, float sl2,
                                           const char* vpage, int vsub, const char* kpage, int ksub,
                                           i32x8_t (&vop)[G::NDB], i32x8_t (&kop)[2 * G::KSTEPS], int (&ksc)[2],
                                           const i32x8_t& ones, const MxLane& ln) {
  constexpr int NDB = G::NDB, NP = NDB + 1, NS = 2 * G::KSTEPS;
  constexpr int EA = mx_early<G>(), EPR = EA / (NP - 1);  // probabilities per region 1 .. NP-1
  static_assert(NS <= NP && EA % 4 == 0 && EPR * (NP - 1) == EA, "block A layout");
  if constexpr (!LOADED) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) vop[db] = mx_v_operand<G>(vpage, ln, vsub, db);
  }
  float mx = -INFINITY;
  fence();
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    if (r < NDB)
      st.acc[0][r] = mma_mx<kFmtFp8, kFmtFp8, 0, 0>(vop[r], pop, st.acc[0][r], kScaleOne, kScaleOne - kPShift);
    else
      lacc = mma_mx<kFmtFp4, kFmtFp8, 0, 0>(ones, pop, lacc, kScaleOne, kScaleOne - kPShift);
    if constexpr (SOFTMAX) {
      if (r < NS) kop[r] = mx_qk_operand<G>(kpage, ln, ksub, r);
      if (r == 0) {
        ksc[0] = mx_k_scales<G>(kpage, ln, ksub * G::SUB);
        ksc[1] = mx_k_scales<G>(kpage, ln, ksub * G::SUB + 32);
      }
      if (r == 0) {
#pragma unroll
        for (int e = 0; e < 32; e += 2) {
          mx = fmaxf(mx, fmaxf(sc[e / 16][e % 16], sc[(e + 1) / 16][(e + 1) % 16]));
          pin(mx);
        }
      }
      if (r == 1) {
        const float m_old = st.m[0];
        mnew = fmaxf(m_old, pair_max(mx) * sl2);
        grow = __any(mnew > m_old + kMxRescale);
        mneg = float(kPShift) - (grow ? mnew : m_old);
      }
      if (r >= 1) {
#pragma unroll
        for (int e = (r - 1) * EPR; e < r * EPR; ++e) mx_prob(sc, pnew, e, sl2, mneg);
      }
    }
    fence();
  }
}

// Block B: S^T = K Q^T of sub-tile i+1 (operands read in block A) alongside the remaining
// probabilities of sub-tile i; NEXT_V: also reads the next block A's V operands (half 1 of
// the V page at vnext).
template <class G, bool NEXT_V>
__device__ __forceinline__ void mx_block_b(f32x16_t (&sc)[2], i32x8_t& pnew, f32x16_t (&sn)[2],
                                           const typename G::QOps& qo, const i32x8_t (&kop)[2 * G::KSTEPS],
                                           const int (&ksc)[2], const char* vnext, i32x8_t (&vop)[G::NDB], float sl2,
                                           float mneg, const MxLane& ln) {
  constexpr int NS = 2 * G::KSTEPS, NDB = G::NDB;
  constexpr int EA = mx_early<G>(), NE = 32 - EA;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    mx_score_mma<G>(sn, j, kop[j], qo, ksc);
    if constexpr (NEXT_V) {
#pragma unroll
      for (int db = j * NDB / NS; db < (j + 1) * NDB / NS; ++db) vop[db] = mx_v_operand<G>(vnext, ln, 1, db);
    }
#pragma unroll
    for (int e = EA + j * NE / NS; e < EA + (j + 1) * NE / NS; ++e) mx_prob(sc, pnew, e, sl2, mneg);
    fence();
  }
}

// Iteration i of the reduced-precision key loop (ODD: i odd), the same steps and buffers as
// key_step: mask sub-tile i if partial; block A (P.V of sub-tile i-1 from pop, row max of
// sub-tile i); the lazy rescale; `mid`; block B (scores of sub-tile i+1, probabilities of
// sub-tile i into pnew).  The caller alternates two registers sets for pop and pnew.
// CLOSING: only the P.V of the last sub-tile.  vop carries the V operands from an odd
// iteration to the even one that follows (whose V page was published before the odd one).
// KBUF / VBUF: the page buffers holding sub-tiles i+1 (K) and i-1 (V), VNBUF the V buffer of
// sub-tile i (read ahead by odd iterations); constants, so every operand address is a lane
// base plus an immediate offset.
template <class G, int ODD, int KBUF, int VBUF, int VNBUF, bool CLOSING = false, class Mid = NoWork>
__device__ __forceinline__ void mx_key_step(int i, const int4& ent, int nsub, const int (&lim_cur)[1], char* smem,
                                            RowState<G>& st, f32x16_t& lacc, f32x16_t (&sc)[2], f32x16_t (&sn)[2],
                                            const i32x8_t& pop, i32x8_t& pnew, const typename G::QOps& qo,
                                            i32x8_t (&vop)[G::NDB], const i32x8_t& ones, const MxLane& ln, float sl2,
                                            int hl, Mid mid = Mid{}) {
  constexpr int SUB = G::SUB;
  constexpr int NEXT = ODD ? 0 : 1;
  const int sub0 = ODD * SUB;
  const bool in_seq = i < nsub;
  const int any_rel = in_seq ? uniform(ent.z) - sub0 : 0;
  const int all_rel = in_seq ? uniform(ent.w) - sub0 : 0;
  const int cur_k0 = uniform(ent.y);
  if (!CLOSING && all_rel < SUB) {
    // The lane's causal limit comes from LDS (kept there rather than in a register that the
    // loop would spill).  Key kb*32 + key_of_reg(r, hl) = kb*32 + 8*(r/4) + r%4 + 4*hl: the
    // lane half's term moves to the limit, so each comparison is against a constant.
    const int lc = reinterpret_cast<const int*>(smem + G::LIMS)[threadIdx.x];
    const int lim = any_rel <= 0 ? 0 : (cur_k0 >= 0 ? lc - cur_k0 - sub0 : all_rel);
    const int limh = lim - 4 * hl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + G::key_of_reg(r, 0) >= limh) sc[kb][r] = -INFINITY;
  }
  const char* vpage = smem + G::VBASE + VBUF * G::VPAGE;  // sub-tile i-1
  const char* kpage = smem + KBUF * G::KPAGE;             // sub-tile i+1
  i32x8_t kop[2 * G::KSTEPS];
  int ksc[2];
  bool grow = false;
  float mnew = 0.0f, mneg = 0.0f;
  mx_block_a<G, !ODD, !CLOSING>(st, lacc, sc, pop, pnew, grow, mnew, mneg, sl2, vpage, NEXT, kpage, NEXT, vop, kop,
                                ksc, ones, ln);
  if (CLOSING) return;
  if (grow) {  // lazy rescale: some row's max grew by more than 2^kMxRescale
    const float alpha = __builtin_amdgcn_exp2f(st.m[0] - mnew);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) st.acc[0][db] *= alpha;
    lacc *= alpha;
    st.m[0] = mnew;
  }
  mid();
  // Odd i: the next iteration's P.V reads sub-tile i, the second half of V page i / 2.
  const char* vnext = smem + G::VBASE + VNBUF * G::VPAGE;
  mx_block_b<G, ODD == 1>(sc, pnew, sn, qo, kop, ksc, vnext, vop, sl2, mneg, ln);
}

// Page t of a reduced-precision piece (PAR = t % 2, the buffer its K and V pages sit in):
// iterations 2t and 2t+1 with the page requests and the barrier between them, as in the bf16
// loop of run_piece.  ent holds the table entry of tile t on entry and of tile t+1 on exit.
template <class G, int PAR>
__device__ __forceinline__ void mx_page(const AttnArgs& a, char* smem, const int4* tab, int t, int ntiles,
                                        size_t head_page, int4& ent, const int (&lim_cur)[1], RowState<G>& st,
                                        f32x16_t& lacc, f32x16_t (&sc)[2], f32x16_t (&sn)[2], i32x8_t& pa,
                                        i32x8_t& pb, const typename G::QOps& qo, i32x8_t (&vop)[G::NDB],
                                        const i32x8_t& ones, const MxLane& lane_base, float sl2, int wave,
                                        int lane) {
  const int hl = lane >> 5;
  const int nsub = 2 * ntiles;
  int z = 0;
  asm volatile("" : "+s"(z));  // an SGPR, so no wait for vector memory is implied
  const MxLane ln{lane_base.kl + z, lane_base.kh + z, lane_base.ks + z, lane_base.v + z};
  // iteration 2t: K of sub-tile 2t+1 in buffer PAR, V of sub-tile 2t-1 (tile t-1) in 1-PAR
  mx_key_step<G, 0, PAR, 1 - PAR, PAR>(2 * t, ent, nsub, lim_cur, smem, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln,
                                       sl2, hl);
  // Table entries, made scalar right away (the barrier below waits for the reads anyway), so
  // that they occupy no vector registers across the page.
  const int4 tn = tab[min(t + 1, ntiles - 1)];
  const int kpage_next = uniform(tab[min(t + 2, ntiles - 1)].x);
  const int4 ent_next = make_int4(uniform(tn.x), uniform(tn.y), uniform(tn.z), uniform(tn.w));
  const int vpage_next = ent_next.x;
  if (t >= 1) wait_loads<0>();
  __syncthreads();
  if (t + 1 < ntiles)
    issue_v<G>(a.vpool + (head_page + vpage_next) * G::VPAGE, smem + G::VBASE + (1 - PAR) * G::VPAGE, wave, lane);
  const auto request_k = [&] {
    if (t + 2 < ntiles)
      issue_k<G>(a.kpool + (head_page + kpage_next) * G::KPAGE, smem + PAR * G::KPAGE, wave, lane);
  };
  // iteration 2t+1: K of sub-tile 2t+2 (tile t+1) in 1-PAR, V of sub-tile 2t in PAR
  mx_key_step<G, 1, 1 - PAR, PAR, PAR>(2 * t + 1, ent, nsub, lim_cur, smem, st, lacc, sn, sc, pb, pa, qo, vop, ones,
                                       ln, sl2, hl, request_k);
  ent = ent_next;
}

// The key loop of a reduced-precision piece: the page schedule of the bf16 loop in run_piece
// (pages requested in iteration 2t+1, one barrier per page), unrolled by two pages so that
// buffer parities are constants, with the row sums accumulated in `lacc` and handed to st.l
// at the end (on lane half 0, so that the pair sum of the epilogue and the merge of split
// pieces see each row once).
template <class G>
__device__ __forceinline__ void mx_key_loop(const AttnArgs& a, char* smem, const int4* tab, RowState<G>& st,
                                            const typename G::QOps& qo, const int (&lim_cur)[1], int ntiles,
                                            size_t head_page, float sl2, int wave, int lane) {
  const int c = lane & 31, hl = lane >> 5;
  const int nsub = 2 * ntiles;
  f32x16_t lacc = {};
  f32x16_t sc[2], sn[2];
  i32x8_t pa = {0, 0, 0, 0, 0, 0, 0, 0};  // P of odd sub-tiles; iteration 0 multiplies the zeroed V buffer 1
  i32x8_t pb = {0, 0, 0, 0, 0, 0, 0, 0};  // P of even sub-tiles
  const MxLane ln = mx_lane<G>(c, hl);
  i32x8_t vop[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) vop[db] = mx_v_operand<G>(smem + G::VBASE + G::VPAGE, ln, 1, db);
  const i32x8_t ones = {kOnesFp4, kOnesFp4, kOnesFp4, kOnesFp4, kOnesFp4, kOnesFp4, kOnesFp4, kOnesFp4};
  reinterpret_cast<int*>(smem + G::LIMS)[threadIdx.x] = lim_cur[0];  // read back by this lane only
  const int4 t0 = tab[0];
  int4 ent = make_int4(uniform(t0.x), uniform(t0.y), uniform(t0.z), uniform(t0.w));
  mx_scores<G>(sc, qo, smem, ln, 0);
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    mx_page<G, 0>(a, smem, tab, t, ntiles, head_page, ent, lim_cur, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln,
                  sl2, wave, lane);
    mx_page<G, 1>(a, smem, tab, t + 1, ntiles, head_page, ent, lim_cur, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln,
                  sl2, wave, lane);
  }
  if (t < ntiles) {  // odd page count: the last page sits in buffer 0
    mx_page<G, 0>(a, smem, tab, t, ntiles, head_page, ent, lim_cur, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln,
                  sl2, wave, lane);
    mx_key_step<G, 0, 0, 0, 0, true>(nsub, ent, nsub, lim_cur, smem, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln, sl2,
                                     hl);
  } else {
    mx_key_step<G, 0, 0, 1, 0, true>(nsub, ent, nsub, lim_cur, smem, st, lacc, sc, sn, pa, pb, qo, vop, ones, ln, sl2,
                                     hl);
  }
  st.l[0] = hl == 0 ? lacc[0] : 0.0f;
}

// The page requests and barriers of the key loop without its compute, for a wave none of
// whose query rows exist (the last, partial query tile of a head): the wave still moves its
// share of every page and meets every barrier, in the order of the bf16 and reduced-precision
// loops (V of tile t+1 into buffer (t+1) % 2 after the barrier of page t, K of tile t+2 into
// buffer t % 2), but leaves the matrix unit and the LDS reads to the waves that have rows.
template <class G>
__device__ __forceinline__ void idle_key_loop(const AttnArgs& a, char* smem, const int4* tab, int ntiles,
                                              size_t head_page, int wave, int lane) {
  for (int t = 0; t < ntiles; ++t) {
    const int vpage_next = uniform(tab[min(t + 1, ntiles - 1)].x);
    const int kpage_next = uniform(tab[min(t + 2, ntiles - 1)].x);
    if (t >= 1) wait_loads<0>();
    __syncthreads();
    if (t + 1 < ntiles)
      issue_v<G>(a.vpool + (head_page + vpage_next) * G::VPAGE, smem + G::VBASE + ((t + 1) & 1) * G::VPAGE, wave,
                 lane);
    if (t + 2 < ntiles)
      issue_k<G>(a.kpool + (head_page + kpage_next) * G::KPAGE, smem + (t & 1) * G::KPAGE, wave, lane);
  }
}

// Length and first page of segment s as window `win` sees it (win < 0: the table as is; else
// the bank segments as is and, of every chunk, the window's pages and tokens).
__device__ __forceinline__ int seg_len(const AttnArgs& a, int win, int s) {
  return (win < 0 || s < a.win.bank_segs) ? a.t.s[s].len : a.win.frames * a.win.tok[win];
}
__device__ __forceinline__ int seg_page(const AttnArgs& a, int win, int s) {
  return (win < 0 || s < a.win.bank_segs) ? a.t.s[s].page : a.t.s[s].page + win * a.win.pages;
}

// Pool page (relative to the head's first page) of tile t of the call's tile list: the
// pages of the segments in visiting order.
__device__ __forceinline__ int tile_page_index(const AttnArgs& a, int win, int t) {
  int s = 0, first = 0;
  for (; s < a.t.n - 1; ++s) {
    const int nt = (seg_len(a, win, s) + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
    if (t < first + nt) break;
    first += nt;
  }
  return uniform(seg_page(a, win, s) + (t - first));
}

// A unit of work: query tile qt of head h over tiles [tb, te) of its tile list; slot < 0:
// the whole list (the unit writes the output), else a piece of split item `it` (record
// `slot`).
struct Unit {
  int h = 0, qt = 0, tb = 0, te = 0, slot = -1;
  SplitItem it{};
};

// Whole item u of XCD x's queue.
__device__ __forceinline__ Unit whole_unit(const AttnArgs& a, int x, int u) {
  Unit un;
  const int item = a.q_first[x] + u;
  un.h = uniform(item / a.q_tiles);
  un.qt = uniform(item - un.h * a.q_tiles);
  un.te = uniform(item_tiles(un.qt, a.fixed_tiles, a.n_q, a.causal_block, a.t.s[a.t.n - 1].len));
  return un;
}

// Piece k of split item r of XCD x.  False for an empty piece of a short item (no work, no
// record).
__device__ __forceinline__ bool piece_unit(const AttnArgs& a, int x, int r, int k, Unit& un) {
  const int C = a.cus_per_xcd;
  // A dword-aligned read of the tile counts keeps the load scalar.
  const int pair = reinterpret_cast<const int32_t*>(a.left_tiles[x])[r >> 1];
  const int T = uniform((pair << (16 * (1 - (r & 1)))) >> 16);
  const int share = a.q_share[x];
  un = Unit{};
  un.tb = uniform(piece_begin(T, share, k));
  un.te = uniform(piece_begin(T, share, k + 1));
  const int item = a.q_first[x] + a.q_whole[x] + r;
  un.h = uniform(item / a.q_tiles);
  un.qt = uniform(item - un.h * a.q_tiles);
  if (un.te <= un.tb) return false;
  if (split_pieces(T, share) > 1) {
    un.slot = (x * C + r) * kMaxPieces + k;
    un.it.x = x;
    un.it.r = r;
    un.it.tiles = T;
    un.it.share = share;
  } else {
    un.tb = 0;
    un.te = T;
  }
  return true;
}

// Unit u of XCD x's queue: its whole items, then piece 0 of each of its split items.
__device__ __forceinline__ bool xcd_unit(const AttnArgs& a, int x, int u, Unit& un) {
  if (u < a.q_whole[x]) {
    un = whole_unit(a, x, u);
    return true;
  }
  return piece_unit(a, x, uniform(u - a.q_whole[x]), 0, un);
}

// Unit v of the device's piece queue: piece k = 1 + v / S of split item j = v % S, the S split
// items of all XCDs in XCD order.
__device__ __forceinline__ bool device_unit(const AttnArgs& a, int v, Unit& un) {
  const int S = a.q_split0[8];
  const int k = uniform(1 + v / S), j = uniform(v - (v / S) * S);
  int x = 0;
  while (x < 7 && j >= a.q_split0[x + 1]) ++x;
  x = uniform(x);
  return piece_unit(a, x, uniform(j - a.q_split0[x]), k, un);
}

// One unit of work (Unit).  win >= 0: window mode, the rows and keys of that window (WinView).
template <class G>
__device__ __forceinline__ void run_piece(const AttnArgs& a, char* smem, int* flag, const Unit& un, int win) {
  const int h = un.h, qt = un.qt, tb = un.tb, te = un.te, slot = un.slot;
  const SplitItem& it = un.it;
  using M = typename G::M;
  using Op = typename G::Op;
  using T = typename G::Elem;
  constexpr int BN = G::BN, D = G::D;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int c = lane & 31, hl = lane >> 5;
  const int q0 = qt * G::BM;
  const int H = a.H, cb = a.causal_block;
  // Rows of this call (window mode: the window's), their first packed row, and the row count
  // of the lse layout [H][rows of the whole call].
  const int n_q = win < 0 ? a.n_q : uniform(a.win.frames * a.win.tok[win]);
  const int row0 = win < 0 ? 0 : uniform(a.win.row0[win]);
  const int lse_rows = a.n_q;
  const int cur = a.t.n - 1;
  const int cur_len = uniform(seg_len(a, win, cur));
  const int ntiles = te - tb;  // tiles [tb, te) of the item's tile list
  const size_t head_page = size_t(h) * a.total_pages;
  __syncthreads();  // the previous piece of this workgroup is done with LDS

  // The first pages (K and V of tile tb, K of tile tb+1) are requested first, their page
  // indices walked from the segment table in scalar code, so that their latency overlaps
  // the query loads and the tile-table build below.
  issue_k<G>(a.kpool + (head_page + tile_page_index(a, win, tb)) * G::KPAGE, smem, wave, lane);
  issue_v<G>(a.vpool + (head_page + tile_page_index(a, win, tb)) * G::VPAGE, smem + G::VBASE, wave, lane);
  if (ntiles > 1)
    issue_k<G>(a.kpool + (head_page + tile_page_index(a, win, tb + 1)) * G::KPAGE, smem + G::KPAGE, wave, lane);

  // Query operands (B operand of K.Q^T), resident for the whole piece.
  typename G::QOps qo;
  int lim_cur[G::QB];
  const T* __restrict__ qg = static_cast<const T*>(a.q);
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const int qrow = q0 + (wave * G::QB + qb) * 32 + c;
    const bool ok = qrow < n_q;
    if constexpr (G::MX) {
      mx_queries<G>(qo, qg + (size_t(row0 + (ok ? qrow : 0)) * H + h) * D, ok, hl);
    } else {
      const T* src = qg + (size_t(row0 + (ok ? qrow : 0)) * H + h) * D + hl * M::EPL;
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) {
        Op v = M::load(reinterpret_cast<const char*>(src + ks * M::K));
        qo.op[qb][ks] = ok ? v : Op{};
      }
    }
    lim_cur[qb] = ok && cb > 0 ? min(cur_len, (qrow / cb + 1) * cb) : cur_len;
  }

  // Keys of the current chunk visible to every / to some query of this workgroup.
  const int qlast = min(q0 + G::BM, n_q) - 1;
  const int cur_all = uniform(cb > 0 ? min(cur_len, (q0 / cb + 1) * cb) : cur_len);
  const int cur_any = uniform(cb > 0 ? min(cur_len, (qlast / cb + 1) * cb) : cur_len);

  RowState<G> st;
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    st.m[qb] = kMaxInit;
    st.l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) st.acc[qb][db] = f32x16_t{};
  }

  // Tile table of the piece: for tile t (visiting order) the page index (relative to the
  // head's first page), the key offset inside the current chunk (-1 for the persistent bank
  // and history), and the keys of the tile visible to some / to every query of the
  // workgroup (relative to the tile start; <= 0 past them).  Entry t - tb holds tile t.
  int4* tab = reinterpret_cast<int4*>(smem + G::TABLE);
  for (int t = tb + tid; t < te; t += G::NW * 64) {
    int s = 0, first = 0;
    for (; s < cur; ++s) {
      const int nt = (seg_len(a, win, s) + BN - 1) / BN;
      if (t < first + nt) break;
      first += nt;
    }
    const int k0 = (t - first) * BN;
    const bool is_cur = s == cur;
    const int len = seg_len(a, win, s);
    tab[t - tb] = make_int4(seg_page(a, win, s) + k0 / SR_PAGE_TOKENS, is_cur ? k0 : -1, (is_cur ? cur_any : len) - k0,
                            (is_cur ? cur_all : len) - k0);
  }
  // V buffer 1 zeroed: iteration 0 multiplies it by all-zero probabilities, so it must not
  // hold NaN bit patterns.
  u32x4_t* vz = reinterpret_cast<u32x4_t*>(smem + G::VBASE + G::VPAGE);
  for (int x = tid; x < G::VPAGE / 16; x += G::NW * 64) vz[x] = u32x4_t{0, 0, 0, 0};
  wait_loads<0>();  // first pages and query operands
  __syncthreads();

  const float sl2 = a.scale_log2;
  const int nsub = 2 * ntiles;  // sub-tiles j = 2t, 2t+1 of tile t
  if (uniform(q0 + wave * G::QB * 32) >= n_q) {
    idle_key_loop<G>(a, smem, tab, ntiles, head_page, wave, lane);
  } else if constexpr (G::MX) {
    mx_key_loop<G>(a, smem, tab, st, qo, lim_cur, ntiles, head_page, sl2, wave, lane);
  } else {
  const auto& qop = qo.op;
  Scores<G> sc;
  Probs<G> pop;
#pragma unroll
  for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
    for (int qb = 0; qb < G::QB; ++qb)
#pragma unroll
      for (int kq = 0; kq < G::PSTEPS; ++kq) pop[kb][qb][kq] = Op{};
  // Table entry of tile 0, read (and waited for) before the LDS operand reads below: the wait
  // at the loop head serves every iteration, so it must not find this read queued behind them.
  int4 ent = tab[0];
  asm volatile("" ::"v"(ent.x), "v"(ent.y), "v"(ent.z), "v"(ent.w) : "memory");
  scores<G>(sc, qop, smem, 0, c, hl);
  Scores<G> sc_odd;  // scores of the odd sub-tile of the current pair (ping-pong with sc)
  // Operand ring: iteration 0 starts with its V operands loaded, from the zeroed buffer that
  // stands for sub-tile -1.
  Op ring[AH];
  if constexpr (G::ES == 2 && G::QB == 1) {
#pragma unroll
    for (int r = 0; r < AH; ++r) ring[r] = pv_operand<G>(smem + G::VBASE + G::VPAGE, 1, r, c, hl);
  }

  // Pair t = iterations 2t (even, first half of tile t) and 2t+1 (odd, second half), then
  // the closing iteration nsub, which only adds the last sub-tile's P.V.  Page requests, in
  // iteration 2t+1: V of tile t+1 at its start (its buffer held tile t-1, last read in
  // iteration 2t) and K of tile t+2 halfway, between its P.V and its scores (its buffer held
  // tile t, last read in iteration 2t); splitting the requests in two halves the burst that
  // the memory pipeline queues at once.  V of tile t+1 and K of tile t+2 are first read in iteration 2t+3:
  // each wave waits for its requests at the end of iteration 2t+2, and the barrier that ends
  // every even iteration publishes those pages and releases the buffers that iteration 2t+3
  // overwrites.
  // The table entries for tile t+1 and the page index of tile t+2 are read at the end of
  // iteration 2t, where the barrier waits for all LDS reads anyway (read earlier, they would
  // make the wave wait for the operand reads queued behind them).
  for (int t = 0; t + 1 < ntiles; ++t) {  // ent: table entry of tile t
    key_step<G, 0>(2 * t, ent, nsub, lim_cur, smem, st, sc, sc_odd, pop, qop, ring, sl2, c, hl);
    const int4 ent_next = tab[t + 1];
    const int kpage_next = tab[min(t + 2, ntiles - 1)].x;  // K of tile t+2, requested at 2t+1
    const int vpage_next = ent_next.x;                     // V of tile t+1, requested at 2t+1
    if (t >= 1) wait_loads<0>();
    __syncthreads();
    issue_v<G>(a.vpool + (head_page + uniform(vpage_next)) * G::VPAGE, smem + G::VBASE + ((t + 1) & 1) * G::VPAGE,
               wave, lane);
    const auto request_k = [&] {
      if (t + 2 < ntiles)
        issue_k<G>(a.kpool + (head_page + uniform(kpage_next)) * G::KPAGE, smem + (t & 1) * G::KPAGE, wave, lane);
    };
    key_step<G, 1>(2 * t + 1, ent, nsub, lim_cur, smem, st, sc_odd, sc, pop, qop, ring, sl2, c, hl, request_k);
    ent = ent_next;
  }
  {
    // The last page, t = ntiles - 1: no pages to request and, in its odd iteration, no scores
    // of a next sub-tile.
    const int t = ntiles - 1;
    key_step<G, 0>(2 * t, ent, nsub, lim_cur, smem, st, sc, sc_odd, pop, qop, ring, sl2, c, hl);
    if (t >= 1) wait_loads<0>();
    __syncthreads();
    key_step<G, 1, false, true>(2 * t + 1, ent, nsub, lim_cur, smem, st, sc_odd, sc, pop, qop, ring, sl2, c, hl);
  }
  key_step<G, 0, true>(nsub, ent, nsub, lim_cur, smem, st, sc, sc_odd, pop, qop, ring, sl2, c, hl);
  }
  __syncthreads();

  // A piece of a split item leaves its partial result in its record; the last of the item's
  // pieces to arrive merges all of them (in piece order, so the result does not depend on
  // which piece came last) and writes the output.  Nobody waits for anybody.
  if (slot >= 0) {
    store_record<G>(a.rec + size_t(slot) * G::REC, st, wave, lane);
    wait_loads<0>();  // this wave's record stores have completed
    __syncthreads();
    if (tid == 0) {
      int32_t* cnt = it.fan > 0 ? a.cnt + it.ctr : a.cnt + it.x * a.cus_per_xcd + it.r;
      const int pieces = for_each_subpiece(a, it, a.cus_per_xcd, [](int) {});
      const int arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = arrived == pieces - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;
    merge_records<G>(a, st, it, wave, lane);
  }

  // Epilogue: O = O^T / l, written token-major; lse = (max + log2 l) * ln 2.
  T* __restrict__ og = static_cast<T*>(a.o);
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const int qrow = q0 + (wave * G::QB + qb) * 32 + c;
    const float l = pair_sum(st.l[qb]);
    const float inv = 1.0f / l;
    if (qrow < n_q) {
      T* orow = og + (size_t(row0 + qrow) * H + h) * D;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          f32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = st.acc[qb][db][4 * ig + e] * inv;
          M::store4(orow + db * 32 + 8 * ig + 4 * hl, v);
        }
      if (a.lse && hl == 0) a.lse[size_t(h) * lse_rows + row0 + qrow] = (st.m[qb] + __log2f(l)) * kLn2;
    }
  }
}

// A unit given by its fields.
template <class G>
__device__ __forceinline__ void run_unit(const AttnArgs& a, char* smem, int* flag, int h, int qt, int tb, int te,
                                         int slot, const SplitItem& it, int win = -1) {
  Unit un;
  un.h = h;
  un.qt = qt;
  un.tb = tb;
  un.te = te;
  un.slot = slot;
  un.it = it;
  run_piece<G>(a, smem, flag, un, win);
}

// The queue split (kernels.hpp): a persistent workgroup takes whole items from its XCD's queue,
// then from the other XCDs' queues, then units of the device's piece queue, until all are
// empty; the last workgroup to finish zeroes the counters for the next call.  Thread 0 claims a
// unit and hands it to the workgroup through LDS; the claim loop ends for every workgroup,
// since each counter only grows and a workgroup gives up on a queue once it is past its end.
template <class G>
__device__ __forceinline__ void queue_split(const AttnArgs& a, char* smem, int* flag, int* claim, int home) {
  const int dev_units = (a.q_levels - 1) * a.q_split0[8];  // units of the device's piece queue
  int y = home, passed = 0;  // thread 0: the XCD queue it claims from, XCD queues found empty
  for (;;) {
    if (threadIdx.x == 0) {
      int kind = -1, u = -1;
      while (passed < 8) {
        const int units = a.q_whole[y] + a.q_left[y];
        if (units > 0) {
          const int v = __hip_atomic_fetch_add(a.qctr + y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v < units) {
            kind = 0;
            u = v;
            break;
          }
        }
        y = (y + 1) & 7;
        ++passed;
      }
      if (kind < 0 && dev_units > 0) {
        const int v = __hip_atomic_fetch_add(a.qctr + kPieceCounter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v < dev_units) {
          kind = 1;
          u = v;
        }
      }
      claim[0] = kind;
      claim[1] = y;
      claim[2] = u;
    }
    __syncthreads();
    const int kind = uniform(claim[0]), x = uniform(claim[1]), u = uniform(claim[2]);
    __syncthreads();  // every thread has read the claim before thread 0 makes the next one
    if (kind < 0) break;
    Unit un;
    if (!(kind == 0 ? xcd_unit(a, x, u, un) : device_unit(a, u, un)))
      continue;  // an empty piece of a short item: no work, no record
    run_piece<G>(a, smem, flag, un, -1);
  }
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(a.qctr + kExitCounter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == a.num_wg - 1) {
      for (int q = 0; q < kQueueCounters; ++q)
        __hip_atomic_store(a.qctr + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class G>
__global__ __launch_bounds__(G::NW * 64, G::NW / 4) void chunk_attention_kernel(const AttnArgs a) {
  __shared__ __align__(1024) char smem[G::LDS_BYTES];
  __shared__ int flag;
  __shared__ int claim[3];

  // Workgroups are dispatched round-robin over the 8 XCDs: hardware id i runs on XCD i % 8
  // as the (i / 8)-th workgroup of that XCD.  Integer divisions are expanded on the vector
  // ALU; readfirstlane keeps every loop bound and branch scalar.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;

  if (a.fan > 0) {
    // Fan split: workgroup j = (h fan + p) q_tiles + qt, numbered so each XCD gets a contiguous
    // range of j, runs piece p of item (h, qt); the query tiles of a head that read the same
    // key tiles then run together on one XCD.
    const int nwg = a.num_wg, per = nwg >> 3, rem = nwg & 7;
    const int j = local + xcd * per + (xcd < rem ? xcd : rem);
    const int hp = j / a.q_tiles;
    const int qt = uniform(j - hp * a.q_tiles);
    const int h = uniform(hp / a.fan);
    const int pc = uniform(hp - h * a.fan);
    const int tiles = item_tiles(qt, a.fixed_tiles, a.n_q, a.causal_block, a.t.s[a.t.n - 1].len);
    const int tb = uniform(pc * tiles / a.fan);
    const int te = uniform((pc + 1) * tiles / a.fan);
    const int item = h * a.q_tiles + qt;
    SplitItem it{};
    it.fan = a.fan;
    it.slot0 = item * a.fan;
    it.ctr = item;
    run_unit<G>(a, smem, &flag, h, qt, tb, te, item * a.fan + pc, it);
    return;
  }
  if (a.split) {
    queue_split<G>(a, smem, &flag, claim, xcd);
    return;
  }
  // One workgroup per item, renumbered so each XCD gets a contiguous range of items: the
  // query tiles of a head then share that XCD's L2 while they stream the same keys.
  const int nwg = a.num_wg, per = nwg >> 3, rem = nwg & 7;
  const int g = local + xcd * per + (xcd < rem ? xcd : rem);
  const int h = uniform(g / a.q_tiles);
  const int qt = uniform(g - h * a.q_tiles);
  const int te = uniform(item_tiles(qt, a.fixed_tiles, a.n_q, a.causal_block, a.t.s[a.t.n - 1].len));
  run_unit<G>(a, smem, &flag, h, qt, 0, te, -1, SplitItem{});
}

// Window mode (a.win.n > 0): one workgroup per item (window, head, query tile), window-major
// and head-major inside a window, renumbered so each XCD gets a contiguous range of items (the
// query tiles of a window and head share that XCD's L2); every item runs whole over its
// window's keys.
template <class G>
__global__ __launch_bounds__(G::NW * 64, G::NW / 4) void windows_attention_kernel(const AttnArgs a) {
  __shared__ __align__(1024) char smem[G::LDS_BYTES];
  __shared__ int flag;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int nwg = a.num_wg, per = nwg >> 3, rem = nwg & 7;
  const int g = local + xcd * per + (xcd < rem ? xcd : rem);
  int w = 0;
  while (w + 1 < a.win.n && g >= a.win.item0[w + 1]) ++w;
  w = uniform(w);
  const int rows = a.win.frames * a.win.tok[w];
  const int qtw = (rows + G::BM - 1) / G::BM;
  const int loc = g - a.win.item0[w];
  const int h = uniform(loc / qtw);
  const int qt = uniform(loc - h * qtw);
  int fixed = 0;
  for (int s = 0; s < a.t.n - 1; ++s) fixed += (seg_len(a, w, s) + G::BN - 1) / G::BN;
  const int te = uniform(item_tiles(qt, fixed, rows, 0, seg_len(a, w, a.t.n - 1)));
  run_unit<G>(a, smem, &flag, h, qt, 0, te, -1, SplitItem{}, w);
}

template <class G>
hipError_t launch_t(const Layout& L, const void* pool, const SegTable& t, int32_t n_q, int32_t cb, const void* q,
                    void* o, float* lse, float scale, const SplitWorkspace& ws, hipStream_t st, const WinView* win) {
  static_assert(SR_MAX_VISIBLE_PAGES <= 32767, "tile counts are stored as int16");
  AttnArgs a{};
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.kpool = static_cast<const char*>(pool);
  a.vpool = static_cast<const char*>(pool) + L.half_bytes;
  a.n_q = n_q;
  a.H = L.H;
  a.total_pages = L.total_pages;
  a.causal_block = cb;
  a.q_tiles = (a.n_q + G::BM - 1) / G::BM;
  a.scale_log2 = scale * kLog2e;
  a.fixed_tiles = 0;
  for (int s = 0; s + 1 < t.n; ++s) a.fixed_tiles += (t.s[s].len + G::BN - 1) / G::BN;
  a.n_items = a.q_tiles * L.H;
  a.split = ws.cus_per_xcd > 0 && !win ? 1 : 0;
  a.cus_per_xcd = ws.cus_per_xcd;
  a.rec = ws.records;
  a.cnt = ws.counters;
  a.fan = 0;
  if (a.split) {
    int32_t min_tiles = 1 << 30;
    for (int32_t qt = 0; qt < a.q_tiles; ++qt) {
      const int32_t tl = item_tiles(qt, a.fixed_tiles, a.n_q, cb, t.s[t.n - 1].len);
      min_tiles = tl < min_tiles ? tl : min_tiles;
    }
    a.fan = fan_pieces(a.n_items, min_tiles, ws.cus_per_xcd);
    if (a.fan < 2) a.fan = 0;
    // Items that fit one round of the device run whole: a two-band split of them only adds the
    // cost of its pieces (measured 9% slower on 228 items of 128 tiles).
    if (a.fan == 0 && a.n_items <= 8 * ws.cus_per_xcd) a.split = 0;
  }
  if (a.fan > 0) {
    a.num_wg = a.n_items * a.fan;  // at most 8 C: records and counters fit the workspace
  } else if (a.split) {
    // Queues: XCD x owns items [first, first + n); the last n mod C of them are split, their
    // pieces in the device's piece queue.  One persistent workgroup per compute unit.
    const int32_t C = ws.cus_per_xcd;
    a.q_levels = 0;
    a.q_split0[0] = 0;
    for (int x = 0; x < 8; ++x) {
      const int32_t first = int32_t(int64_t(x) * a.n_items / 8);
      const int32_t n = int32_t(int64_t(x + 1) * a.n_items / 8) - first;
      a.q_first[x] = first;
      a.q_left[x] = n % C;
      a.q_whole[x] = n - n % C;
      int32_t split_tiles = 0;
      for (int32_t r = 0; r < a.q_left[x]; ++r) {
        a.left_tiles[x][r] =
            int16_t(item_tiles((first + a.q_whole[x] + r) % a.q_tiles, a.fixed_tiles, a.n_q, cb, t.s[t.n - 1].len));
        split_tiles += a.left_tiles[x][r];
      }
      a.q_share[x] = (split_tiles + C - 1) / C;
      for (int32_t r = 0; r < a.q_left[x]; ++r) {
        const int32_t np = split_pieces(a.left_tiles[x][r], a.q_share[x]);
        a.q_levels = np > a.q_levels ? np : a.q_levels;
      }
      a.q_split0[x + 1] = a.q_split0[x] + a.q_left[x];
    }
    a.qctr = ws.counters + 8 * C;
    a.num_wg = 8 * C;
  } else {
    a.num_wg = win ? win->item0[win->n] : a.n_items;
  }
  if (win) a.win = *win;
  a.t = t;
  if (win) {
    if constexpr (G::MX) return hipErrorNotSupported;  // refused on the host: no windowed SR_MX caches
    else hipLaunchKernelGGL((windows_attention_kernel<G>), dim3(a.num_wg), dim3(G::NW * 64), 0, st, a);
  } else {
    hipLaunchKernelGGL((chunk_attention_kernel<G>), dim3(a.num_wg), dim3(G::NW * 64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Layout& L, const void* pool, const SegTable& t, int32_t n_q, int32_t cb,
                            const void* q, void* o, float* lse, float softmax_scale, const SplitWorkspace& ws,
                            hipStream_t st, const WinView* win) {
  if (L.dtype == SR_MX)
    return L.D == 128 ? launch_t<GeoMx<128>>(L, pool, t, n_q, cb, q, o, lse, softmax_scale, ws, st, win)
                      : launch_t<GeoMx<64>>(L, pool, t, n_q, cb, q, o, lse, softmax_scale, ws, st, win);
  if (L.dtype == SR_BF16)
    return L.D == 128 ? launch_t<Geo<uint16_t, 128, 1, 8>>(L, pool, t, n_q, cb, q, o, lse, softmax_scale, ws, st, win)
                      : launch_t<Geo<uint16_t, 64, 1, 8>>(L, pool, t, n_q, cb, q, o, lse, softmax_scale, ws, st, win);
  // fp32 caches are head_dim 64 only (validated on the host): a double-buffered 128-key
  // fp32 tile at head_dim 128 would need 256 KiB of LDS.
  return launch_t<Geo<float, 64, 1, 8>>(L, pool, t, n_q, cb, q, o, lse, softmax_scale, ws, st, win);
}

}  // namespace sr
