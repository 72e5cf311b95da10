// Device-side entry points used by the C ABI (capi.cpp).  All launches are asynchronous
// on the given stream and return the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "core.hpp"

namespace sr {

// Segments of one call: the ring's (bank, up to SR_MAX_WINDOW history chunks, current) or, for the
// global-token attention of a windowed cache, the bank and every window's part of the current chunk.
constexpr int kMaxSegs = SR_MAX_LAYOUT_WINDOWS + 2;
static_assert(kMaxSegs >= SR_MAX_WINDOW + 2, "ring segments fit");

// One logical key segment as the kernels see it: first pool page and valid tokens.
struct DevSeg {
  int32_t page;
  int32_t len;
};

// Segment table of one call, built on the host when the ring changes and passed by value
// (no per-call host-to-device copy).  Segments are in visiting order; the last one is the
// "current" segment, the only one whose visibility can depend on the query row (see
// item_tiles): the current chunk for chunk and window calls, the bank for prefix calls.
struct SegTable {
  int32_t n;
  DevSeg s[kMaxSegs];
};

// Queries per workgroup of the attention kernel (8 waves x 32 queries).
constexpr int kQueryTile = 256;

// Window layout of a windowed cache as the kernels see it (sr_window_layout plus prefix sums).
// In window mode an attention call runs every window as its own short sequence: window w's
// rows are packed rows [row0[w], row0[w+1]) of q / out; its keys are the call's bank segments
// unchanged and, of every other segment (a chunk), the window's pages (page + w * pages) holding
// frames * tok[w] tokens.  Its (head, query tile) items are [item0[w], item0[w+1]) of the launch.
struct WinView {
  int32_t n = 0;          // windows; 0 = not window mode
  int32_t frames = 0;     // latent frames per chunk
  int32_t pages = 0;      // pages per window in a slot
  int32_t bank_segs = 0;  // leading segments of the table that are banks (not window-split)
  int32_t tok[SR_MAX_LAYOUT_WINDOWS] = {};  // tokens per frame of each window
  int32_t row0[SR_MAX_LAYOUT_WINDOWS + 1] = {};
  int32_t item0[SR_MAX_LAYOUT_WINDOWS + 1] = {};
};

// Key tiles (cache pages) that query tile `qt` visits: every page of the segments before the
// last (`fixed_tiles`) plus the last segment's pages up to the last causal block that one of
// the tile's queries can see.  Query row i sees the last segment's keys j with
// floor(j / cb) <= floor(i / cb) (chunk calls: the rows are the current chunk's tokens), or
// all of them when cb == 0 (window and prefix calls).  n_q: query rows; cur_len: length of
// the last segment.
__host__ __device__ inline int32_t item_tiles(int32_t qt, int32_t fixed_tiles, int32_t n_q, int32_t cb,
                                              int32_t cur_len) {
  int32_t any = cur_len;
  if (cb > 0) {
    const int32_t end = (qt + 1) * kQueryTile < n_q ? (qt + 1) * kQueryTile : n_q;
    const int32_t blocks_end = ((end - 1) / cb + 1) * cb;
    any = blocks_end < cur_len ? blocks_end : cur_len;
  }
  return fixed_tiles + (any + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
}

// Floats of one workgroup's partial result in the split schedule: per lane of the 8 waves, 17
// eight-byte words: its output accumulators (head_dim 128 rounded to bf16, or head_dim 64 in
// fp32 or bf16) and one (max, sum) pair.
constexpr int32_t kRecordWordsPerLane = 17;
__host__ __device__ constexpr int32_t attn_record_floats(int32_t /*head_dim*/) {
  return 8 * 64 * 2 * kRecordWordsPerLane;
}

// Split schedule.  Workgroup i of a launch runs on XCD i % 8, and each XCD (own L2, C compute
// units) owns a contiguous range of the head-major (head, query tile) items, so that the query
// tiles of a head stream the same pages at about the same time and each page is fetched past
// L2 about once per XCD.  The launch has one persistent workgroup per compute unit (8 C).  XCD
// x runs a multiple of C of its items whole ("whole" items); its last `left` < C items, which
// would otherwise leave units idle in a final round, are cut into key-tile pieces ("split"
// items).  XCD x's queue holds its whole items, then piece 0 of each of its split items (the
// largest pieces, which stream the pages of heads the XCD's L2 already holds).  The later
// pieces of all XCDs' split items form one queue for the device, every item's piece 1 first,
// then every piece 2, and so on, so that the queue ends in the smallest pieces whichever XCD is
// late.  A workgroup takes the next unit of its own XCD's queue through an atomic counter, then
// of the other XCDs' queues, then of the device's piece queue.  (With all pieces in per-XCD
// queues, an XCD that ran its whole items more slowly than the others, by several per cent
// depending on the data it streams, took its own big pieces late and ended up to 120 us after
// them; with all pieces in the device queue, the first pieces ran on other XCDs than the one
// holding their pages, 0.7% slower on 456 items of 128 tiles.)  Piece k of split item r of XCD
// x leaves a partial record in slot (x C + r) kMaxPieces + k; the last piece of an item to
// finish merges the item's records in slot order and writes its output, so the result does not
// depend on which workgroup ran which piece.
constexpr int32_t kMaxCusPerXcd = 64;  // largest C (split items per XCD are fewer)
constexpr int32_t kMaxPieces = 8;      // pieces of a split item (record slots r kMaxPieces + k)
constexpr int32_t kMinPiece = 8;       // key tiles below which the rest of an item is not halved
constexpr int32_t kQueueCounters = 16; // per call: 8 whole-item queues, exit, piece queue, padding
constexpr int32_t kExitCounter = 8, kPieceCounter = 9;

// First key tile of piece k (0 .. kMaxPieces) of a split item of T tiles when the XCD's split
// work is `share` tiles per compute unit: piece 0 takes 85% of the share (the largest unit a
// unit can take without running past the others), then each piece takes half of what is left
// while that half is at least kMinPiece tiles, and the last piece takes the rest
// (piece_begin(T, share, k) = T past the last piece).  Piece 0 may take the whole item.
__host__ __device__ inline int32_t piece_begin(int32_t T, int32_t share, int32_t k) {
  if (k <= 0) return 0;
  int32_t b = share * 85 / 100;
  b = b < 1 ? 1 : (b > T ? T : b);
  for (int32_t j = 1; j < k; ++j) {  // piece j starts at b
    const int32_t half = (T - b) / 2;
    if (half < kMinPiece || j == kMaxPieces - 1) return T;  // piece j is the last
    b += half;
  }
  return b;
}
// Non-empty pieces of a split item of T tiles.
__host__ __device__ inline int32_t split_pieces(int32_t T, int32_t share) {
  int32_t n = 0;
  for (int32_t k = 0; k < kMaxPieces; ++k) n += piece_begin(T, share, k + 1) > piece_begin(T, share, k);
  return n;
}

// Even ("fan") split for launches with fewer (head, query tile) items than compute units, where
// the queues above would leave most units idle (a one-GPU share of a head-sharded run):
// each item's key tiles are cut into P equal pieces, P at most the units per item, every piece
// at least kFanMinTiles long (twice the measured start-and-finish cost of a piece), and P at
// most kFanMaxPieces (the merging piece reads the records one after the other, about a
// quarter tile-time each).  Piece p of item i leaves its record in slot i P + p; the item's
// last piece to arrive (counter i) merges them in slot order.  Returns P, or 1 for no fan split.
constexpr int32_t kFanMinTiles = 8;
constexpr int32_t kFanMaxPieces = 32;
inline int32_t fan_pieces(int32_t n_items, int32_t min_tiles, int32_t C) {
  const int32_t units = 8 * C;
  if (n_items <= 0 || n_items >= units) return 1;
  int32_t p = units / n_items;
  if (p > min_tiles / kFanMinTiles) p = min_tiles / kFanMinTiles;
  if (p > kFanMaxPieces) p = kFanMaxPieces;
  return p < 2 ? 1 : p;
}

// C of the split schedule for a device with num_cus compute units.
inline int32_t split_cus_per_xcd(int32_t num_cus) {
  const int32_t C = num_cus / 8;
  return C < 1 ? 1 : (C > kMaxCusPerXcd ? kMaxCusPerXcd : C);
}

// Attention workspace: 8 XCDs x C x kMaxPieces records, then 8C arrival counters and the split
// schedule's kQueueCounters queue counters (256-byte aligned).
inline size_t attn_records_bytes(int32_t head_dim, int32_t num_cus) {
  return size_t(8) * kMaxPieces * split_cus_per_xcd(num_cus) * attn_record_floats(head_dim) * sizeof(float);
}
inline size_t attn_counters_bytes(int32_t num_cus) {
  return ((size_t(8) * split_cus_per_xcd(num_cus) + kQueueCounters) * sizeof(int32_t) + 255) & ~size_t(255);
}

// Split schedule of one call (see launch_attention): the XCD width and where partial results go.
struct SplitWorkspace {
  int32_t cus_per_xcd = 0;      // 0 = one workgroup per (head, query tile), no workspace
  float* records = nullptr;
  int32_t* counters = nullptr;  // zero between calls
};

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

// Copies n tokens of K/V ([n][H][D], token-major) into pages [page0, page0 + npages) of
// every head, K as rows and V transposed, and zeroes those pages past token n.
hipError_t launch_append(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0,
                         int32_t npages, hipStream_t st);
// The same for a chunk packed window by window: window w's rows [row0[w], row0[w+1]) go to pages
// [page0 + w * pages, page0 + (w+1) * pages), zeroed past its tokens.  One launch.
hipError_t launch_append_windows(const Layout& L, void* pool, const void* k, const void* v, const WinView& win,
                                 int32_t page0, hipStream_t st);

// Rotary table of one call: for rotation pair j (features 2j, 2j+1), the position axis it
// follows (0 time, 1 y, 2 x) and its angle per unit of position.
struct RopeTable {
  double theta[64];
  int32_t axis[64];
};

// Fused qk-RMSNorm + rotary embedding + cache write: qkv [n][3][H][D], positions [n][3];
// writes the normalised, rotated queries to qout [n][H][D] and the normalised, rotated keys
// and the values into pages [page0, page0 + npages) of every head (zeros past token n).
hipError_t launch_prep_append(const Layout& L, void* pool, const void* qkv, const int32_t* pos, int32_t n,
                              const float* gq, const float* gk, float eps, const RopeTable& rt, void* qout,
                              int32_t page0, int32_t npages, hipStream_t st);

// Writes the logical sequence of `t` ([ntok][H][D], token-major) to kout / vout.  win (or
// nullptr): segments past win->bank_segs are chunks of a windowed cache, read window by window.
hipError_t launch_gather(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                         const WinView* win, hipStream_t st);

// Attention of n_q query rows q over the key segments of t (pages of `pool`), the last
// segment seen per causal block of cb rows (cb == 0: whole; see item_tiles).  With
// ws.cus_per_xcd > 0 the split schedule (queues of units, see above) is used.  win (or nullptr): window mode
// (WinView; n_q is then the packed row count, cb 0, no split).
hipError_t launch_attention(const Layout& L, const void* pool, const SegTable& t, int32_t n_q, int32_t cb,
                            const void* q, void* o, float* lse, float softmax_scale, const SplitWorkspace& ws,
                            hipStream_t st, const WinView* win = nullptr);

// Split-K attention of at most kFewRows query rows (bf16 caches, head_dim 64 or 128, a
// workspace attached): every segment of t visible to every row, one workgroup per (head, two
// pages), records merged by each head's last workgroup (few_attention.hip).
constexpr int32_t kFewRows = 32;
bool few_attention_fits(const Layout& L, const SegTable& t, int32_t n_q, const SplitWorkspace& ws);
hipError_t launch_few_attention(const Layout& L, const void* pool, const SegTable& t, int32_t n_q, const void* q,
                                void* o, float* lse, float softmax_scale, const SplitWorkspace& ws, hipStream_t st);

// Dense bf16 MFMA probe (probe.hip): `workgroups` workgroups of kProbeThreads threads, each
// running 4 chains of `iters` 32x32x16 MFMAs; writes one float per thread to out.
constexpr int32_t kProbeThreads = 512;
constexpr int32_t kProbeChains = 4;
hipError_t launch_mfma_probe(float* out, int32_t workgroups, int32_t iters, hipStream_t st);

// Global-to-LDS read probe (probe.hip): reads `bytes` of src (a whole number of kLdsProbeBlock
// blocks) once with global_load_lds_dwordx4, one block per workgroup of kLdsProbeThreads threads,
// each thread writing one float to out.
constexpr int32_t kLdsProbeBlock = 65536;
constexpr int32_t kLdsProbeThreads = 256;
hipError_t launch_lds_read_probe(const void* src, int64_t bytes, float* out, hipStream_t st);

// Library-owned scratch of sr_global_attention_static (static_scratch.hip): records of the
// split-K global-token kernel (at most kStaticRecordFloats floats: 4 MiB) and kStaticCounters
// arrival counters.  Fills *ws with this device's copy (looked up, and its counters zeroed on
// stream st, on the device's first call).
constexpr int32_t kStaticRecordFloats = 1 << 20;
constexpr int32_t kStaticCounters = 4096;
hipError_t static_scratch_workspace(SplitWorkspace* ws, hipStream_t st);
// Records (floats) and counters the few-row kernel needs for n_q rows over the pages of t.
int64_t few_attention_record_floats(const Layout& L, const SegTable& t, int32_t n_q);
// The few-row kernel can take the call at all (bf16, head_dim 64 or 128, 1..kFewRows rows, the
// wave-merge buffer holds the rows), whatever workspace it gets.
bool few_attention_shape_ok(const Layout& L, const SegTable& t, int32_t n_q);

}  // namespace sr
