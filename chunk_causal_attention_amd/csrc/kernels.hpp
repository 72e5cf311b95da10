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

// Floats of one workgroup's partial result in the split schedule: per lane of the 8 waves,
// the head_dim/2 output accumulators it holds plus its running max and sum, padded to
// whole 16-byte chunks.
__host__ __device__ constexpr int32_t attn_record_floats(int32_t head_dim) { return 8 * 64 * (head_dim / 2 + 4); }

// Split schedule.  Workgroup i of a launch runs on XCD i % 8 as that XCD's (i / 8)-th
// workgroup, and each XCD (own L2, C compute units) gets a contiguous range of the head-major
// (head, query tile) items.  An XCD runs its items whole, C at a time: the query tiles of a
// head then stream the same pages at the same time, so each page is fetched past L2 about
// once per XCD.  The last `left` < C items of an XCD would leave units idle in a final round;
// instead, split workgroup r < left runs tiles [0, min(b, T_r)) of split item r ("band 0"),
// and the remaining tiles [b, T_r) of all split items, laid out one item after the other
// ("band 1"), are dealt in runs of s tiles to the other split workgroups.  Band-0 workgroups
// stream the same pages together, and so do band-1 workgroups.  A band-1 piece is at most s
// long (the plan guarantees it), so it is cut by at most one workgroup boundary: sub-piece 0
// and possibly 1.  Every piece of a split item leaves a partial record, in slot
// x * 4C + 2r (band 0) or x * 4C + 2C + 2r + sub (band 1); the last piece of an item to
// finish merges the item's records in slot order and writes its output.
constexpr int32_t kPieceOverheadTiles = 4;  // measured cost of starting and ending a piece
constexpr int32_t kMaxCusPerXcd = 64;       // largest C (split items per XCD are fewer)

struct XcdPlan {
  int32_t first;  // first item of the XCD
  int32_t whole;  // items run whole (a multiple of C, or 0)
  int32_t left;   // split items (< C), items first + whole ...
  int32_t b;      // band-0 width
  int32_t s;      // band-1 tiles per workgroup (0: no band 1)
  int32_t u1;     // band-1 tiles in all
  int32_t wgs;    // split workgroups: left band-0 + ceil(u1 / s) band-1
};

__host__ __device__ inline int32_t band1_len(int32_t t, int32_t b) { return t > b ? t - b : 0; }

// Estimated duration (tiles, plus kPieceOverheadTiles per piece) of the split round of an
// XCD for band-0 width b; -1 if band 1 would need a run shorter than one of its pieces.
inline int32_t split_estimate(const int16_t* T, int32_t left, int32_t C, int32_t b, int32_t* s_out, int32_t* u1_out) {
  int32_t u1 = 0, maxlen = 0, band0 = 0;
  for (int32_t r = 0; r < left; ++r) {
    const int32_t l1 = band1_len(T[r], b);
    u1 += l1;
    maxlen = l1 > maxlen ? l1 : maxlen;
    const int32_t l0 = T[r] < b ? T[r] : b;
    band0 = l0 > band0 ? l0 : band0;
  }
  *u1_out = u1;
  *s_out = 0;
  int32_t worst = band0 + kPieceOverheadTiles;
  if (u1 == 0) return worst;
  const int32_t s = (u1 + (C - left) - 1) / (C - left);
  if (s < maxlen) return -1;
  *s_out = s;
  // Pieces overlapping each run [q s, (q+1) s): two pointers over the band-1 pieces.
  int32_t i = 0, start = 0;  // piece i starts at unit `start`
  for (int32_t lo = 0; lo < u1; lo += s) {
    const int32_t hi = lo + s < u1 ? lo + s : u1;
    while (i < left && start + band1_len(T[i], b) <= lo) start += band1_len(T[i++], b);
    int32_t n = 0;
    for (int32_t k = i, a = start; k < left && a < hi; a += band1_len(T[k++], b)) n += band1_len(T[k], b) > 0;
    const int32_t w = (hi - lo) + n * kPieceOverheadTiles;
    worst = w > worst ? w : worst;
  }
  return worst;
}

// Plan of XCD x; T receives the tile counts of its split items.
inline XcdPlan xcd_plan(int32_t x, int32_t n_items, int32_t q_tiles, int32_t fixed_tiles, int32_t n_q, int32_t cb,
                        int32_t cur_len, int32_t C, int16_t* T) {
  XcdPlan p{};
  p.first = int32_t(int64_t(x) * n_items / 8);
  const int32_t n = int32_t(int64_t(x + 1) * n_items / 8) - p.first;
  p.left = n % C;
  p.whole = n - p.left;
  if (p.left == 0) return p;
  int32_t tmax = 0;
  for (int32_t r = 0; r < p.left; ++r) {
    T[r] = int16_t(item_tiles((p.first + p.whole + r) % q_tiles, fixed_tiles, n_q, cb, cur_len));
    tmax = T[r] > tmax ? T[r] : tmax;
  }
  // Best b: every stride-th candidate, then the neighbours of the best one.
  int32_t best = -1, best_b = tmax;
  auto consider = [&](int32_t b) {
    if (b < 1 || b > tmax) return;
    int32_t s, u1;
    const int32_t e = split_estimate(T, p.left, C, b, &s, &u1);
    if (e >= 0 && (best < 0 || e < best || (e == best && b > best_b))) {
      best = e;
      best_b = b;
    }
  };
  const int32_t stride = tmax / 64 > 1 ? tmax / 64 : 1;
  for (int32_t b = 1; b <= tmax; b += stride) consider(b);
  consider(tmax);
  for (int32_t d = -stride; d <= stride; ++d) consider(best_b + d);
  // Split only if it saves at least 1/16 of running the items whole.
  const int32_t whole_cost = tmax + kPieceOverheadTiles / 2;
  if (best < 0 || best > whole_cost - (whole_cost >> 4)) best_b = tmax;
  p.b = best_b;
  split_estimate(T, p.left, C, p.b, &p.s, &p.u1);
  p.wgs = p.left + (p.u1 > 0 ? (p.u1 + p.s - 1) / p.s : 0);
  return p;
}

// Even ("fan") split for launches with fewer (head, query tile) items than compute units, where
// the two-band plan above would leave most units idle (a one-GPU share of a head-sharded run):
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

// Attention workspace: 8 XCDs x 4C records, then 8C arrival counters (256-byte aligned).
inline size_t attn_records_bytes(int32_t head_dim, int32_t num_cus) {
  return size_t(8) * 4 * split_cus_per_xcd(num_cus) * attn_record_floats(head_dim) * sizeof(float);
}
inline size_t attn_counters_bytes(int32_t num_cus) {
  return (size_t(8) * split_cus_per_xcd(num_cus) * sizeof(int32_t) + 255) & ~size_t(255);
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
// ws.cus_per_xcd > 0 the split schedule (xcd_plan) is used.  win (or nullptr): window mode
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
