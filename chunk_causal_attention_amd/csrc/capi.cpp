// C ABI of the KV cache and the attention call (declared in sr.h).  Host-side validation
// happens before anything is enqueued; see the conventions at the top of sr.h.
#include <algorithm>
#include <cmath>
#include <new>

#include <hip/hip_runtime.h>

#include "core.hpp"
#include "kernels.hpp"

struct sr_kvcache {
  sr_ring ring;
  char* pool = nullptr;
  int32_t num_cus = 0;        // compute units of the device the cache was created on
  sr::SplitWorkspace split;   // grid 0: no workspace attached
  size_t ws_bytes = 0;
  bool windowed = false;      // a window layout is set (sr_kvcache_set_window_layout)
  sr::WinView win;            // the layout with its prefix sums; bank_segs = (P > 0)
};

namespace {

sr_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SR_OK;
  return sr::fail(SR_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Segment table of a call on `bank` (ring must have a current chunk).
sr::SegTable make_table(const sr_ring& r, int32_t bank, int32_t* total) {
  sr_segment segs[sr::kMaxSegs];
  int32_t n = 0;
  sr_ring_segments(&r, bank, segs, sr::kMaxSegs, &n);
  sr::SegTable t{};
  t.n = n;
  int32_t sum = 0;
  for (int i = 0; i < n; ++i) {
    t.s[i] = sr::DevSeg{segs[i].page, segs[i].length};
    sum += segs[i].length;
  }
  if (total) *total = sum;
  return t;
}

bool pool_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

sr_status device_cus(int32_t* n) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_status(e, "device query");
  if (cus <= 0) return sr::fail(SR_E_DEVICE, "device reports %d compute units", cus);
  *n = cus;
  return SR_OK;
}

// Checks shared by the attention calls (before anything is enqueued).
sr_status check_attention_args(const sr_kvcache* c, int32_t bank, const void* q, const void* out, const float* lse,
                               float softmax_scale) {
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  if (!q || !out || !sr::aligned16(q) || !sr::aligned16(out))
    return sr::fail(SR_E_INVALID, "q and out must be non-null and 16-byte aligned");
  if (q == out) return sr::fail(SR_E_INVALID, "q must not alias out");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return sr::fail(SR_E_INVALID, "lse must be 4-byte aligned");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return sr::fail(SR_E_INVALID, "softmax_scale must be finite and > 0");
  const sr::Layout& L = c->ring.L;
  if (bank < 0 || bank >= L.banks) return sr::fail(SR_E_INVALID, "bank %d outside [0, %d)", bank, L.banks);
  return SR_OK;
}

// Calls that treat a chunk as one contiguous run of tokens do not apply to a windowed cache.
sr_status check_not_windowed(const sr_kvcache* c) {
  if (c->windowed) return sr::fail(SR_E_STATE, "the cache has a window layout: use the window calls");
  return SR_OK;
}

sr_status check_pages(const sr::SegTable& t) {
  int32_t pages = 0;
  for (int i = 0; i < t.n; ++i) pages += (t.s[i].len + SR_PAGE_TOKENS - 1) / SR_PAGE_TOKENS;
  if (pages > SR_MAX_VISIBLE_PAGES)
    return sr::fail(SR_E_UNSUPPORTED, "the call visits %d pages of keys, more than %d", pages, SR_MAX_VISIBLE_PAGES);
  return SR_OK;
}

}  // namespace

extern "C" {

sr_status sr_kvcache_init(const sr_kvcache_config* cfg, void* pool, size_t pool_bytes, const void* persistent_k,
                          const void* persistent_v, void* stream, sr_kvcache** out) {
  sr::clear_error();
  if (!out) return sr::fail(SR_E_INVALID, "null output pointer");
  sr::Layout L;
  sr_status st = sr::make_layout(cfg, &L);
  if (st != SR_OK) return st;
  if (!pool || !pool_aligned(pool)) return sr::fail(SR_E_INVALID, "pool must be non-null and 256-byte aligned");
  if (pool_bytes < L.bytes)
    return sr::fail(SR_E_NOMEM, "pool has %zu bytes, the layout needs %zu", pool_bytes, L.bytes);
  if (L.P > 0 && (!persistent_k || !persistent_v || !sr::aligned16(persistent_k) || !sr::aligned16(persistent_v)))
    return sr::fail(SR_E_INVALID, "persistent K/V must be non-null and 16-byte aligned when persistent_tokens > 0");
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != SR_OK) return st;
  sr_kvcache* c = new (std::nothrow) sr_kvcache;
  if (!c) return sr::fail(SR_E_NOMEM, "host allocation failed");
  c->ring.L = L;
  c->pool = static_cast<char*>(pool);
  c->num_cus = cus;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = device_status(sr::launch_zero(pool, L.bytes, s), "pool zero");
  const size_t bank_elems = size_t(L.P) * L.H * L.D;
  for (int b = 0; st == SR_OK && b < L.banks && L.P > 0; ++b) {
    const char* pk = static_cast<const char*>(persistent_k) + b * bank_elems * L.esize;
    const char* pv = static_cast<const char*>(persistent_v) + b * bank_elems * L.esize;
    st = device_status(sr::launch_append(L, pool, pk, pv, L.P, L.bank_page(b), L.pages_per_bank, s), "bank copy");
  }
  if (st != SR_OK) {
    delete c;
    return st;
  }
  *out = c;
  return SR_OK;
}

sr_status sr_kvcache_append_chunk(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v, int32_t n_tokens,
                                  void* stream) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  if (!k || !v || !sr::aligned16(k) || !sr::aligned16(v))
    return sr::fail(SR_E_INVALID, "chunk K/V must be non-null and 16-byte aligned");
  sr_status st = check_not_windowed(c);
  if (st != SR_OK) return st;
  int32_t slot;
  int64_t committed;
  st = sr::plan_append(c->ring, chunk_id, n_tokens, &slot, &committed);
  if (st != SR_OK) return st;
  const sr::Layout& L = c->ring.L;
  st = device_status(sr::launch_append(L, c->pool, k, v, n_tokens, L.slot_page(slot), L.pages_per_slot,
                                       static_cast<hipStream_t>(stream)),
                     "chunk append");
  if (st != SR_OK) return st;
  sr::commit_append(c->ring, chunk_id, n_tokens);
  return SR_OK;
}

sr_status sr_kvcache_append_qkv(sr_kvcache* c, int64_t chunk_id, const void* qkv, const int32_t* positions,
                                int32_t n_tokens, const float* q_gain, const float* k_gain, const sr_qk_prep* prep,
                                void* q_out, void* stream) {
  sr::clear_error();
  if (!c || !prep) return sr::fail(SR_E_INVALID, "null cache or parameters");
  if (!qkv || !q_out || !sr::aligned16(qkv) || !sr::aligned16(q_out))
    return sr::fail(SR_E_INVALID, "qkv and q_out must be non-null and 16-byte aligned");
  if (!positions || !q_gain || !k_gain || (reinterpret_cast<uintptr_t>(positions) & 3u) ||
      (reinterpret_cast<uintptr_t>(q_gain) & 3u) || (reinterpret_cast<uintptr_t>(k_gain) & 3u))
    return sr::fail(SR_E_INVALID, "positions and gains must be non-null and 4-byte aligned");
  const sr::Layout& L = c->ring.L;
  if (L.dtype == SR_MX) return sr::fail(SR_E_UNSUPPORTED, "the fused qkv append is not available for SR_MX caches");
  if (c->windowed) return check_not_windowed(c);
  const int32_t pairs = L.D / 2;
  const int32_t* sec = prep->rope_sections;
  if (sec[0] < 0 || sec[1] < 0 || sec[2] < 0 || sec[0] + sec[1] + sec[2] != pairs)
    return sr::fail(SR_E_INVALID, "rope_sections (%d, %d, %d) must be >= 0 and sum to head_dim / 2 = %d", sec[0],
                    sec[1], sec[2], pairs);
  if (!(prep->rope_base > 1.0f) || !std::isfinite(prep->rope_base))
    return sr::fail(SR_E_INVALID, "rope_base must be finite and > 1");
  if (!(prep->rms_eps >= 0.0f) || !std::isfinite(prep->rms_eps))
    return sr::fail(SR_E_INVALID, "rms_eps must be finite and >= 0");
  int32_t slot;
  int64_t committed;
  sr_status st = sr::plan_append(c->ring, chunk_id, n_tokens, &slot, &committed);
  if (st != SR_OK) return st;
  // q_out [n][H][D] must not overlap the qkv rows the kernel still reads.
  const size_t row = size_t(L.H) * L.D * L.esize;
  const char* a0 = static_cast<const char*>(qkv);
  const char* b0 = static_cast<const char*>(q_out);
  if (b0 < a0 + 3 * row * n_tokens && a0 < b0 + row * n_tokens)
    return sr::fail(SR_E_INVALID, "q_out must not overlap qkv");
  sr::RopeTable rt{};
  for (int32_t j = 0, a = 0, k = 0; j < pairs; ++j, ++k) {
    while (k >= sec[a]) {
      k = 0;
      ++a;
    }
    rt.axis[j] = a;
    rt.theta[j] = std::pow(double(prep->rope_base), -double(k) / double(sec[a]));
  }
  st = device_status(sr::launch_prep_append(L, c->pool, qkv, positions, n_tokens, q_gain, k_gain, prep->rms_eps, rt,
                                            q_out, L.slot_page(slot), L.pages_per_slot,
                                            static_cast<hipStream_t>(stream)),
                     "qkv append");
  if (st != SR_OK) return st;
  sr::commit_append(c->ring, chunk_id, n_tokens);
  return SR_OK;
}

sr_status sr_kvcache_evict(sr_kvcache* c, int64_t* evicted_chunk_id) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  return sr_ring_evict(&c->ring, evicted_chunk_id);
}

sr_status sr_chunk_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse, float softmax_scale,
                             void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st == SR_OK) st = check_not_windowed(c);
  if (st != SR_OK) return st;
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk: append one first");
  const sr::SegTable t = make_table(c->ring, bank, nullptr);
  st = check_pages(t);
  if (st != SR_OK) return st;
  const sr::Layout& L = c->ring.L;
  return device_status(sr::launch_attention(L, c->pool, t, c->ring.cur_len, L.cb, q, out, lse, softmax_scale, c->split,
                                            static_cast<hipStream_t>(stream)),
                       "chunk attention");
}

sr_status sr_window_attention(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out, float* lse,
                              float softmax_scale, void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st == SR_OK) st = check_not_windowed(c);
  if (st != SR_OK) return st;
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk: append one first");
  const int32_t moving = sr::moving_tokens(c->ring);
  if (n_rows != moving)
    return sr::fail(SR_E_INVALID, "n_rows %d: the window's moving part (history + current) has %d tokens", n_rows,
                    moving);
  const sr::SegTable t = make_table(c->ring, bank, nullptr);
  st = check_pages(t);
  if (st != SR_OK) return st;
  return device_status(sr::launch_attention(c->ring.L, c->pool, t, n_rows, 0, q, out, lse, softmax_scale, c->split,
                                            static_cast<hipStream_t>(stream)),
                       "window attention");
}

sr_status sr_prefix_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse, float softmax_scale,
                              void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st == SR_OK) st = check_not_windowed(c);
  if (st != SR_OK) return st;
  const sr::Layout& L = c->ring.L;
  if (L.P == 0) return sr::fail(SR_E_INVALID, "the cache has no persistent tokens");
  sr::SegTable t{};
  t.n = 1;
  t.s[0] = sr::DevSeg{L.bank_page(bank), L.P};
  st = check_pages(t);
  if (st != SR_OK) return st;
  return device_status(sr::launch_attention(L, c->pool, t, L.P, 0, q, out, lse, softmax_scale, c->split,
                                            static_cast<hipStream_t>(stream)),
                       "prefix attention");
}

sr_status sr_kvcache_update_chunk(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v, int32_t n_tokens,
                                  void* stream) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  if (!k || !v || !sr::aligned16(k) || !sr::aligned16(v))
    return sr::fail(SR_E_INVALID, "chunk K/V must be non-null and 16-byte aligned");
  sr_status st = check_not_windowed(c);
  if (st != SR_OK) return st;
  int32_t slot;
  st = sr::plan_update(c->ring, chunk_id, n_tokens, &slot);
  if (st != SR_OK) return st;
  const sr::Layout& L = c->ring.L;
  st = device_status(sr::launch_append(L, c->pool, k, v, n_tokens, L.slot_page(slot), L.pages_per_slot,
                                       static_cast<hipStream_t>(stream)),
                     "chunk update");
  if (st != SR_OK) return st;
  sr::commit_update(c->ring, chunk_id, n_tokens);
  return SR_OK;
}

sr_status sr_attention_workspace_bytes(const sr_kvcache_config* cfg, int32_t num_workgroups, size_t* bytes) {
  sr::clear_error();
  if (!bytes) return sr::fail(SR_E_INVALID, "null output pointer");
  sr::Layout L;
  sr_status st = sr::make_layout(cfg, &L);
  if (st != SR_OK) return st;
  if (num_workgroups < 0) return sr::fail(SR_E_INVALID, "num_workgroups must be >= 0");
  if (num_workgroups == 0) {
    st = device_cus(&num_workgroups);
    if (st != SR_OK) return st;
  }
  *bytes = sr::attn_records_bytes(L.D, num_workgroups) + sr::attn_counters_bytes(num_workgroups);
  return SR_OK;
}

sr_status sr_kvcache_set_workspace(sr_kvcache* c, void* ws, size_t ws_bytes, void* stream) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  if (!ws) {
    c->split = sr::SplitWorkspace{};
    c->ws_bytes = 0;
    return SR_OK;
  }
  if (!pool_aligned(ws)) return sr::fail(SR_E_INVALID, "workspace must be 256-byte aligned");
  const sr::Layout& L = c->ring.L;
  const size_t rec = sr::attn_records_bytes(L.D, c->num_cus);
  const size_t need = rec + sr::attn_counters_bytes(c->num_cus);
  if (ws_bytes < need) return sr::fail(SR_E_NOMEM, "workspace has %zu bytes, the cache needs %zu", ws_bytes, need);
  char* base = static_cast<char*>(ws);
  // Counters start at zero; every attention call leaves them at zero again.
  sr_status st = device_status(sr::launch_zero(base + rec, need - rec, static_cast<hipStream_t>(stream)),
                               "workspace zero");
  if (st != SR_OK) return st;
  c->split.cus_per_xcd = sr::split_cus_per_xcd(c->num_cus);
  c->split.records = reinterpret_cast<float*>(base);
  c->split.counters = reinterpret_cast<int32_t*>(base + rec);
  c->ws_bytes = ws_bytes;
  return SR_OK;
}

sr_status sr_kvcache_gather(const sr_kvcache* c, int32_t bank, void* k_out, void* v_out, int32_t max_tokens,
                            int32_t* n_tokens, void* stream) {
  sr::clear_error();
  if (!c || !n_tokens) return sr::fail(SR_E_INVALID, "null argument");
  if (!k_out || !v_out) return sr::fail(SR_E_INVALID, "null output buffers");
  const sr::Layout& L = c->ring.L;
  if (bank < 0 || bank >= L.banks) return sr::fail(SR_E_INVALID, "bank %d outside [0, %d)", bank, L.banks);
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk");
  int32_t total = 0;
  const sr::SegTable t = make_table(c->ring, bank, &total);
  if (total > max_tokens) return sr::fail(SR_E_INVALID, "sequence has %d tokens, room for %d", total, max_tokens);
  *n_tokens = total;
  return device_status(sr::launch_gather(L, c->pool, t, total, k_out, v_out, c->windowed ? &c->win : nullptr,
                                         static_cast<hipStream_t>(stream)),
                       "gather");
}

}  // extern "C"

namespace {

// Validates a window layout against a cache geometry (host only) and fills the kernels' view.
sr_status window_view(const sr::Layout& L, const sr_window_layout& w, sr::WinView* out) {
  if (L.dtype == SR_MX) return sr::fail(SR_E_UNSUPPORTED, "window layouts are available for SR_BF16 and SR_F32 caches");
  if (w.num_windows < 1 || w.num_windows > SR_MAX_LAYOUT_WINDOWS)
    return sr::fail(SR_E_INVALID, "num_windows %d outside [1, %d]", w.num_windows, SR_MAX_LAYOUT_WINDOWS);
  if (w.frames_per_chunk < 1 || w.window_pages < 1)
    return sr::fail(SR_E_INVALID, "frames_per_chunk and window_pages must be >= 1");
  if (int64_t(w.num_windows) * w.window_pages > L.pages_per_slot)
    return sr::fail(SR_E_INVALID, "%d windows x %d pages exceed the %d pages of a slot", w.num_windows, w.window_pages,
                    L.pages_per_slot);
  sr::WinView v{};
  v.n = w.num_windows;
  v.frames = w.frames_per_chunk;
  v.pages = w.window_pages;
  v.bank_segs = L.P > 0 ? 1 : 0;
  for (int i = 0; i < v.n; ++i) {
    const int32_t tok = w.window_tokens[i];
    if (tok < 1 || int64_t(tok) * v.frames > int64_t(w.window_pages) * SR_PAGE_TOKENS)
      return sr::fail(SR_E_INVALID, "window %d: %d tokens x %d frames do not fit %d pages", i, tok, v.frames,
                      w.window_pages);
    // A window's keys of one chunk must fit the attention kernel's tile table on their own.
    if (int64_t(tok) * v.frames > int64_t(SR_MAX_VISIBLE_PAGES) * SR_PAGE_TOKENS)
      return sr::fail(SR_E_INVALID, "window %d: %d tokens x %d frames exceed the %d pages one call can visit", i, tok,
                      v.frames, SR_MAX_VISIBLE_PAGES);
    v.tok[i] = tok;
    v.row0[i + 1] = v.row0[i] + v.frames * tok;
    v.item0[i + 1] = v.item0[i] + L.H * ((v.frames * tok + sr::kQueryTile - 1) / sr::kQueryTile);
  }
  *out = v;
  return SR_OK;
}

}  // namespace

extern "C" {

sr_status sr_window_layout_check(const sr_kvcache_config* cfg, const sr_window_layout* layout) {
  sr::clear_error();
  if (!cfg || !layout) return sr::fail(SR_E_INVALID, "null config or layout");
  sr::Layout L;
  sr_status st = sr::make_layout(cfg, &L);
  if (st != SR_OK) return st;
  sr::WinView v;
  return window_view(L, *layout, &v);
}

sr_status sr_kvcache_set_window_layout(sr_kvcache* c, const sr_window_layout* layout) {
  sr::clear_error();
  if (!c || !layout) return sr::fail(SR_E_INVALID, "null cache or layout");
  if (c->windowed || c->ring.has_current || c->ring.hist_count > 0)
    return sr::fail(SR_E_STATE, "the window layout is set once, before the first append");
  sr::WinView v;
  const sr_status st = window_view(c->ring.L, *layout, &v);
  if (st != SR_OK) return st;
  c->win = v;
  c->windowed = true;
  return SR_OK;
}

sr_status sr_kvcache_set_bank(sr_kvcache* c, int32_t bank, const void* k, const void* v, void* stream) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  const sr::Layout& L = c->ring.L;
  if (bank < 0 || bank >= L.banks) return sr::fail(SR_E_INVALID, "bank %d outside [0, %d)", bank, L.banks);
  if (L.P == 0) return sr::fail(SR_E_INVALID, "the cache has no persistent tokens");
  if (!k || !v || !sr::aligned16(k) || !sr::aligned16(v))
    return sr::fail(SR_E_INVALID, "bank K/V must be non-null and 16-byte aligned");
  return device_status(sr::launch_append(L, c->pool, k, v, L.P, L.bank_page(bank), L.pages_per_bank,
                                         static_cast<hipStream_t>(stream)),
                       "bank write");
}

sr_status sr_kvcache_append_windows(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v, void* stream) {
  sr::clear_error();
  if (!c) return sr::fail(SR_E_INVALID, "null cache");
  if (!c->windowed) return sr::fail(SR_E_STATE, "no window layout: set one first");
  if (!k || !v || !sr::aligned16(k) || !sr::aligned16(v))
    return sr::fail(SR_E_INVALID, "chunk K/V must be non-null and 16-byte aligned");
  const int32_t T = c->win.row0[c->win.n];
  int32_t slot;
  int64_t committed;
  sr_status st = sr::plan_append(c->ring, chunk_id, T, &slot, &committed);
  if (st != SR_OK) return st;
  const sr::Layout& L = c->ring.L;
  st = device_status(sr::launch_append_windows(L, c->pool, k, v, c->win, L.slot_page(slot),
                                               static_cast<hipStream_t>(stream)),
                     "window append");
  if (st != SR_OK) return st;
  sr::commit_append(c->ring, chunk_id, T);
  return SR_OK;
}

sr_status sr_windows_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse, float softmax_scale,
                               void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st != SR_OK) return st;
  if (!c->windowed) return sr::fail(SR_E_STATE, "no window layout: set one first");
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk: append one first");
  const sr::SegTable t = make_table(c->ring, bank, nullptr);
  const sr::Layout& L = c->ring.L;
  // The largest window's key list: the bank pages and that window's pages of every chunk.
  int32_t most = 0;
  for (int w = 0; w < c->win.n; ++w) most = std::max(most, c->win.frames * int32_t(c->win.tok[w]));
  sr::SegTable widest = t;
  for (int s = c->win.bank_segs; s < widest.n; ++s) widest.s[s].len = most;
  st = check_pages(widest);
  if (st != SR_OK) return st;
  return device_status(sr::launch_attention(L, c->pool, t, c->win.row0[c->win.n], 0, q, out, lse, softmax_scale,
                                            sr::SplitWorkspace{}, static_cast<hipStream_t>(stream), &c->win),
                       "windows attention");
}

sr_status sr_global_attention(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out, float* lse,
                              float softmax_scale, void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st != SR_OK) return st;
  if (!c->windowed) return sr::fail(SR_E_STATE, "no window layout: set one first");
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk: append one first");
  if (n_rows < 1) return sr::fail(SR_E_INVALID, "n_rows %d < 1", n_rows);
  const sr::Layout& L = c->ring.L;
  // Keys: the bank, then every window's pages of the current chunk's slot.
  sr::SegTable t{};
  if (L.P > 0) t.s[t.n++] = sr::DevSeg{L.bank_page(bank), L.P};
  const int32_t cur_page = L.slot_page(c->ring.slot_of(c->ring.cur_id));
  for (int w = 0; w < c->win.n; ++w)
    t.s[t.n++] = sr::DevSeg{cur_page + w * c->win.pages, c->win.frames * c->win.tok[w]};
  st = check_pages(t);
  if (st != SR_OK) return st;
  if (sr::few_attention_fits(L, t, n_rows, c->split))
    return device_status(sr::launch_few_attention(L, c->pool, t, n_rows, q, out, lse, softmax_scale, c->split,
                                                  static_cast<hipStream_t>(stream)),
                         "global attention");
  return device_status(sr::launch_attention(L, c->pool, t, n_rows, 0, q, out, lse, softmax_scale, c->split,
                                            static_cast<hipStream_t>(stream)),
                       "global attention");
}

sr_status sr_probe_mfma_bf16(float* out, int32_t workgroups, int32_t iters, void* stream) {
  sr::clear_error();
  if (!out) return sr::fail(SR_E_INVALID, "null output");
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return sr::fail(SR_E_INVALID, "workgroups %d or iters %d out of range", workgroups, iters);
  return device_status(sr::launch_mfma_probe(out, workgroups, iters, static_cast<hipStream_t>(stream)), "mfma probe");
}

sr_status sr_probe_lds_read(const void* src, int64_t bytes, float* out, void* stream) {
  sr::clear_error();
  if (!src || !out) return sr::fail(SR_E_INVALID, "null buffer");
  if (bytes <= 0 || bytes % sr::kLdsProbeBlock != 0 || bytes / sr::kLdsProbeBlock > (int64_t(1) << 24))
    return sr::fail(SR_E_INVALID, "bytes %lld is not a positive multiple of %d up to 2^24 blocks",
                    static_cast<long long>(bytes), sr::kLdsProbeBlock);
  return device_status(sr::launch_lds_read_probe(src, bytes, out, static_cast<hipStream_t>(stream)), "lds probe");
}

sr_status sr_global_attention_static(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out,
                                     float* lse, float softmax_scale, void* stream) {
  sr::clear_error();
  sr_status st = check_attention_args(c, bank, q, out, lse, softmax_scale);
  if (st != SR_OK) return st;
  if (!c->windowed) return sr::fail(SR_E_STATE, "no window layout: set one first");
  if (!c->ring.has_current) return sr::fail(SR_E_STATE, "no current chunk: append one first");
  if (n_rows < 1) return sr::fail(SR_E_INVALID, "n_rows %d < 1", n_rows);
  const sr::Layout& L = c->ring.L;
  sr::SegTable t{};
  if (L.P > 0) t.s[t.n++] = sr::DevSeg{L.bank_page(bank), L.P};
  const int32_t cur_page = L.slot_page(c->ring.slot_of(c->ring.cur_id));
  for (int w = 0; w < c->win.n; ++w)
    t.s[t.n++] = sr::DevSeg{cur_page + w * c->win.pages, c->win.frames * c->win.tok[w]};
  st = check_pages(t);
  if (st != SR_OK) return st;
  if (!sr::few_attention_shape_ok(L, t, n_rows))
    return sr::fail(SR_E_UNSUPPORTED, "the static-scratch call takes bf16 caches, head_dim 64 or 128 and 1..%d rows",
                    sr::kFewRows);
  const int64_t need = sr::few_attention_record_floats(L, t, n_rows);
  if (need > sr::kStaticRecordFloats || L.H > sr::kStaticCounters)
    return sr::fail(SR_E_UNSUPPORTED,
                    "the call needs %lld floats of records for %d heads; the static scratch holds %d floats and %d heads",
                    (long long)need, L.H, sr::kStaticRecordFloats, sr::kStaticCounters);
  sr::SplitWorkspace ws;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = device_status(sr::static_scratch_workspace(&ws, s), "static scratch");
  if (st != SR_OK) return st;
  return device_status(sr::launch_few_attention(L, c->pool, t, n_rows, q, out, lse, softmax_scale, ws, s),
                       "global attention (static scratch)");
}

const sr_ring* sr_kvcache_ring(const sr_kvcache* c) { return c ? &c->ring : nullptr; }

sr_status sr_kvcache_destroy(sr_kvcache* c) {
  sr::clear_error();
  delete c;
  return SR_OK;
}

}  // extern "C"
