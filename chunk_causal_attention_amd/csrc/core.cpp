// Host core: errors, layout, ring state machine (see core.hpp and sr.h).
#include "core.hpp"

#include <cstdarg>
#include <cstdio>
#include <new>

namespace sr {

static thread_local char g_err[512];

sr_status fail(sr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

const char* last_error() { return g_err; }

static int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

sr_status make_layout(const sr_kvcache_config* cfg, Layout* out) {
  if (!cfg || !out) return fail(SR_E_INVALID, "null config or output");
  const sr_kvcache_config& c = *cfg;
  if (c.dtype != SR_BF16 && c.dtype != SR_F32 && c.dtype != SR_MX)
    return fail(SR_E_INVALID, "dtype %d is not SR_BF16, SR_F32 or SR_MX", c.dtype);
  if (c.num_heads < 1 || c.num_heads > 4096) return fail(SR_E_INVALID, "num_heads %d outside [1, 4096]", c.num_heads);
  if (c.head_dim != 64 && c.head_dim != 128) return fail(SR_E_UNSUPPORTED, "head_dim %d: only 64 and 128", c.head_dim);
  if (c.dtype == SR_F32 && c.head_dim != 64) return fail(SR_E_UNSUPPORTED, "SR_F32 supports head_dim 64 only");
  if (c.persistent_tokens < 0 || c.persistent_tokens > (1 << 24))
    return fail(SR_E_INVALID, "persistent_tokens %d outside [0, 2^24]", c.persistent_tokens);
  if (c.num_banks < 1 || c.num_banks > 64) return fail(SR_E_INVALID, "num_banks %d outside [1, 64]", c.num_banks);
  if (c.chunk_capacity < 1 || c.chunk_capacity > (1 << 24))
    return fail(SR_E_INVALID, "chunk_capacity %d outside [1, 2^24]", c.chunk_capacity);
  if (c.window_chunks < 0 || c.window_chunks > SR_MAX_WINDOW)
    return fail(SR_E_INVALID, "window_chunks %d outside [0, %d]", c.window_chunks, SR_MAX_WINDOW);
  if (c.causal_block < 1) return fail(SR_E_INVALID, "causal_block %d < 1", c.causal_block);

  Layout L;
  L.H = c.num_heads;
  L.D = c.head_dim;
  L.P = c.persistent_tokens;
  L.banks = c.num_banks;
  L.cap = c.chunk_capacity;
  L.W = c.window_chunks;
  L.cb = c.causal_block;
  L.dtype = c.dtype;
  L.esize = c.dtype == SR_F32 ? 4 : 2;  // element size of the token-major inputs and outputs
  L.pages_per_bank = ceil_div(L.P, SR_PAGE_TOKENS);
  L.pages_per_slot = ceil_div(L.cap, SR_PAGE_TOKENS);
  const int64_t pages = int64_t(L.banks) * L.pages_per_bank + int64_t(L.W + 1) * L.pages_per_slot;
  if (pages > (int64_t(1) << 30) / SR_PAGE_TOKENS) return fail(SR_E_INVALID, "pool of %lld pages is too large", (long long)pages);
  L.total_pages = static_cast<int32_t>(pages);
  if (c.dtype == SR_MX) {
    L.kpage_bytes = mx_kpage_bytes(L.D);
    L.vpage_bytes = mx_vpage_bytes(L.D);
  } else {
    L.kpage_bytes = L.vpage_bytes = size_t(SR_PAGE_TOKENS) * size_t(L.D) * size_t(L.esize);
  }
  L.half_bytes = size_t(L.H) * size_t(L.total_pages) * L.kpage_bytes;
  L.bytes = L.half_bytes + size_t(L.H) * size_t(L.total_pages) * L.vpage_bytes;
  *out = L;
  return SR_OK;
}

sr_status plan_append(const sr_ring& r, int64_t chunk_id, int32_t n_tokens, int32_t* slot, int64_t* committed) {
  if (chunk_id < 0 || chunk_id == INT64_MAX) return fail(SR_E_INVALID, "chunk_id %lld out of range", (long long)chunk_id);
  if (n_tokens < 1 || n_tokens > r.L.cap)
    return fail(SR_E_INVALID, "n_tokens %d outside [1, chunk_capacity=%d]", n_tokens, r.L.cap);
  int64_t com = -1;
  if (r.has_current && chunk_id != r.cur_id) {
    if (chunk_id != r.cur_id + 1)
      return fail(SR_E_INVALID, "chunk_id %lld: expected %lld (next step) or %lld (next chunk)", (long long)chunk_id,
                  (long long)r.cur_id, (long long)(r.cur_id + 1));
    if (r.L.W > 0 && r.hist_count == r.L.W)
      return fail(SR_E_STATE, "window holds %d chunks: evict before appending chunk %lld", r.L.W, (long long)chunk_id);
    com = r.L.W > 0 ? r.cur_id : -1;
  }
  if (slot) *slot = r.slot_of(chunk_id);
  if (committed) *committed = com;
  return SR_OK;
}

void commit_append(sr_ring& r, int64_t chunk_id, int32_t n_tokens) {
  if (r.has_current && chunk_id == r.cur_id + 1 && r.L.W > 0) {
    r.hist_id[r.hist_count] = r.cur_id;
    r.hist_len[r.hist_count] = r.cur_len;
    ++r.hist_count;
  }
  r.has_current = true;
  r.cur_id = chunk_id;
  r.cur_len = n_tokens;
}

sr_status plan_update(const sr_ring& r, int64_t chunk_id, int32_t n_tokens, int32_t* slot) {
  if (n_tokens < 1 || n_tokens > r.L.cap)
    return fail(SR_E_INVALID, "n_tokens %d outside [1, chunk_capacity=%d]", n_tokens, r.L.cap);
  bool resident = r.has_current && chunk_id == r.cur_id;
  for (int i = 0; i < r.hist_count && !resident; ++i) resident = r.hist_id[i] == chunk_id;
  if (!resident) return fail(SR_E_INVALID, "chunk %lld is not in the window", (long long)chunk_id);
  if (slot) *slot = r.slot_of(chunk_id);
  return SR_OK;
}

void commit_update(sr_ring& r, int64_t chunk_id, int32_t n_tokens) {
  if (r.has_current && chunk_id == r.cur_id) {
    r.cur_len = n_tokens;
    return;
  }
  for (int i = 0; i < r.hist_count; ++i)
    if (r.hist_id[i] == chunk_id) r.hist_len[i] = n_tokens;
}

int32_t moving_tokens(const sr_ring& r) {
  int32_t n = r.has_current ? r.cur_len : 0;
  for (int i = 0; i < r.hist_count; ++i) n += r.hist_len[i];
  return n;
}

}  // namespace sr

extern "C" {

sr_status sr_ring_create(const sr_kvcache_config* cfg, sr_ring** out) {
  sr::clear_error();
  if (!out) return sr::fail(SR_E_INVALID, "null output pointer");
  sr::Layout L;
  sr_status st = sr::make_layout(cfg, &L);
  if (st != SR_OK) return st;
  sr_ring* r = new (std::nothrow) sr_ring;
  if (!r) return sr::fail(SR_E_NOMEM, "host allocation failed");
  r->L = L;
  *out = r;
  return SR_OK;
}

sr_status sr_ring_append(sr_ring* r, int64_t chunk_id, int32_t n_tokens, int32_t* slot, int64_t* committed_id) {
  sr::clear_error();
  if (!r) return sr::fail(SR_E_INVALID, "null ring");
  int32_t s;
  int64_t com;
  sr_status st = sr::plan_append(*r, chunk_id, n_tokens, &s, &com);
  if (st != SR_OK) return st;
  sr::commit_append(*r, chunk_id, n_tokens);
  if (slot) *slot = s;
  if (committed_id) *committed_id = com;
  return SR_OK;
}

sr_status sr_ring_update(sr_ring* r, int64_t chunk_id, int32_t n_tokens, int32_t* slot) {
  sr::clear_error();
  if (!r) return sr::fail(SR_E_INVALID, "null ring");
  int32_t s;
  sr_status st = sr::plan_update(*r, chunk_id, n_tokens, &s);
  if (st != SR_OK) return st;
  sr::commit_update(*r, chunk_id, n_tokens);
  if (slot) *slot = s;
  return SR_OK;
}

sr_status sr_ring_evict(sr_ring* r, int64_t* evicted_id) {
  sr::clear_error();
  if (!r) return sr::fail(SR_E_INVALID, "null ring");
  if (r->hist_count == 0) return sr::fail(SR_E_STATE, "no history chunk to evict");
  const int64_t id = r->hist_id[0];
  for (int i = 1; i < r->hist_count; ++i) {
    r->hist_id[i - 1] = r->hist_id[i];
    r->hist_len[i - 1] = r->hist_len[i];
  }
  --r->hist_count;
  if (evicted_id) *evicted_id = id;
  return SR_OK;
}

sr_status sr_ring_segments(const sr_ring* r, int32_t bank, sr_segment* out, int32_t max, int32_t* n) {
  sr::clear_error();
  if (!r || !n || (!out && max > 0)) return sr::fail(SR_E_INVALID, "null argument");
  if (bank < 0 || bank >= r->L.banks) return sr::fail(SR_E_INVALID, "bank %d outside [0, %d)", bank, r->L.banks);
  if (!r->has_current) return sr::fail(SR_E_STATE, "no current chunk");
  const int32_t count = (r->L.P > 0 ? 1 : 0) + r->hist_count + 1;
  if (max < count) return sr::fail(SR_E_INVALID, "need room for %d segments, got %d", count, max);
  int32_t k = 0;
  if (r->L.P > 0) out[k++] = sr_segment{-1, SR_SEG_PERSISTENT, bank, r->L.bank_page(bank), r->L.P};
  for (int i = 0; i < r->hist_count; ++i) {
    const int32_t s = r->slot_of(r->hist_id[i]);
    out[k++] = sr_segment{r->hist_id[i], SR_SEG_HISTORY, s, r->L.slot_page(s), r->hist_len[i]};
  }
  const int32_t s = r->slot_of(r->cur_id);
  out[k++] = sr_segment{r->cur_id, SR_SEG_CURRENT, s, r->L.slot_page(s), r->cur_len};
  *n = k;
  return SR_OK;
}

sr_status sr_ring_destroy(sr_ring* r) {
  sr::clear_error();
  delete r;
  return SR_OK;
}

const char* sr_status_string(sr_status s) {
  switch (s) {
    case SR_OK: return "SR_OK";
    case SR_E_INVALID: return "SR_E_INVALID";
    case SR_E_STATE: return "SR_E_STATE";
    case SR_E_NOMEM: return "SR_E_NOMEM";
    case SR_E_DEVICE: return "SR_E_DEVICE";
    case SR_E_UNSUPPORTED: return "SR_E_UNSUPPORTED";
  }
  return "SR_E_UNKNOWN";
}

const char* sr_last_error(void) { return sr::last_error(); }

sr_status sr_kvcache_required_bytes(const sr_kvcache_config* cfg, size_t* bytes) {
  sr::clear_error();
  if (!bytes) return sr::fail(SR_E_INVALID, "null output pointer");
  sr::Layout L;
  sr_status st = sr::make_layout(cfg, &L);
  if (st != SR_OK) return st;
  *bytes = L.bytes;
  return SR_OK;
}

}  // extern "C"
