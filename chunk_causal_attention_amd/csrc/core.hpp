// Host core of the streaming KV cache: argument validation, pool layout, ring state machine.
// Pure C++ (no HIP calls), so it is exercised on machines without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "sr.h"

namespace sr {

// Pool geometry derived from a validated config (see the pool layout in sr.h).
struct Layout {
  int32_t H = 0, D = 0, P = 0, banks = 0, cap = 0, W = 0, cb = 0, dtype = 0, esize = 0;
  int32_t pages_per_bank = 0, pages_per_slot = 0, total_pages = 0;
  size_t kpage_bytes = 0, vpage_bytes = 0;  // one (head, page) of K / of V
  size_t half_bytes = 0;  // bytes of the K region; the V region follows at this offset
  size_t bytes = 0;       // whole pool

  int32_t bank_page(int32_t b) const { return b * pages_per_bank; }
  int32_t slot_page(int32_t s) const { return banks * pages_per_bank + s * pages_per_slot; }
  int32_t slots() const { return W + 1; }
};

// Records a thread-local message for sr_last_error() and returns `s`.
sr_status fail(sr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

sr_status make_layout(const sr_kvcache_config* cfg, Layout* out);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of one (head, page) of a reduced-precision (SR_MX) cache: K holds per token and
// 32-feature block 24 bytes of FP6 codes and one scale byte, padded to whole KiB (the
// attention kernel copies pages to LDS in 1 KiB pieces per wave); V one FP8 byte per element.
constexpr size_t mx_kpage_bytes(int32_t D) { return (size_t(D / 32) * (SR_PAGE_TOKENS * 25) + 1023) & ~size_t(1023); }
constexpr size_t mx_vpage_bytes(int32_t D) { return size_t(D) * SR_PAGE_TOKENS; }

}  // namespace sr

// Chunk bookkeeping of one cache.  History is a run of consecutive chunk ids ending just
// before the current id, so ids map to distinct ring slots id mod (W+1).
struct sr_ring {
  sr::Layout L;
  bool has_current = false;
  int64_t cur_id = -1;
  int32_t cur_len = 0;
  int32_t hist_count = 0;
  int64_t hist_id[SR_MAX_WINDOW];   // oldest first
  int32_t hist_len[SR_MAX_WINDOW];

  int32_t slot_of(int64_t id) const { return static_cast<int32_t>(id % (L.W + 1)); }
};

namespace sr {
// Validates an append without changing the ring.  On success fills the slot written
// and the id committed (-1 if none).
sr_status plan_append(const sr_ring& r, int64_t chunk_id, int32_t n_tokens, int32_t* slot, int64_t* committed);
// Applies a planned append (must follow a successful plan_append with the same arguments).
void commit_append(sr_ring& r, int64_t chunk_id, int32_t n_tokens);
// Validates an in-place update of a chunk in the window (a history chunk or the current one)
// without changing the ring; on success fills the chunk's slot.
sr_status plan_update(const sr_ring& r, int64_t chunk_id, int32_t n_tokens, int32_t* slot);
// Applies a planned update: the chunk's length becomes n_tokens.
void commit_update(sr_ring& r, int64_t chunk_id, int32_t n_tokens);
// Tokens of the moving part of the window: history chunks plus the current chunk.
int32_t moving_tokens(const sr_ring& r);
}  // namespace sr
