// Device-side entry points used by the C ABI (capi.cpp).  All launches are asynchronous
// on the given stream and return the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "core.hpp"

namespace sr {

constexpr int kMaxSegs = SR_MAX_WINDOW + 2;

// One logical key segment as the kernels see it: first pool page and valid tokens.
struct DevSeg {
  int32_t page;
  int32_t len;
};

// Segment table of one call, built on the host when the ring changes and passed by value
// (no per-call host-to-device copy).  Segments are in visiting order; the last one is the
// current chunk.
struct SegTable {
  int32_t n;
  DevSeg s[kMaxSegs];
};

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

// Copies n tokens of K/V ([n][H][D], token-major) into pages [page0, page0 + npages) of
// every head, K as rows and V transposed, and zeroes those pages past token n.
hipError_t launch_append(const Layout& L, void* pool, const void* k, const void* v, int32_t n, int32_t page0,
                         int32_t npages, hipStream_t st);

// Writes the logical sequence of `t` ([ntok][H][D], token-major) to kout / vout.
hipError_t launch_gather(const Layout& L, const void* pool, const SegTable& t, int32_t ntok, void* kout, void* vout,
                         hipStream_t st);

// Chunk attention of the current chunk's queries over the segments of `t`.
hipError_t launch_attention(const Layout& L, const void* pool, const SegTable& t, const void* q, void* o, float* lse,
                            float softmax_scale, hipStream_t st);

}  // namespace sr
