/*
 * sr.h -- streaming chunk-causal attention over a paged KV cache, for AMD MI355X (gfx950).
 *
 * What the library computes (StreamRender-H3 project page, "Interactive Coding Worlds
 * with Real-time Streaming Diffusion Render"):
 *   - "2.3 A Real-Time Interaction Loop", step 4: the session's conditioning is encoded
 *     once, then each chunk is generated in a few denoising steps (two in the racing demo)
 *     conditioned on the session's appearance and on the renderer's own recent output.
 *   - "3.1.2 Historical Context and Temporal Consistency", prefix cache: every window is a
 *     fixed prefix (conditioning, reference image, sink) plus a moving part; the moving rows
 *     attend to the whole window, bidirectionally.
 *   - "3.3 Inference Acceleration and End-to-End Deployment": the static context's K/V are
 *     computed once per denoising timestep and each timestep keeps its own bank (static-context
 *     KV caching); K/V live in persistent per-layer buffers in the layout the attention kernel
 *     reads, the static part written once and the dynamic region updated in place (persistent
 *     KV layout); sequence metadata is prepared once, with no host-device synchronisation
 *     (attention metadata reuse).
 *   - "3.2 Fast Causal H3 VAE", inference items: a preallocated ring buffer whose slots are
 *     written in place, never concatenated or repartitioned; empty slots are hidden from the
 *     kernel rather than masked.
 *
 * One attention call: the current chunk's n query tokens attend over
 *   [ persistent tokens of bank b | history chunks in the window, oldest first | current chunk ]
 * where current query i sees current key j iff floor(j / causal_block) <= floor(i / causal_block).
 * With causal_block >= chunk size the whole window is visible (bidirectional).
 *
 * Page-literal window variant (same pages, "3.1.2", prefix cache): the moving part of the
 * window -- the history chunks and the current chunk -- is recomputed every step, so all of
 * its rows are queries over the whole window, bidirectionally (sr_window_attention), its K/V
 * are rewritten in place (sr_kvcache_update_chunk), and the prefix rows attend to their bank
 * only (sr_prefix_attention), which yields the next layer's bank once per denoising step.
 *
 * Conventions shared by every call
 *   - Device memory is owned by the caller (e.g. torch tensors): pools, inputs, outputs and
 *     the optional attention workspace.  The library never allocates or frees device
 *     memory.  Host allocations: the opaque handles only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All device work is
 *     enqueued on it in call order; no call blocks or synchronises the host.
 *   - Token-major tensors are contiguous [n][H][D] (the layout a fused qkv projection emits).
 *     Element type: bf16 (raw 16-bit patterns) for SR_BF16, IEEE fp32 for SR_F32.
 *   - Device pointers must be 16-byte aligned; the pool 256-byte aligned.
 *   - Every call validates its arguments on the host before enqueuing anything.  On error it
 *     returns a status, enqueues nothing and leaves the handle's state unchanged;
 *     sr_last_error() gives a thread-local message.  A failed kernel launch returns
 *     SR_E_DEVICE.  Faults inside kernels surface at the caller's next synchronisation.
 *   - Handles are not thread-safe; distinct handles are independent.
 */
#ifndef SR_H
#define SR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sr_status {
  SR_OK = 0,
  SR_E_INVALID = 1,     /* bad argument: null/misaligned pointer, size or index out of range */
  SR_E_STATE = 2,       /* call not allowed in the current cache state (e.g. window full) */
  SR_E_NOMEM = 3,       /* pool smaller than sr_kvcache_required_bytes, or host allocation failed */
  SR_E_DEVICE = 4,      /* HIP runtime error while enqueuing */
  SR_E_UNSUPPORTED = 5  /* valid request the library does not implement (e.g. head_dim) */
} sr_status;

/* Cache element types.  SR_MX is the reduced-precision video attention of "The road to the
 * fastest, cheapest H3" (Accelerating the denoiser, item 2): keys stored as MXFP6 (FP6 E2M3
 * elements, one E8M0 scale per 32 consecutive features), values as FP8 E4M3, queries
 * quantized to MXFP6 by the attention call itself.  Its inputs and outputs (K, V, q, out,
 * gather) are bf16; see "Reduced-precision cache" below. */
typedef enum sr_dtype { SR_BF16 = 0, SR_F32 = 1, SR_MX = 2 } sr_dtype;

/* Tokens per pool page.  Every segment starts on a page boundary. */
#define SR_PAGE_TOKENS 128
/* Largest window of history chunks (the segment table is passed to kernels by value). */
#define SR_MAX_WINDOW 14
/* Most pages of keys one attention call may visit: sum over the visited segments
 * (persistent bank, history chunks, current chunk) of ceil(length / SR_PAGE_TOKENS).
 * sr_chunk_attention returns SR_E_UNSUPPORTED beyond it. */
#define SR_MAX_VISIBLE_PAGES 1024

typedef struct sr_kvcache_config {
  int32_t num_heads;         /* H >= 1 (batch folded into heads) */
  int32_t head_dim;          /* D: 64 or 128 for SR_BF16 and SR_MX; 64 for SR_F32 */
  int32_t persistent_tokens; /* P >= 0: reference-image + prompt (+ sink) tokens per bank */
  int32_t num_banks;         /* >= 1: one per denoising step */
  int32_t chunk_capacity;    /* >= 1: most tokens a chunk may have (ring slot size) */
  int32_t window_chunks;     /* W in [0, SR_MAX_WINDOW]: history chunks kept; the ring has W+1 slots */
  int32_t causal_block;      /* >= 1: tokens per causal block inside the current chunk */
  int32_t dtype;             /* sr_dtype */
} sr_kvcache_config;

/* ------------------------------------------------------------------------------------------
 * Ring state (host only, no device work).  The chunk bookkeeping of the cache as its own
 * object, so it can be driven and inspected without a GPU.  sr_kvcache owns one.
 *
 * Rules ("3.2 Fast Causal H3 VAE", ring buffer written in place; "2.3 A Real-Time
 * Interaction Loop", several denoising steps per chunk):
 *   - the first append may use any chunk_id >= 0;
 *   - appending the current id again replaces the current chunk (next denoising step);
 *   - appending current id + 1 commits the current chunk to the history (what was appended
 *     last stays) and makes the new id current; if the history already holds W chunks this is
 *     SR_E_STATE ("evict first"); with W == 0 the committed chunk is dropped;
 *   - any other id is SR_E_INVALID;
 *   - evict drops the oldest history chunk (SR_E_STATE if there is none);
 *   - chunk id c lives in ring slot c mod (W+1).
 * ------------------------------------------------------------------------------------------ */
typedef struct sr_ring sr_ring;

typedef enum sr_segment_kind { SR_SEG_PERSISTENT = 0, SR_SEG_HISTORY = 1, SR_SEG_CURRENT = 2 } sr_segment_kind;

typedef struct sr_segment {
  int64_t chunk_id; /* -1 for the persistent bank */
  int32_t kind;     /* sr_segment_kind */
  int32_t slot;     /* ring slot, or the bank index for the persistent segment */
  int32_t page;     /* first pool page of the segment */
  int32_t length;   /* valid tokens */
} sr_segment;

/* Validates `cfg` and creates an empty ring.  *out is set on success only. */
sr_status sr_ring_create(const sr_kvcache_config* cfg, sr_ring** out);
/* Applies one append.  On success *slot is the ring slot written and *committed_id the
 * chunk committed to the history by this call, or -1 (either pointer may be NULL).
 * SR_E_INVALID also for n_tokens outside [1, chunk_capacity]. */
sr_status sr_ring_append(sr_ring* r, int64_t chunk_id, int32_t n_tokens, int32_t* slot, int64_t* committed_id);
/* Drops the oldest history chunk; *evicted_id (nullable) receives its id. */
sr_status sr_ring_evict(sr_ring* r, int64_t* evicted_id);
/* Replaces, in place, a chunk that is in the window (a history chunk or the current one):
 * its length becomes n_tokens and *slot (nullable) receives its ring slot.  SR_E_INVALID for
 * an id outside the window or n_tokens outside [1, chunk_capacity]; the state is unchanged. */
sr_status sr_ring_update(sr_ring* r, int64_t chunk_id, int32_t n_tokens, int32_t* slot);
/* Logical key segments of an attention call on `bank`, in visiting order:
 * persistent bank (omitted when P == 0), history oldest first, current.  Writes at most
 * `max` entries to `out` and the count to *n.  SR_E_STATE if there is no current chunk,
 * SR_E_INVALID if `max` is too small or `bank` out of range. */
sr_status sr_ring_segments(const sr_ring* r, int32_t bank, sr_segment* out, int32_t max, int32_t* n);
sr_status sr_ring_destroy(sr_ring* r);

/* ------------------------------------------------------------------------------------------
 * KV cache (one handle per attention layer).
 *
 * Pool layout in HBM.  The K region (half_bytes = bytes / 2) is followed by the V region.
 * Each region holds, for head h and page p (128 tokens), one page of 128 * D elements at
 * element offset (h * total_pages + p) * 128 * D.  Inside a page, with E = 16 / element
 * size (8 for bf16, 4 for fp32), token t (0..127) and feature d:
 *   K: ((d / E) * 128 + row(t)) * E + d % E
 *   V: ((t / E) * D + d) * E + t % E
 * row(t) permutes t inside its block of 32 (bf16: swap bits 2 and 3; fp32: 32-block row
 * 8*(r/8) + 4*(r%2) + (r/2)%4 for r = t % 32).  This is the order in which the attention
 * kernel's matrix instructions consume the page, so a page is copied into LDS unchanged.
 * Pages are numbered: banks first (ceil(P/128) pages each), then the W+1 ring slots
 * (ceil(capacity/128) pages each).  Tokens past a segment's valid length are kept at zero.
 *
 * Reduced-precision cache (SR_MX).  K/V are given in bf16 and quantized when written
 * (append, update, the persistent banks), nearest with ties to the even mantissa and
 * saturation, the sign bit kept; every input must be finite:
 *   K: for each token and block of 32 features, X = floor(log2 max|k|) - 2 (at least -127),
 *      codes = E2M3(k / 2^X) (largest 7.5);
 *   V: E4M3 per element (largest 448).
 * The attention call quantizes q the same way as K and computes softmax(scale q~.k~) v~ over
 * the dequantized values (probabilities are rounded to FP8 for the P.V product).
 * The K region holds, per (head, page), 3200 * D / 32 bytes rounded up to a multiple of 1024
 * (13312 for D = 128); the V region, after it, 128 * D bytes.  With NB = D / 32 blocks, block b of token t (0..127) packs its 32 codes
 * little-endian, 6 bits each, into 24 bytes: bytes 0-15 at (b * 128 + t) * 16, bytes 16-23 at
 * NB * 2048 + (b * 128 + t) * 8; the scale bytes X + 127 of token t are the NB bytes at
 * NB * 3072 + t * NB, block b at position (b % 2) * NB / 2 + b / 2.  V code (t, d) is byte
 * (g * D + d) * 16 + i, where r = t % 32, g = 4 * (t / 64) + 2 * ((t / 32) % 2) + (r / 4) % 2
 * and i = 4 * (r / 8) + r % 4: the order in which the attention kernel's matrix
 * instructions consume them.  sr_kvcache_gather returns the dequantized K/V as bf16 (exact).
 * sr_kvcache_append_qkv is SR_E_UNSUPPORTED on such a cache.
 * ------------------------------------------------------------------------------------------ */
typedef struct sr_kvcache sr_kvcache;

/* Bytes the pool must have for `cfg`. */
sr_status sr_kvcache_required_bytes(const sr_kvcache_config* cfg, size_t* bytes);

/* Creates a cache on `pool` (device, caller-owned, >= required bytes, kept alive until
 * destroy and until its queued work is done).  Enqueues: zero the pool, then copy the
 * persistent banks persistent_k / persistent_v (device, [num_banks][P][H][D], may be NULL
 * when P == 0) into their pages.  The caller may reuse those buffers once the stream has
 * passed this call. */
sr_status sr_kvcache_init(const sr_kvcache_config* cfg, void* pool, size_t pool_bytes,
                          const void* persistent_k, const void* persistent_v, void* stream,
                          sr_kvcache** out);

/* Appends one chunk's K/V (device, [n_tokens][H][D]) under the ring rules above and
 * enqueues the copy into slot chunk_id mod (W+1), zeroing the slot past n_tokens.
 * ("3.3 Inference Acceleration", persistent KV layout: only the dynamic region is written.) */
sr_status sr_kvcache_append_chunk(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v,
                                  int32_t n_tokens, void* stream);

/* Parameters of the qk preparation done by sr_kvcache_append_qkv. */
typedef struct {
  int32_t rope_sections[3]; /* rotation pairs following position axis t, y, x (in that order of
                               pairs); each >= 0, summing to head_dim / 2 */
  float rope_base;          /* > 1: pair k of a section of n pairs turns by pos * base^(-k/n) */
  float rms_eps;            /* >= 0, added to the mean square */
} sr_qk_prep;

/* Fused append after the qkv projection ("3.2 Fast Causal H3 VAE", iteration 6: qk-norm, the
 * rotary embedding and the K/V cache write in one kernel after the qkv GEMM; inference items:
 * each new token gets its rotary position once, when it is written; iteration 4: positions are
 * stream-absolute, so scores depend only on position differences).
 *   qkv        device [n_tokens][3][H][D] in the cache dtype: q, k, v of each token.
 *   positions  device int32 [n_tokens][3]: (t, y, x) of each token, t the stream-absolute
 *              latent-frame index.
 *   q_gain, k_gain  device fp32 [D]: RMSNorm gains of q and k (shared by the heads).
 *   q_out      device [n_tokens][H][D] in the cache dtype (must not overlap qkv): the prepared
 *              queries, for the attention call that follows.
 * For q and k of every (token, head): y = x / sqrt(mean(x^2) + rms_eps) * gain, then rotation
 * pair j = (y_2j, y_2j+1) in section a (pairs assigned to t, y, x in order) at index k within
 * it turns by positions[a] * rope_base^(-k / rope_sections[a]).  Computed in fp32 and rounded
 * to the cache dtype (nearest even).  The prepared K and the unchanged V are then appended
 * exactly as by sr_kvcache_append_chunk (same ring rules and errors).  SR_E_INVALID, with
 * nothing enqueued, for bad pointers or parameters.  The caller may reuse qkv / positions
 * once the stream has passed the call. */
sr_status sr_kvcache_append_qkv(sr_kvcache* c, int64_t chunk_id, const void* qkv, const int32_t* positions,
                                int32_t n_tokens, const float* q_gain, const float* k_gain,
                                const sr_qk_prep* prep, void* q_out, void* stream);

/* Drops the oldest history chunk (host metadata only; nothing is enqueued). */
sr_status sr_kvcache_evict(sr_kvcache* c, int64_t* evicted_chunk_id);

/* Rewrites, in place, the K/V of a chunk in the window (device, [n_tokens][H][D]): a history
 * chunk or the current one (for the current one this equals appending its id again).  The
 * slot past n_tokens is zeroed and the chunk's length becomes n_tokens.  For the page-literal
 * window variant, where the recent history is recomputed every step ("3.1.2 Historical
 * Context and Temporal Consistency", prefix cache; "3.3 Inference Acceleration", persistent
 * KV layout: the dynamic region is updated in place).  SR_E_INVALID (nothing enqueued) for an
 * id outside the window, n_tokens outside [1, chunk_capacity] or bad pointers.  The caller
 * may reuse k / v once the stream has passed the call. */
sr_status sr_kvcache_update_chunk(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v,
                                  int32_t n_tokens, void* stream);

/* Attention of the current chunk's queries q (device, [n][H][D], n = current chunk length)
 * over bank `bank` + history + current (see top of file).  out: device [n][H][D] in the
 * cache dtype.  lse: device fp32 [H][n] natural-log log-sum-exp of the scaled logits, or
 * NULL.  softmax_scale > 0 multiplies q.k (usually 1/sqrt(D)).  SR_E_STATE without a
 * current chunk; SR_E_UNSUPPORTED if the call would visit more than SR_MAX_VISIBLE_PAGES
 * pages.  q must not alias out.  Uses the cache's workspace, if one is attached (below). */
sr_status sr_chunk_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse,
                             float softmax_scale, void* stream);

/* Page-literal window variant ("3.1.2 Historical Context and Temporal Consistency": the moving
 * part attends to the entire window, attention inside the window is bidirectional).  Queries:
 * the n_rows moving rows q (device, [n_rows][H][D]), history chunks oldest first and then the
 * current chunk, n_rows = their total length (else SR_E_INVALID).  Every row sees every key of
 * bank `bank` + history + current; the cache's causal_block does not apply.  out [n_rows][H][D]
 * in the cache dtype, lse fp32 [H][n_rows] or NULL, softmax_scale, errors, workspace and
 * aliasing as for sr_chunk_attention. */
sr_status sr_window_attention(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out,
                              float* lse, float softmax_scale, void* stream);

/* The prefix rows' attention ("3.1.2", prefix cache: the prefix attends only to itself; "3.3",
 * static-context KV caching: computed once per denoising step and session).  Queries: the P
 * prefix rows q (device, [P][H][D]) of bank `bank`; keys: that bank's persistent tokens only.
 * out [P][H][D], lse fp32 [H][P] or NULL.  Needs no current chunk.  SR_E_INVALID when the
 * cache has no persistent tokens; otherwise as sr_chunk_attention. */
sr_status sr_prefix_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse,
                              float softmax_scale, void* stream);

/* ------------------------------------------------------------------------------------------
 * Attention workspace (optional, caller-owned device memory).
 *
 * Without a workspace, sr_chunk_attention runs one workgroup per (head, 256-query tile),
 * each over that tile's whole key list, and the last round of workgroups can leave compute
 * units idle.  With a workspace attached, each of the device's 8 XCDs (C = compute units / 8,
 * at most 64) owns a share of the (head, query tile) items: it runs them whole, C at a time,
 * and cuts the key tiles of its last (< C) items into up to eight pieces, largest first.  One
 * persistent workgroup per compute unit takes whole items from its XCD's queue, then from the
 * other XCDs' queues, then pieces from one queue for the device that holds every split item's
 * first piece, then every second piece, and so on, so that the last units taken anywhere are
 * the smallest.  A piece of a split item leaves its partial result (output, running max and
 * sum per query; the output rounded to bf16 for bf16 and reduced-precision caches) in the
 * workspace, and the last of the item's pieces to finish merges them in a fixed order and
 * writes out / lse.  No workgroup waits for another.  The kernel shape is tuned per device
 * ("3.3 Inference Acceleration and End-to-End Deployment", attention kernel tuning); this
 * split is the MI355X choice.
 *
 * Layout: 64 C records of 8 x 64 x 34 floats, then 8 C int32 arrival counters and 16 int32
 * queue counters (rounded up to 256 bytes).  The counters must be zero when a call starts;
 * sr_kvcache_set_workspace zeroes them and every call leaves them zero.  Results with and
 * without a workspace agree within rounding (different summation order); with a workspace
 * they are bit-reproducible from call to call.
 * ------------------------------------------------------------------------------------------ */

/* Workspace bytes for caches of `cfg` on a device with `num_workgroups` compute units
 * (0: the current device's count, which is what sr_kvcache_set_workspace uses). */
sr_status sr_attention_workspace_bytes(const sr_kvcache_config* cfg, int32_t num_workgroups, size_t* bytes);

/* Attaches workspace `ws` (device, 256-byte aligned, >= sr_attention_workspace_bytes(cfg, 0)
 * bytes, else SR_E_NOMEM) to the cache and enqueues the zeroing of its counters on `stream`;
 * ws == NULL detaches it.  One workspace may serve several caches whose attention calls are
 * ordered (one stream); calls that may overlap need separate workspaces.  The caller keeps
 * it alive while calls that use it are queued. */
sr_status sr_kvcache_set_workspace(sr_kvcache* c, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Windowed caches: the streaming decoder ("3.2 Fast Causal H3 VAE").
 *
 * Iteration 2: the decoder takes chunks of two latent frames; each chunk's attention sees its
 * own latent frames and the cached K/V of the four before it (a window of W = 2 chunks), and
 * attention runs inside non-overlapping windows of 16 x 16 tokens.  Iteration 3, item 4: a
 * window's attention is an independent sequence of its own (at 720p: 512 query rows, 1,541
 * keys) without padded rows, and ring slots that hold nothing yet are left out of its keys.
 * Iterations 4 and 6: five global tokens (four register tokens, one class token) see the
 * whole frame and are recomputed for each chunk instead of being cached; every window's rows
 * see them as well.
 *
 * A cache with a window layout stores every chunk's frame tokens window by window: window w
 * owns window_pages pages of each ring slot, from page w * window_pages of the slot, and holds
 * frames_per_chunk * window_tokens[w] tokens (its tokens of the chunk's first latent frame,
 * then of the second, ...).  The chunk's K/V, queries and outputs are packed the same way,
 * windows in order, with no padding: T = frames_per_chunk * sum(window_tokens) rows.  The
 * global tokens live in a persistent bank (persistent_tokens = their count), rewritten for
 * every chunk with sr_kvcache_set_bank.  On such a cache sr_kvcache_append_chunk,
 * sr_kvcache_update_chunk, sr_kvcache_append_qkv, sr_chunk_attention, sr_window_attention and
 * sr_prefix_attention return SR_E_STATE; sr_kvcache_gather returns the packed sequence.
 * ------------------------------------------------------------------------------------------ */
#define SR_MAX_LAYOUT_WINDOWS 64

typedef struct sr_window_layout {
  int32_t num_windows;       /* 1 .. SR_MAX_LAYOUT_WINDOWS */
  int32_t frames_per_chunk;  /* >= 1: latent frames per chunk */
  int32_t window_pages;      /* >= 1: pages per window in a ring slot;
                                num_windows * window_pages <= pages of a slot (ceil(capacity / 128)) */
  int32_t window_tokens[SR_MAX_LAYOUT_WINDOWS]; /* 1 .. 128 * window_pages / frames_per_chunk each
                                                   (entries past num_windows are ignored) */
} sr_window_layout;

/* Sets the window layout (host only).  Allowed once, before the first append; SR_E_STATE after
 * it, otherwise the errors of sr_window_layout_check. */
sr_status sr_kvcache_set_window_layout(sr_kvcache* c, const sr_window_layout* layout);

/* Checks a window layout against a cache config without a cache (host only, no device work):
 * SR_E_INVALID for a config or layout that does not fit (windows beyond a slot's pages, a
 * window's frames_per_chunk * window_tokens[w] tokens beyond its window_pages pages or beyond
 * the SR_MAX_VISIBLE_PAGES pages one attention call can visit), SR_E_UNSUPPORTED for an SR_MX
 * cache. */
sr_status sr_window_layout_check(const sr_kvcache_config* cfg, const sr_window_layout* layout);

/* Rewrites the persistent tokens of `bank` in place: k, v device [P][H][D] (any cache; the
 * decoder's global tokens, rebuilt for every chunk).  SR_E_INVALID when P == 0.  The caller may
 * reuse k / v once the stream has passed the call. */
sr_status sr_kvcache_set_bank(sr_kvcache* c, int32_t bank, const void* k, const void* v, void* stream);

/* Appends one chunk of a windowed cache: k, v device [T][H][D] packed window by window (see
 * above).  Ring rules and errors of sr_kvcache_append_chunk with n_tokens = T; each window's
 * pages are zeroed past its tokens. */
sr_status sr_kvcache_append_windows(sr_kvcache* c, int64_t chunk_id, const void* k, const void* v, void* stream);

/* Window attention of the current chunk: q device [T][H][D] packed like the chunk; the rows of
 * window w attend to the persistent tokens of `bank` (the global tokens), window w's tokens of
 * the history chunks (oldest first) and of the current chunk, every row seeing every one of
 * them.  out [T][H][D] in the cache dtype, lse fp32 [H][T] or NULL, softmax_scale > 0.  One
 * launch for all windows, heads and query tiles (the workspace is not used).  SR_E_STATE
 * without a window layout or a current chunk; q must not alias out. */
sr_status sr_windows_attention(sr_kvcache* c, int32_t bank, const void* q, void* out, float* lse,
                               float softmax_scale, void* stream);

/* Global-token attention: n_rows >= 1 queries q (device [n_rows][H][D], the global tokens)
 * attend to the persistent tokens of `bank` and to every window's tokens of the current chunk
 * (the whole frame), all visible.  out [n_rows][H][D], lse [H][n_rows] or NULL.  Iteration 6:
 * split-K.  On a bf16 cache with a workspace attached and n_rows <= 32, every head's keys are
 * split four pages per workgroup over the device and each head's partial results are merged by
 * its last workgroup (in a fixed order: repeated calls give the same bits); otherwise the call
 * runs on the chunk-attention kernel (with its split schedule when a workspace is attached).
 * The workspace must not be in use by a call on another stream.  SR_E_STATE without a window
 * layout or a current chunk; SR_E_INVALID for n_rows < 1. */
sr_status sr_global_attention(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out, float* lse,
                              float softmax_scale, void* stream);

/* sr_global_attention for callers that cannot allocate device memory (code under graph
 * capture, serving loops, harnesses that forbid hipMalloc): the same split-K call, with its
 * records and arrival counters in a scratch array the library owns -- 4 MiB of records
 * (2^20 floats) and 4096 counters, one copy per GPU held until the process ends -- instead of
 * the cache's workspace; no device memory is allocated by this call or by the library.  The
 * result equals sr_global_attention's with a workspace attached, bit for bit.  All calls on one
 * GPU share its copy: calls that overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller.  The first call on a GPU looks up that GPU's copy and enqueues
 * one small kernel on `stream` that zeroes its counters; every call leaves them at zero.
 * Same arguments and errors as sr_global_attention, plus SR_E_UNSUPPORTED when the call does
 * not fit the few-row kernel (a cache other than SR_BF16, head_dim other than 64 or 128, more
 * than 32 rows) or needs more scratch than the array holds (H * ceil(pages / 4) * (64 + n_rows *
 * head_dim) floats of records, pages = the call's key pages; H <= 4096); nothing is enqueued
 * then. */
sr_status sr_global_attention_static(sr_kvcache* c, int32_t bank, const void* q, int32_t n_rows, void* out, float* lse,
                                     float softmax_scale, void* stream);

/* Copies the logical key/value sequence of a call on `bank` (persistent, history oldest
 * first, current) into k_out / v_out (device, [max_tokens][H][D]), bit-exact.  *n_tokens
 * receives the length; SR_E_INVALID if it exceeds max_tokens (nothing enqueued).  For tests
 * and debugging.  A windowed cache's chunks come out packed window by window. */
sr_status sr_kvcache_gather(const sr_kvcache* c, int32_t bank, void* k_out, void* v_out,
                            int32_t max_tokens, int32_t* n_tokens, void* stream);

/* Measurement aid (not part of the attention path): the dense bf16 MFMA rate of the device.
 * Launches `workgroups` workgroups of 512 threads; every wave runs 4 independent chains of
 * `iters` v_mfma_f32_32x32x16_bf16 instructions on register operands, 4 * 32768 * iters flops
 * per wave, and each thread writes one float to out (device, >= workgroups * 512 floats, owned by
 * the caller).  Two workgroups per compute unit keep every SIMD busy; the flops over the launch's
 * duration are the sustained peak at the running clock.  SR_E_INVALID for a null out,
 * workgroups outside [1, 2^20] or iters outside [1, 2^24]; SR_E_DEVICE for a launch failure. */
sr_status sr_probe_mfma_bf16(float* out, int32_t workgroups, int32_t iters, void* stream);

/* Measurement aid (not part of the attention path): reads `bytes` of src (device) once with the
 * global-to-LDS 16-byte loads the attention kernel streams its cache pages with, one 64 KiB
 * block per 256-thread workgroup, each thread writing one float to out (device, >= bytes / 256
 * floats, owned by the caller).  Run beside a plain device copy under the profiler, it shows
 * that the fetch counter counts these loads as it counts the copy's, so one scale factor serves
 * both.  SR_E_INVALID for a null buffer or bytes not a positive multiple of 65536 (at most 2^24
 * blocks); SR_E_DEVICE for a launch failure. */
sr_status sr_probe_lds_read(const void* src, int64_t bytes, float* out, void* stream);

/* The handle's ring state, for inspection (owned by the cache). */
const sr_ring* sr_kvcache_ring(const sr_kvcache* c);

/* Frees the host handle only (the pool stays the caller's). */
sr_status sr_kvcache_destroy(sr_kvcache* c);

const char* sr_status_string(sr_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* sr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SR_H */
