// fp64 CPU oracle of streaming chunk-causal attention, plain C++17.
//
// TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU-baseline leg
// load it; the HIP library never does.  It includes nothing from the library (no kernels,
// headers, helpers or tables); both sides only consume the same seeded inputs.
//
// What it computes (StreamRender-H3 project page, "3.1.2 Historical Context and Temporal
// Consistency", prefix cache; "3.3 Inference Acceleration and End-to-End Deployment",
// static-context KV caching): the current chunk's query tokens attend, one softmax per row,
// over the persistent tokens of the denoising step's bank, the history chunks kept in the
// rolling window, and the current chunk, bidirectionally inside each causal block of the
// current chunk.  The method reaches the plain masked softmax-attention result exactly (an
// online softmax only reorders the rounding), so this file is that definition written out:
//
//   for one head, query row i and the set S(i) of keys visible to it
//     s_j = scale * sum_d q_{i,d} k_{j,d}          (j in S(i))
//     m   = max_{j in S(i)} s_j
//     w_j = exp(s_j - m)                           (j in S(i); 0 for the other keys)
//     l   = sum_j w_j
//     o_i = sum_j w_j v_j / l,    lse_i = m + ln l
//
//   with, for a chunk call on bank b and causal block cb,
//     S(i) = every persistent token of bank b, every token of the history chunks in the
//            window, and the current-chunk tokens j with floor(j / cb) <= floor(i / cb).
//
// The cache model keeps its own state: a std::deque of committed chunks, oldest first.
//   * persistent banks, fixed for the session, one per denoising step (project page 3.3);
//   * append(id): the first call takes any id >= 0; the current id again replaces the
//     current chunk (the next denoising step of the same chunk); current + 1 commits the
//     current chunk to the history first (its last K/V stay) -- an error if the history
//     already holds W chunks (evict first), and with W == 0 the committed chunk is dropped;
//     any other id is an error;
//   * evict drops the oldest history chunk (an error when there is none);
//   * update(id) rewrites a chunk still in the window in place (the page-literal reading of
//     3.1.2, where the moving part is recomputed every step);
//   * chunks not in the window are never attended (project page "3.2 Fast Causal H3 VAE":
//     empty ring slots are hidden from the kernel, not masked).
//   Rejected calls change nothing.
//
// A second route, full_sequence_attention, lays the whole stream out as one sequence
// [prefix; chunk 0; ...; chunk c] with no cache and an explicit mask written from the window
// rule (the prefix sees only itself; chunk c's rows see the prefix, the W chunks before c and
// their own causal blocks of c), and applies the same definition.
//
// Inputs are the storage values given to the GPU (bf16 bit patterns or fp32), widened to
// fp64 exactly.  Work is spread over std::thread workers, one (head, 64-row block) at a time;
// every output element is computed by one worker in the order written above.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <limits>
#include <thread>
#include <vector>

namespace {

constexpr int kBf16 = 0;  // storage: bf16 bit patterns (uint16)
constexpr int kF32 = 1;   // storage: fp32
constexpr int kRowBlock = 64;

size_t elem_bytes(int dtype) { return dtype == kBf16 ? 2 : 4; }

// One stored element, widened to fp64 (exact for both storage types).
double widen(const uint8_t* base, size_t index, int dtype) {
  if (dtype == kBf16) {
    uint16_t b;
    std::memcpy(&b, base + 2 * index, 2);
    const uint32_t u = uint32_t(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  float f;
  std::memcpy(&f, base + 4 * index, 4);
  return f;
}

double dot(const double* a, const double* b, int n) {
  double acc = 0.0;
#pragma omp simd reduction(+ : acc)
  for (int d = 0; d < n; ++d) acc += a[d] * b[d];
  return acc;
}

// The definition for query rows [0, nr) of one head: q [nr][D], k [nk][D], v [nk][Dv] in fp64,
// visible(r, j).  Writes o [nr][Dv], lse [nr] and, if probs is not null, w / l [nr][nk].
// Returns false if a row sees no key.  s: scratch of nr * nk doubles.
template <class Visible>
bool attend(int nr, int nk, int D, int Dv, const double* q, const double* k, const double* v, double scale,
            Visible visible, double* o, double* lse, double* probs, std::vector<double>& s) {
  const double neg_inf = -std::numeric_limits<double>::infinity();
  s.assign(size_t(nr) * nk, neg_inf);
  // scores of the visible keys (key-major, so each key row is read once per block of rows)
  for (int j = 0; j < nk; ++j)
    for (int r = 0; r < nr; ++r)
      if (visible(r, j)) s[size_t(r) * nk + j] = scale * dot(q + size_t(r) * D, k + size_t(j) * D, D);
  std::vector<double> m(nr), l(nr);
  for (int r = 0; r < nr; ++r) {
    double* sr = &s[size_t(r) * nk];
    double mx = neg_inf;
    bool any = false;
    for (int j = 0; j < nk; ++j)
      if (visible(r, j)) {
        mx = any ? std::max(mx, sr[j]) : sr[j];
        any = true;
      }
    if (!any) return false;
    double sum = 0.0;
    for (int j = 0; j < nk; ++j) {
      sr[j] = visible(r, j) ? std::exp(sr[j] - mx) : 0.0;  // w_j
      sum += sr[j];
    }
    m[r] = mx;
    l[r] = sum;
  }
  for (int r = 0; r < nr; ++r)
    for (int e = 0; e < Dv; ++e) o[size_t(r) * Dv + e] = 0.0;
  for (int j = 0; j < nk; ++j) {
    const double* vj = v + size_t(j) * Dv;
    for (int r = 0; r < nr; ++r) {
      const double w = s[size_t(r) * nk + j];
      if (w == 0.0) continue;
      double* orow = o + size_t(r) * Dv;
      for (int e = 0; e < Dv; ++e) orow[e] += w * vj[e];
    }
  }
  for (int r = 0; r < nr; ++r) {
    for (int e = 0; e < Dv; ++e) o[size_t(r) * Dv + e] /= l[r];
    lse[r] = m[r] + std::log(l[r]);
    if (probs)
      for (int j = 0; j < nk; ++j) probs[size_t(r) * nk + j] = s[size_t(r) * nk + j] / l[r];
  }
  return true;
}

struct Chunk {
  int64_t id = -1;
  int32_t n = 0;
  std::vector<uint8_t> k, v;  // storage bytes [n][H][D]
};

struct Cache {
  int H = 0, D = 0, P = 0, dtype = kBf16, window = 0, capacity = 0;
  std::vector<std::vector<uint8_t>> bank_k, bank_v;  // [P][H][D] each
  std::deque<Chunk> history;                         // committed chunks in the window, oldest first
  bool has_current = false;
  Chunk current;

  size_t token_bytes() const { return size_t(H) * D * elem_bytes(dtype); }
  Chunk make(int64_t id, const void* k, const void* v, int n) const {
    Chunk c;
    c.id = id;
    c.n = n;
    const size_t bytes = size_t(n) * token_bytes();
    c.k.assign(static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(k) + bytes);
    c.v.assign(static_cast<const uint8_t*>(v), static_cast<const uint8_t*>(v) + bytes);
    return c;
  }
  bool shape_ok(int n) const { return n >= 1 && (capacity == 0 || n <= capacity); }

  // The logical key/value sequence of a call on `bank`: bank, history oldest first, current.
  // Returns the segments' (bytes, token count) in visiting order.
  std::vector<std::pair<const Chunk*, int>> segments() const {
    std::vector<std::pair<const Chunk*, int>> out;
    for (const Chunk& c : history) out.push_back({&c, c.n});
    out.push_back({&current, current.n});
    return out;
  }
};

// Widened K and V of one head over a list of segments ([tokens][H][D] storage each).
void widen_head(const std::vector<std::pair<const uint8_t*, int>>& segs, int H, int D, int dtype, int h,
                std::vector<double>& out) {
  size_t n = 0;
  for (auto& s : segs) n += size_t(s.second);
  out.resize(n * D);
  size_t t = 0;
  for (auto& s : segs)
    for (int i = 0; i < s.second; ++i, ++t)
      for (int d = 0; d < D; ++d) out[t * D + d] = widen(s.first, (size_t(i) * H + h) * D + d, dtype);
}

int default_threads() {
  const unsigned n = std::thread::hardware_concurrency();
  return n == 0 ? 1 : int(n);
}

// Runs f(item) for items [0, n) on `threads` workers.
template <class F>
void parallel_for(int n, int threads, F f) {
  if (threads <= 0) threads = default_threads();
  if (threads > n) threads = n;
  if (threads <= 1) {
    for (int i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int> next{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (int i = next++; i < n; i = next++) f(i);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int orc_hardware_threads(void) { return default_threads(); }

// The definition over an explicit visibility matrix (uint8 [nq][nk]); fp64 in and out.
// probs may be null.  Returns 0, or 1 if a row sees no key.
int orc_attention(int nq, int nk, int D, int Dv, const double* q, const double* k, const double* v,
                  const uint8_t* visible, double scale, double* o, double* lse, double* probs) {
  std::vector<double> s;
  const bool ok = attend(nq, nk, D, Dv, q, k, v, scale,
                         [&](int r, int j) { return visible[size_t(r) * nk + j] != 0; }, o, lse, probs, s);
  return ok ? 0 : 1;
}

// Cache model.  pk, pv: [banks][P][H][D] storage values (P may be 0).  capacity 0: no limit.
int orc_cache_create(int banks, int P, int H, int D, int dtype, int window, int capacity, const void* pk,
                     const void* pv, void** out) {
  if (banks < 1 || P < 0 || H < 1 || D < 1 || (dtype != kBf16 && dtype != kF32) || window < 0 || !out) return 1;
  Cache* c = new Cache;
  c->H = H;
  c->D = D;
  c->P = P;
  c->dtype = dtype;
  c->window = window;
  c->capacity = capacity;
  const size_t bank_bytes = size_t(P) * c->token_bytes();
  for (int b = 0; b < banks; ++b) {
    const uint8_t* kb = static_cast<const uint8_t*>(pk) + b * bank_bytes;
    const uint8_t* vb = static_cast<const uint8_t*>(pv) + b * bank_bytes;
    c->bank_k.emplace_back(kb, kb + bank_bytes);
    c->bank_v.emplace_back(vb, vb + bank_bytes);
  }
  *out = c;
  return 0;
}

void orc_cache_destroy(void* c) { delete static_cast<Cache*>(c); }

// Returns 0 on success, 1 if the state machine rejects the call (state unchanged).
int orc_cache_append(void* cp, int64_t id, const void* k, const void* v, int n) {
  Cache& c = *static_cast<Cache*>(cp);
  if (id < 0 || !c.shape_ok(n)) return 1;
  if (!c.has_current || id == c.current.id) {
    c.current = c.make(id, k, v, n);
    c.has_current = true;
    return 0;
  }
  if (id != c.current.id + 1) return 1;
  if (c.window > 0) {
    if (int(c.history.size()) == c.window) return 1;  // the window is full: evict first
    c.history.push_back(std::move(c.current));
  }
  c.current = c.make(id, k, v, n);
  return 0;
}

int orc_cache_update(void* cp, int64_t id, const void* k, const void* v, int n) {
  Cache& c = *static_cast<Cache*>(cp);
  if (!c.shape_ok(n)) return 1;
  if (c.has_current && id == c.current.id) {
    c.current = c.make(id, k, v, n);
    return 0;
  }
  for (Chunk& h : c.history)
    if (h.id == id) {
      h = c.make(id, k, v, n);
      return 0;
    }
  return 1;
}

int orc_cache_evict(void* cp, int64_t* evicted) {
  Cache& c = *static_cast<Cache*>(cp);
  if (c.history.empty()) return 1;
  if (evicted) *evicted = c.history.front().id;
  c.history.pop_front();
  return 0;
}

int orc_cache_set_bank(void* cp, int bank, const void* k, const void* v) {
  Cache& c = *static_cast<Cache*>(cp);
  if (bank < 0 || bank >= int(c.bank_k.size())) return 1;
  const size_t bytes = size_t(c.P) * c.token_bytes();
  c.bank_k[bank].assign(static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(k) + bytes);
  c.bank_v[bank].assign(static_cast<const uint8_t*>(v), static_cast<const uint8_t*>(v) + bytes);
  return 0;
}

// Chunk ids the current chunk attends to, oldest first, then the current id; returns the count.
int orc_cache_visible_ids(const void* cp, int64_t* ids, int max) {
  const Cache& c = *static_cast<const Cache*>(cp);
  int n = 0;
  for (const Chunk& h : c.history)
    if (n < max) ids[n++] = h.id;
  if (c.has_current && n < max) ids[n++] = c.current.id;
  return n;
}

// Tokens of the logical sequence of a call on `bank` and how many precede the current chunk.
int orc_cache_sequence_len(const void* cp, int bank, int* n_total, int* n_fixed) {
  const Cache& c = *static_cast<const Cache*>(cp);
  if (!c.has_current || bank < 0 || bank >= int(c.bank_k.size())) return 1;
  int fixed = c.P;
  for (const Chunk& h : c.history) fixed += h.n;
  *n_fixed = fixed;
  *n_total = fixed + c.current.n;
  return 0;
}

// Copies the logical sequence (bank, history oldest first, current) to k_out, v_out: storage
// values [n_total][H][D], exactly as given.
int orc_cache_gather(const void* cp, int bank, void* k_out, void* v_out) {
  const Cache& c = *static_cast<const Cache*>(cp);
  if (!c.has_current || bank < 0 || bank >= int(c.bank_k.size())) return 1;
  uint8_t* ko = static_cast<uint8_t*>(k_out);
  uint8_t* vo = static_cast<uint8_t*>(v_out);
  std::memcpy(ko, c.bank_k[bank].data(), c.bank_k[bank].size());
  std::memcpy(vo, c.bank_v[bank].data(), c.bank_v[bank].size());
  size_t off = c.bank_k[bank].size();
  for (auto& seg : c.segments()) {
    std::memcpy(ko + off, seg.first->k.data(), seg.first->k.size());
    std::memcpy(vo + off, seg.first->v.data(), seg.first->v.size());
    off += seg.first->k.size();
  }
  return 0;
}

// One chunk call: q [n_q][H][D] storage values of the current chunk (row i is current token
// i).  Computes heads[0..n_heads) and rows[0..n_rows) (null: all of them) into o
// [n_rows][n_heads][D] and lse [n_heads][n_rows] (fp64).  threads <= 0: all hardware threads.
// Returns 0; 1 for a bad call (no current chunk, q not the current chunk's length, bad
// bank, head or row); 2 if a row sees no key.
int orc_chunk_attention(const void* cp, int bank, const void* q, int n_q, double scale, int causal_block,
                        const int* heads, int n_heads, const int* rows, int n_rows, int threads, double* o,
                        double* lse) {
  const Cache& c = *static_cast<const Cache*>(cp);
  if (!c.has_current || bank < 0 || bank >= int(c.bank_k.size()) || n_q != c.current.n || causal_block < 1) return 1;
  const int H = c.H, D = c.D, dt = c.dtype;
  std::vector<int> hs(heads ? heads : nullptr, heads ? heads + n_heads : nullptr);
  if (!heads)
    for (int h = 0; h < H; ++h) hs.push_back(h);
  std::vector<int> rs(rows ? rows : nullptr, rows ? rows + n_rows : nullptr);
  if (!rows)
    for (int r = 0; r < n_q; ++r) rs.push_back(r);
  for (int h : hs)
    if (h < 0 || h >= H) return 1;
  for (int r : rs)
    if (r < 0 || r >= n_q) return 1;
  const int nh = int(hs.size()), nr = int(rs.size());

  std::vector<std::pair<const uint8_t*, int>> segs;
  segs.push_back({c.bank_k[bank].data(), c.P});
  for (const Chunk& h : c.history) segs.push_back({h.k.data(), h.n});
  segs.push_back({c.current.k.data(), c.current.n});
  std::vector<std::pair<const uint8_t*, int>> vsegs;
  vsegs.push_back({c.bank_v[bank].data(), c.P});
  for (const Chunk& h : c.history) vsegs.push_back({h.v.data(), h.n});
  vsegs.push_back({c.current.v.data(), c.current.n});
  int n_fixed = c.P;
  for (const Chunk& h : c.history) n_fixed += h.n;
  const int nk = n_fixed + c.current.n;

  // Widened K and V of every requested head, then one work item per (head, block of rows).
  std::vector<std::vector<double>> kh(nh), vh(nh);
  parallel_for(nh, threads, [&](int i) {
    widen_head(segs, H, D, dt, hs[i], kh[i]);
    widen_head(vsegs, H, D, dt, hs[i], vh[i]);
  });
  const int blocks = (nr + kRowBlock - 1) / kRowBlock;
  std::atomic<int> status{0};
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  parallel_for(nh * blocks, threads, [&](int item) {
    const int hi = item / blocks, r0 = (item % blocks) * kRowBlock, r1 = std::min(nr, r0 + kRowBlock);
    const int h = hs[hi], m = r1 - r0;
    std::vector<double> qr(size_t(m) * D), ob(size_t(m) * D), lb(m), s;
    for (int r = 0; r < m; ++r)
      for (int d = 0; d < D; ++d) qr[size_t(r) * D + d] = widen(qb, (size_t(rs[r0 + r]) * H + h) * D + d, dt);
    // Row i sees every key before the current chunk and the current chunk's keys of its own
    // causal block and the blocks before it: the first n_fixed + min(n_cur, (i/cb + 1) cb) keys.
    std::vector<int> limit(m);
    for (int r = 0; r < m; ++r) limit[r] = n_fixed + std::min(c.current.n, (rs[r0 + r] / causal_block + 1) * causal_block);
    const auto visible = [&](int r, int j) { return j < limit[r]; };
    if (!attend(m, nk, D, D, qr.data(), kh[hi].data(), vh[hi].data(), scale, visible, ob.data(), lb.data(), nullptr,
                s)) {
      status = 2;
      return;
    }
    for (int r = 0; r < m; ++r) {
      for (int d = 0; d < D; ++d) o[(size_t(r0 + r) * nh + hi) * D + d] = ob[size_t(r) * D + d];
      lse[size_t(hi) * nr + r0 + r] = lb[r];
    }
  });
  return status.load();
}

// The independent dense route over the whole stream, no cache: the sequence [prefix; chunk 0;
// ...; chunk c] (chunk_lens[t] tokens each, concatenated in chunks_k / chunks_v, storage
// [tokens][H][D]) and the last chunk's queries q [chunk_lens[c]][H][D].  The mask is the
// window rule: the last chunk's rows see the prefix, the `window` chunks before it, and their
// own causal blocks of the last chunk.  Writes o [n][H][D] and lse [H][n] (fp64).
int orc_full_sequence_attention(int P, int H, int D, int dtype, const void* pk, const void* pv, int n_chunks,
                                const int* chunk_lens, const void* chunks_k, const void* chunks_v, const void* q,
                                int window, int causal_block, double scale, int threads, double* o, double* lse) {
  if (n_chunks < 1 || causal_block < 1 || window < 0) return 1;
  const size_t tb = size_t(H) * D * elem_bytes(dtype);
  std::vector<int> start(n_chunks + 1, P);  // first sequence position of each chunk
  for (int t = 0; t < n_chunks; ++t) start[t + 1] = start[t] + chunk_lens[t];
  const int N = start[n_chunks], c = n_chunks - 1, n = chunk_lens[c];
  std::vector<std::pair<const uint8_t*, int>> ks{{static_cast<const uint8_t*>(pk), P}},
      vs{{static_cast<const uint8_t*>(pv), P}};
  size_t off = 0;
  for (int t = 0; t < n_chunks; ++t) {
    ks.push_back({static_cast<const uint8_t*>(chunks_k) + off, chunk_lens[t]});
    vs.push_back({static_cast<const uint8_t*>(chunks_v) + off, chunk_lens[t]});
    off += size_t(chunk_lens[t]) * tb;
  }
  // mask row of query i (token i of chunk c) over the whole stream
  const auto visible = [&](int i, int j) {
    if (j < P) return true;
    int t = 0;
    while (j >= start[t + 1]) ++t;
    if (t < c) return c - t <= window;
    return (j - start[c]) / causal_block <= i / causal_block;
  };
  std::atomic<int> status{0};
  parallel_for(H, threads, [&](int h) {
    std::vector<double> kh, vh, qh(size_t(n) * D), oh(size_t(n) * D), lh(n), s;
    widen_head(ks, H, D, dtype, h, kh);
    widen_head(vs, H, D, dtype, h, vh);
    for (int i = 0; i < n; ++i)
      for (int d = 0; d < D; ++d)
        qh[size_t(i) * D + d] = widen(static_cast<const uint8_t*>(q), (size_t(i) * H + h) * D + d, dtype);
    if (!attend(n, N, D, D, qh.data(), kh.data(), vh.data(), scale, visible, oh.data(), lh.data(), nullptr, s)) {
      status = 2;
      return;
    }
    for (int i = 0; i < n; ++i) {
      for (int d = 0; d < D; ++d) o[(size_t(i) * H + h) * D + d] = oh[size_t(i) * D + d];
      lse[size_t(h) * n + i] = lh[i];
    }
  });
  return status.load();
}

}  // extern "C"
