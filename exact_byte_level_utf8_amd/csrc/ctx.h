// Tokenizer context shared by the host sources of the library (capi.hip,
// repair.hip): device tables, per-call scratch, pinned staging, the stream,
// and the pipeline launch of one call.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tok.h"
#include "ext_internal.h"

using namespace tok;  // internal header of the library's host sources only

// Device address of the no-allocation scratch array on `device` (current),
// looked up on the first call for that device (noalloc.hip); nullptr if the
// lookup failed.
uint8_t* noalloc_scratch(int device);

#define HIP_OK(expr)                       \
  do {                                     \
    if ((expr) != hipSuccess) {            \
      (void)hipGetLastError();             \
      return TOK_E_DEVICE;                 \
    }                                      \
  } while (0)

inline uint64_t next_pow2(uint64_t x) {
  uint64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

template <typename T>
inline void dfree(T*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}

template <typename T>
inline void hfree(T*& p) {
  if (p) (void)hipHostFree((void*)p);
  p = nullptr;
}

constexpr int kStages = 3;  // pre-tokenization, piece pass, assembly

// Key of a captured pipeline: every argument baked into its kernel launches.
struct GraphKey {
  const uint8_t* text;
  uint64_t n;
  const uint64_t* doc_off;
  uint32_t n_docs;
  int32_t* out;
  uint32_t* spans;
  uint64_t out_cap;
  uint64_t* out_off;
  hipStream_t s;
  bool words;
  bool lits;  // the added-token literal pass ahead of the pipeline
  bool operator==(const GraphKey& o) const {
    return text == o.text && n == o.n && doc_off == o.doc_off && n_docs == o.n_docs && out == o.out &&
           spans == o.spans && out_cap == o.out_cap && out_off == o.out_off && s == o.s && words == o.words &&
           lits == o.lits;
  }
};

struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec;
  uint64_t gen;   // the call number baked into the graph's status reports
  uint64_t used;  // last use, for eviction
};

constexpr size_t kMaxGraphs = 8;

struct tok_ctx {
  int device = 0;
  int pattern = 0;
  uint32_t n_merges = 0;
  uint32_t max_tok_len = 1;
  uint32_t n_whole = 0, n_not_self = 0;
  uint64_t config_hash = 0;
  uint32_t repair_window = 512;    // first repair window, code points
  uint32_t repair_doublings = 5;   // window doublings before the full encode
  uint32_t repair_margin = 8;      // code points into the window of a certifying boundary
  std::vector<uint32_t> tok_len;  // host copy
  std::vector<uint8_t> tok_bytes;  // host copy of every token's bytes, concatenated
  std::vector<uint64_t> tok_off;   // token i is tok_bytes[tok_off[i] .. tok_off[i + 1])

  // device tables
  uint64_t* d_merge_slots = nullptr;
  uint32_t merge_buckets = 0;
  uint32_t* d_pair_rank = nullptr;
  uint64_t* d_word_slots = nullptr;
  uint32_t word_buckets = 0;
  uint64_t* d_long_slots = nullptr;
  uint32_t long_buckets = 0;
  uint32_t* d_tok_len = nullptr;
  uint32_t* d_tok_min = nullptr;  // per token: (x >> min_shift) << 16 | (y >> min_shift), see Tables
  uint32_t min_shift = 0;
  uint32_t* d_unit_tab = nullptr;  // kUnitTabWords: where no token can span a byte boundary (tok_internal.h)
  uint64_t* d_hand_tick = nullptr;  // Bufs::hand_tick, for the context's life (never cleared after load)

  // every token's bytes on the device, made on first use (device repair)
  uint8_t* d_tok_bytes = nullptr;
  uint64_t* d_tok_off = nullptr;

  // added-token literals (tok_set_added_tokens); n_lit == 0: none
  uint32_t n_lit = 0;
  std::vector<std::vector<uint8_t>> lit_str;        // host copy, for the repair
  std::vector<int32_t> lit_id;
  std::vector<std::vector<uint32_t>> lit_by_first;  // literal indices by first byte
  uint32_t lit_max_len = 0;
  bool lit_ids_clash = false;  // an ID shared with the vocabulary or another literal
  uint8_t* d_lit_bytes = nullptr;
  uint32_t* d_lit_off = nullptr;
  int32_t* d_lit_ids = nullptr;
  uint32_t* d_lit_key2 = nullptr;
  uint16_t* d_lit_order = nullptr;
  int32_t* d_lit_key1 = nullptr;
  uint32_t* d_lit_first = nullptr;
  uint64_t* d_lit_by_id = nullptr;
  LitBufs lb{};
  uint64_t lit_cap = 0;   // input bytes lb covers
  uint64_t lit_docs = 0;  // documents lb covers

  // scratch, grown on demand
  uint64_t cap = 0;  // input bytes the scratch covers
  Bufs b{};
  Counters* d_ctr = nullptr;  // device address of h_ctr
  uint64_t gen = 0;           // number of the last call
  uint8_t* d_text = nullptr;  // staging for host-memory calls
  int32_t* d_ids = nullptr;
  uint32_t* d_spans = nullptr;  // span staging of host-memory calls, made on first use
  uint64_t doc_cap = 0;
  uint64_t* d_doc = nullptr;
  uint64_t* d_outoff = nullptr;

  // pinned host memory
  uint8_t* h_text = nullptr;
  int32_t* h_ids = nullptr;
  uint32_t* h_spans = nullptr;
  uint64_t* h_doc = nullptr;
  Counters* h_ctr = nullptr;

  hipStream_t stream = nullptr;
  uint32_t prof = 0;  // bit i: time stage i with events
  hipEvent_t ev0[kStages] = {}, ev1[kStages] = {};  // start / end of each stage's kernel
  float stage_ms[kStages] = {};

  // graph replay (off by default): one captured pipeline per call shape
  bool graph_mode = false;
  std::vector<GraphEntry> graphs;
  std::vector<GraphKey> seen;  // shapes met once, not captured yet
  uint64_t graph_tick = 0;

  void drop_graphs() {
    for (auto& g : graphs) (void)hipGraphExecDestroy(g.exec);
    graphs.clear();
    seen.clear();
  }

  Tables tables(bool words = true) const {
    Tables t{};
    t.merge_slots = d_merge_slots;
    t.merge_buckets = merge_buckets;
    t.pair_rank = d_pair_rank;
    t.word_slots = words ? d_word_slots : nullptr;
    t.word_buckets = words ? word_buckets : 0;
    t.long_slots = words ? d_long_slots : nullptr;
    t.long_buckets = words ? long_buckets : 0;
    t.tok_len = d_tok_len;
    t.tok_min = d_tok_min;
    t.min_shift = min_shift;
    t.max_tok_len = max_tok_len;
    return t;
  }

  void free_scratch() {
    drop_graphs();  // their launches point into the scratch
    dfree(b.flags);
    dfree(b.staging);
    dfree(b.tile_cnt);
    dfree(b.tile_first);
    dfree(b.sum1);
    dfree(b.sum2);
    dfree(b.ws_sym);
    dfree(b.ws_rk);
    dfree(b.ws_sel);
    dfree(b.hand_state);
    free_lit_bufs();
    dfree(d_text);
    dfree(d_ids);
    dfree(d_spans);
    hfree(h_text);
    hfree(h_ids);
    hfree(h_spans);
    cap = 0;
  }

  // Make the scratch cover n input bytes (capacity grows in powers of two).
  int ensure(uint64_t n) {
    if (n <= cap && b.flags) return TOK_OK;
    (void)hipStreamSynchronize(stream);
    free_scratch();
    const uint64_t c = std::max<uint64_t>(next_pow2(n), 1u << 16);
    const uint64_t chunks = c / kChunk, tiles = c / kPieceTile;
    if (hipMalloc((void**)&b.flags, (chunks + 8) * sizeof(uint16_t)) != hipSuccess ||
        hipMalloc((void**)&b.staging, (c + 64) * sizeof(int32_t)) != hipSuccess ||
        hipMalloc((void**)&b.tile_cnt, tiles * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.tile_first, tiles * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.ws_sym, (c + 64) * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.ws_rk, (c + 64) * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.ws_sel, (c + 64) * sizeof(uint64_t)) != hipSuccess ||
        hipMalloc((void**)&b.sum1, ((tiles >> kSum1Shift) + 1) * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.sum2, ((tiles >> kSum2Shift) + 1) * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc((void**)&b.hand_state, (c / kPretokTile + 1) * sizeof(uint64_t)) != hipSuccess ||
        hipMemsetAsync(b.hand_state, 0, (c / kPretokTile + 1) * sizeof(uint64_t), stream) != hipSuccess) {
      (void)hipGetLastError();
      free_scratch();
      return TOK_E_NOMEM;
    }
    b.ctr = d_ctr;
    cap = c;
    return TOK_OK;
  }

  // Fill every per-call device buffer with byte v and wait (a diagnostic:
  // no call may depend on what an earlier one left in them).  The hand-over
  // words of the case-splitting pre-tokenization are not per-call data: they
  // carry the numbering of the calls, and are left as they are.
  int fill_scratch(uint8_t v) {
    auto fill = [&](void* p, uint64_t bytes) { return !p || hipMemsetAsync(p, v, bytes, stream) == hipSuccess; };
    bool ok = true;
    if (b.flags) {
      const uint64_t chunks = cap / kChunk, tiles = cap / kPieceTile;
      ok = fill(b.flags, (chunks + 8) * 2) && fill(b.staging, (cap + 64) * 4) && fill(b.tile_cnt, tiles * 4) &&
           fill(b.tile_first, tiles * 4) && fill(b.ws_sym, (cap + 64) * 4) && fill(b.ws_rk, (cap + 64) * 4) &&
           fill(b.ws_sel, (cap + 64) * 8) && fill(b.sum1, ((tiles >> kSum1Shift) + 1) * 4) &&
           fill(b.sum2, ((tiles >> kSum2Shift) + 1) * 4) && fill(d_text, cap + 64) && fill(d_ids, (cap + 64) * 4) &&
           fill(d_spans, (cap + 64) * 4);
    }
    if (ok && lb.cand) {
      const uint64_t parts = lit_docs + 2 * lit_cap;
      ok = fill(lb.cand, lit_cap * 8) && fill(lb.tile_cnt, lit_cap / kLitTile * 4) && fill(lb.sel, lit_cap * 8) &&
           fill(lb.cut, (parts + 2) * 8) && fill(lb.part_lit, (parts + 2) * 4) &&
           fill(lb.doc_part, (lit_docs + 2) * 4) && fill(lb.out_off, (parts + 2) * 8) &&
           fill(lb.fin, (parts + 2) * 4) && fill(lb.misc, 32) && fill(lb.ids, (lit_cap + 64) * 4) &&
           fill(lb.spans, (lit_cap + 64) * 4) && fill(lb.lmark, lit_cap + 64) && fill(lb.lid_at, lit_cap * 4);
    }
    if (ok && d_doc) ok = fill(d_doc, doc_cap * 8) && fill(d_outoff, doc_cap * 8);
    if (!ok || hipStreamSynchronize(stream) != hipSuccess) {
      (void)hipGetLastError();
      return TOK_E_DEVICE;
    }
    return TOK_OK;
  }

  void free_lit_tables() {
    drop_graphs();  // their launches carry these tables
    dfree(d_lit_bytes);
    dfree(d_lit_off);
    dfree(d_lit_ids);
    dfree(d_lit_key2);
    dfree(d_lit_order);
    dfree(d_lit_key1);
    dfree(d_lit_first);
    dfree(d_lit_by_id);
    n_lit = 0;
    lit_str.clear();
    lit_id.clear();
    lit_by_first.clear();
    lit_max_len = 0;
    lit_ids_clash = false;
  }

  void free_lit_bufs() {
    drop_graphs();  // their launches point into these buffers
    dfree(lb.cand);
    dfree(lb.tile_cnt);
    dfree(lb.sel);
    dfree(lb.cut);
    dfree(lb.part_lit);
    dfree(lb.doc_part);
    dfree(lb.out_off);
    dfree(lb.fin);
    dfree(lb.misc);
    dfree(lb.ids);
    dfree(lb.spans);
    dfree(lb.lmark);
    dfree(lb.lid_at);
    lit_cap = 0;
    lit_docs = 0;
  }

  Literals literals() const {
    return Literals{d_lit_bytes, d_lit_off, d_lit_ids, d_lit_key2, d_lit_order, d_lit_key1, d_lit_first, d_lit_by_id,
                    n_lit};
  }

  // Buffers of the literal pass for the current capacity and n_docs
  // documents (after ensure()): at most cap literals, so at most n_docs +
  // 2 cap parts.
  int ensure_lit_bufs(uint64_t n_docs) {
    if (lit_cap == cap && n_docs <= lit_docs && lb.cand) return TOK_OK;
    free_lit_bufs();
    const uint64_t tiles = cap / kLitTile;
    const uint64_t docs = std::max<uint64_t>(next_pow2(n_docs), 64);
    const uint64_t parts = docs + 2 * cap;
    if (hipMalloc((void**)&lb.cand, cap * 8) != hipSuccess ||
        hipMalloc((void**)&lb.tile_cnt, tiles * 4) != hipSuccess ||
        hipMalloc((void**)&lb.sel, cap * 8) != hipSuccess ||
        hipMalloc((void**)&lb.cut, (parts + 2) * 8) != hipSuccess ||
        hipMalloc((void**)&lb.part_lit, (parts + 2) * 4) != hipSuccess ||
        hipMalloc((void**)&lb.doc_part, (docs + 2) * 4) != hipSuccess ||
        hipMalloc((void**)&lb.out_off, (parts + 2) * 8) != hipSuccess ||
        hipMalloc((void**)&lb.fin, (parts + 2) * 4) != hipSuccess ||
        hipMalloc((void**)&lb.misc, 32) != hipSuccess ||
        hipMalloc((void**)&lb.ids, (cap + 64) * 4) != hipSuccess ||
        hipMalloc((void**)&lb.spans, (cap + 64) * 4) != hipSuccess ||
        hipMalloc((void**)&lb.lmark, cap + 64) != hipSuccess || hipMalloc((void**)&lb.lid_at, cap * 4) != hipSuccess) {
      (void)hipGetLastError();
      free_lit_bufs();
      return TOK_E_NOMEM;
    }
    lit_cap = cap;
    lit_docs = docs;
    return TOK_OK;
  }

  // Encode with the added-token literals: the literal pass (matches never
  // cross a document boundary), the pipeline over the parts as documents
  // whose count the kernels read on the device, and the insertion of the
  // literal IDs, all enqueued at once; one synchronization.  doc_off /
  // n_docs / out_off: the caller's documents and their output offsets, or
  // nullptr for one request.  spans (optional): each ID's first byte.
  // Whether a call folds the literal IDs into the piece pass: every call but
  // those with span export (whose assembly scans token byte lengths, which a
  // literal's ID does not give) and empty ones.
  static bool folds_literals(uint64_t n, const uint32_t* spans) { return n > 0 && !spans; }

  // The same, enqueued under call number `call` without waiting (after
  // ensure_lit_bufs()).  Folded: the literal pass marks the taken literals,
  // the pipeline over the parts takes each as one piece with its ID and
  // writes the result, and only a batch's document offsets are mapped after
  // it.  Otherwise the pipeline encodes the literals' own bytes too, and the
  // insertion puts the literal IDs in place of those tokens.
  void enqueue_added(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, int32_t* out,
                     uint64_t out_cap, uint64_t* out_off, hipStream_t s, uint64_t call, uint32_t* spans) {
    Bufs bb = b;
    bb.gen = call;
    bb.n_docs_dev = lb.misc + 2;
    LitBufs l = lb;
    l.fold = folds_literals(n, spans) ? 1u : 0u;
    launch_literal_pass(text, n, doc_off, n_docs, literals(), l, d_ctr, call, s);
    if (l.fold) {
      const Literals L = literals();
      bb.lit = LitMarks{lb.sel, lb.misc + 1, L.off, L.ids, lb.lmark, lb.lid_at};
      enqueue(text, n, lb.cut, 1, out, nullptr, out_cap, lb.out_off, s, bb, true, nullptr);
      if (out_off) launch_literal_doc_offsets(l, out_off, doc_off ? n_docs : 1u, s);
      return;
    }
    enqueue(text, n, lb.cut, 1, lb.ids, spans ? lb.spans : nullptr, n, lb.out_off, s, bb, true, nullptr);
    launch_literal_insert(n, literals(), l, out, spans, out_cap, out_off, d_ctr, call, s);
  }

  int run_added(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, int32_t* out,
                uint64_t out_cap, uint64_t* out_off, hipStream_t s, uint32_t* total, uint32_t* spans = nullptr) {
    int rc = ensure_lit_bufs(doc_off ? n_docs : 1);
    if (rc) return rc;
    volatile Counters* c = h_ctr;
    uint64_t call = 0;
    GraphEntry* g = nullptr;
    if (graph_mode && !prof && n > 0)
      g = graph_for(GraphKey{text, n, doc_off, n_docs, out, spans, out_cap, out_off, s, true, true});
    if (g) {  // a replay reports the call number baked in at capture: clear its words first
      call = g->gen;
      c->err_utf8 = 0;
      c->err_docs = 0;
      c->done = 0;
      c->lit_done = 0;
      c->ins_done = 0;
      HIP_OK(hipGraphLaunch(g->exec, s));
    } else {
      call = ++gen;
      enqueue_added(text, n, doc_off, n_docs, out, out_cap, out_off, s, call, spans);
    }
    HIP_OK(hipGetLastError());
    HIP_OK(hipStreamSynchronize(s));
    if (prof) {
      for (int i = 0; i < kStages; ++i) {
        float ms = 0.f;
        if (((prof >> i) & 1u) && hipEventElapsedTime(&ms, ev0[i], ev1[i]) != hipSuccess) ms = 0.f;
        stage_ms[i] = ((prof >> i) & 1u) ? ms : 0.f;
      }
    }
    if (c->err_docs == call) return TOK_E_ARG;  // the caller's document offsets (the parts are well formed)
    if (c->err_utf8 == call) return TOK_E_UTF8;
    if (c->lit_done != call || c->done != call || (!folds_literals(n, spans) && c->ins_done != call))
      return TOK_E_DEVICE;
    *total = c->total;
    return TOK_OK;
  }

  int ensure_tok_bytes() {
    if (d_tok_bytes) return TOK_OK;
    if (hipMalloc((void**)&d_tok_bytes, tok_bytes.size() + 64) != hipSuccess ||
        hipMalloc((void**)&d_tok_off, tok_off.size() * 8) != hipSuccess) {
      (void)hipGetLastError();
      dfree(d_tok_bytes);
      dfree(d_tok_off);
      return TOK_E_NOMEM;
    }
    if (hipMemcpy(d_tok_bytes, tok_bytes.data(), tok_bytes.size(), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_tok_off, tok_off.data(), tok_off.size() * 8, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipGetLastError();
      dfree(d_tok_bytes);
      dfree(d_tok_off);
      return TOK_E_DEVICE;
    }
    return TOK_OK;
  }

  // Staging of host-memory calls (device copies of the text and IDs, pinned
  // host buffers), sized like the scratch (after ensure()); calls on device
  // buffers never allocate it.
  int ensure_host() {
    if (d_text) return TOK_OK;
    if (hipMalloc((void**)&d_text, cap + 64) != hipSuccess ||
        hipMalloc((void**)&d_ids, (cap + 64) * sizeof(int32_t)) != hipSuccess ||
        hipHostMalloc((void**)&h_text, cap + 64, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&h_ids, (cap + 64) * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      dfree(d_text);
      dfree(d_ids);
      hfree(h_text);
      hfree(h_ids);
      return TOK_E_NOMEM;
    }
    return TOK_OK;
  }

  // Span staging for host-memory calls, sized like d_ids (after ensure()).
  int ensure_spans() {
    if (d_spans) return TOK_OK;
    if (hipMalloc((void**)&d_spans, (cap + 64) * sizeof(uint32_t)) != hipSuccess ||
        hipHostMalloc((void**)&h_spans, (cap + 64) * sizeof(uint32_t), hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      dfree(d_spans);
      hfree(h_spans);
      return TOK_E_NOMEM;
    }
    return TOK_OK;
  }

  int ensure_docs(uint64_t n_docs) {
    if (n_docs + 1 <= doc_cap && d_doc) return TOK_OK;
    (void)hipStreamSynchronize(stream);
    drop_graphs();
    dfree(d_doc);
    dfree(d_outoff);
    hfree(h_doc);
    const uint64_t c = std::max<uint64_t>(next_pow2(n_docs + 1), 64);
    if (hipMalloc((void**)&d_doc, c * 8) != hipSuccess || hipMalloc((void**)&d_outoff, c * 8) != hipSuccess ||
        hipHostMalloc((void**)&h_doc, c * 8, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      dfree(d_doc);
      dfree(d_outoff);
      hfree(h_doc);
      doc_cap = 0;
      return TOK_E_NOMEM;
    }
    doc_cap = c;
    return TOK_OK;
  }

  // After a call's synchronization: the durations of its timed stages (the
  // first `last` stages ran), 0 for the others.
  void collect_stage_times(int last) {
    if (!prof) return;
    for (int i = 0; i < kStages; ++i) {
      float ms = 0.f;
      const bool timed = i < last && ((prof >> i) & 1u);
      if (timed && hipEventElapsedTime(&ms, ev0[i], ev1[i]) != hipSuccess) ms = 0.f;
      stage_ms[i] = timed ? ms : 0.f;
    }
  }

  // start and end events for stage i when it is timed, else none
  hipEvent_t e0(int i) const { return (prof >> i) & 1u ? ev0[i] : nullptr; }
  hipEvent_t e1(int i) const { return (prof >> i) & 1u ? ev1[i] : nullptr; }

  // The three stages of one call, enqueued on s (eagerly or under capture).
  void enqueue(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, int32_t* out,
               uint32_t* spans, uint64_t out_cap, uint64_t* out_off, hipStream_t s, const Bufs& bb, bool words,
               uint16_t* out_flags) {
    const Tables t = tables(words);
    if (n == 0) {  // only a batch of empty documents gets here
      launch_empty_batch(bb, doc_off, n_docs, out_off, s);
      return;
    }
    // the pre-tokenization alone (out_flags) gives piece starts; the pipeline
    // also starts a unit of BPE between bytes that no token spans
    launch_pretok(text, n, doc_off, n_docs, pattern, out_flags ? nullptr : d_unit_tab, bb, s, e0(0), e1(0));
    if (out_flags) return;
    launch_pieces(text, n, t, bb, doc_off, n_docs, out_off, s, e0(1), e1(1));
    launch_assemble(n, bb, out, spans, d_tok_len, out_cap, doc_off, n_docs, out_off, s, e0(2), e1(2));
  }

  // The captured pipeline for this call shape: found, or captured now on s
  // with a fresh call number when the shape was met before.  nullptr for a
  // shape met for the first time (it runs eagerly, so one-off shapes pay no
  // capture) or when capture fails.
  GraphEntry* graph_for(const GraphKey& k) {
    for (auto& g : graphs)
      if (g.key == k) {
        g.used = ++graph_tick;
        return &g;
      }
    auto it = std::find(seen.begin(), seen.end(), k);
    if (it == seen.end()) {
      if (seen.size() >= 2 * kMaxGraphs) seen.erase(seen.begin());
      seen.push_back(k);
      return nullptr;
    }
    seen.erase(it);
    Bufs bb = b;
    bb.gen = ++gen;
    hipGraph_t gr = nullptr;
    hipGraphExec_t ex = nullptr;
    if (hipStreamBeginCapture(k.s, hipStreamCaptureModeThreadLocal) != hipSuccess) return nullptr;
    if (k.lits)
      enqueue_added(k.text, k.n, k.doc_off, k.n_docs, k.out, k.out_cap, k.out_off, k.s, bb.gen, k.spans);
    else
      enqueue(k.text, k.n, k.doc_off, k.n_docs, k.out, k.spans, k.out_cap, k.out_off, k.s, bb, k.words, nullptr);
    const bool captured = hipStreamEndCapture(k.s, &gr) == hipSuccess && gr;
    const bool made = captured && hipGraphInstantiate(&ex, gr, nullptr, nullptr, 0) == hipSuccess;
    if (gr) (void)hipGraphDestroy(gr);
    if (!made) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (graphs.size() >= kMaxGraphs) {
      auto lru = std::min_element(graphs.begin(), graphs.end(),
                                  [](const GraphEntry& a, const GraphEntry& c) { return a.used < c.used; });
      (void)hipGraphExecDestroy(lru->exec);
      graphs.erase(lru);
    }
    graphs.push_back(GraphEntry{k, ex, bb.gen, ++graph_tick});
    return &graphs.back();
  }

  // Enqueue the pipeline over d_text[0..n) and wait for it.  out_flags: stop
  // after pre-tokenization, with the flag words written there.  In graph mode
  // a call without stage timing replays the pipeline captured for its shape;
  // the status words are cleared first, since every replay reports the call
  // number that was captured.
  int run(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, int32_t* out,
          uint32_t* spans, uint64_t out_cap, uint64_t* out_off, hipStream_t s, bool words, uint16_t* out_flags,
          uint32_t* total) {
    volatile Counters* c = h_ctr;
    uint64_t call = 0;
    GraphEntry* g = nullptr;
    if (graph_mode && !prof && !out_flags && n > 0)
      g = graph_for(GraphKey{text, n, doc_off, n_docs, out, spans, out_cap, out_off, s, words, false});
    if (g) {
      call = g->gen;
      c->err_utf8 = 0;
      c->err_docs = 0;
      c->done = 0;
      HIP_OK(hipGraphLaunch(g->exec, s));
    } else {
      Bufs bb = b;
      if (out_flags) bb.flags = out_flags;
      bb.gen = call = ++gen;
      enqueue(text, n, doc_off, n_docs, out, spans, out_cap, out_off, s, bb, words, out_flags);
    }
    HIP_OK(hipGetLastError());
    HIP_OK(hipStreamSynchronize(s));
    collect_stage_times(n == 0 ? 0 : out_flags ? 1 : kStages);
    if (c->err_docs == call) return TOK_E_ARG;
    if (c->err_utf8 == call) return TOK_E_UTF8;
    if (out_flags) return TOK_OK;
    if (c->done != call) return TOK_E_DEVICE;
    if (total) *total = c->total;
    return TOK_OK;
  }

  // Run only the merge stages over pieces given by host-built flag words (the
  // load-time self-encoding check of vocabulary strings).
  int run_pieces(const uint8_t* h_bytes, uint64_t n, const std::vector<uint16_t>& flags,
                 std::vector<int32_t>& ids) {
    int rc = ensure(n);
    if (!rc) rc = ensure_host();
    if (rc) return rc;
    HIP_OK(hipMemcpyAsync(d_text, h_bytes, n, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(b.flags, flags.data(), flags.size() * 2, hipMemcpyHostToDevice, stream));
    Bufs bb = b;
    bb.gen = ++gen;
    const uint32_t tiles = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
    std::vector<uint32_t> zero((tiles >> kSum1Shift) + 1, 0);  // group sums start at zero
    HIP_OK(hipMemcpyAsync(bb.sum1, zero.data(), zero.size() * 4, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(bb.sum2, zero.data(), ((tiles >> kSum2Shift) + 1) * 4, hipMemcpyHostToDevice, stream));
    const Tables t = tables(false);
    launch_pieces(d_text, n, t, bb, nullptr, 0, nullptr, stream);
    launch_assemble(n, bb, d_ids, nullptr, nullptr, n, nullptr, 0, nullptr, stream);
    HIP_OK(hipGetLastError());
    HIP_OK(hipStreamSynchronize(stream));
    const volatile Counters* c = h_ctr;
    if (c->done != bb.gen) return TOK_E_DEVICE;
    ids.resize(c->total);
    HIP_OK(hipMemcpy(ids.data(), d_ids, ids.size() * 4, hipMemcpyDeviceToHost));
    return TOK_OK;
  }

  ~tok_ctx() {
    if (stream) (void)hipStreamSynchronize(stream);
    free_scratch();  // and the captured graphs
    dfree(d_merge_slots);
    dfree(d_pair_rank);
    dfree(d_word_slots);
    dfree(d_long_slots);
    dfree(d_tok_len);
    dfree(d_tok_min);
    dfree(d_unit_tab);
    dfree(d_hand_tick);
    free_lit_tables();
    dfree(d_tok_bytes);
    dfree(d_tok_off);
    dfree(d_doc);
    dfree(d_outoff);
    hfree(h_doc);
    hfree(h_ctr);
    for (int i = 0; i < kStages; ++i) {
      if (ev0[i]) (void)hipEventDestroy(ev0[i]);
      if (ev1[i]) (void)hipEventDestroy(ev1[i]);
    }
    if (stream) (void)hipStreamDestroy(stream);
  }
};

