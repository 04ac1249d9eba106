// Host runtime and C ABI of the tokenizer library (declarations and contract
// in include/tok.h).
//
// tok_load validates the merge list and builds the device tables (GraphTok,
// section 5 "Runtime and asset loading" and "Device representation": the
// host resolves every merge to token IDs and builds open-addressed device
// tables at context construction).  Every encode call enqueues the whole
// pipeline on one stream: pre-tokenization -> piece pass (whole-piece hits and
// merge rounds, one run of IDs per tile) -> assembly (output offsets, copy,
// document offsets).  The kernels write the call's results (total, error
// reports) straight into a pinned, device-mapped counter block, so the call
// needs one stream synchronization and no copy to learn its count (TokTier,
// "Exact GPU Tokenization": counts stay on the device and host
// synchronizations drop to a minimum per request; the host path adds one more
// for the ID copy).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/tok.h"
#include "tok_internal.h"

using namespace tok;

namespace {

#define HIP_OK(expr)                       \
  do {                                     \
    if ((expr) != hipSuccess) {            \
      (void)hipGetLastError();             \
      return TOK_E_DEVICE;                 \
    }                                      \
  } while (0)

uint64_t next_pow2(uint64_t x) {
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
void dfree(T*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}

template <typename T>
void hfree(T*& p) {
  if (p) (void)hipHostFree((void*)p);
  p = nullptr;
}

constexpr int kStages = 3;

}  // namespace

struct tok_ctx {
  int device = 0;
  int pattern = 0;
  uint32_t n_merges = 0;
  uint32_t max_tok_len = 1;
  uint32_t n_whole = 0, n_not_self = 0;
  uint64_t config_hash = 0;
  std::vector<uint32_t> tok_len;  // host copy

  // device tables
  uint64_t* d_merge_slots = nullptr;
  uint32_t merge_buckets = 0;
  uint32_t* d_pair_rank = nullptr;
  uint64_t* d_word_slots = nullptr;
  uint32_t word_buckets = 0;
  uint32_t* d_tok_len = nullptr;

  // scratch, grown on demand
  uint64_t cap = 0;  // input bytes the scratch covers
  Bufs b{};
  Counters* d_ctr = nullptr;  // device address of h_ctr
  uint64_t gen = 0;           // number of the last call
  uint8_t* d_text = nullptr;  // staging for host-memory calls
  int32_t* d_ids = nullptr;
  uint64_t doc_cap = 0;
  uint64_t* d_doc = nullptr;
  uint64_t* d_outoff = nullptr;

  // pinned host memory
  uint8_t* h_text = nullptr;
  int32_t* h_ids = nullptr;
  uint64_t* h_doc = nullptr;
  Counters* h_ctr = nullptr;

  hipStream_t stream = nullptr;
  bool prof = false;
  hipEvent_t ev[kStages + 1] = {};
  float stage_ms[kStages] = {};

  Tables tables(bool words = true) const {
    Tables t{};
    t.merge_slots = d_merge_slots;
    t.merge_buckets = merge_buckets;
    t.pair_rank = d_pair_rank;
    t.word_slots = words ? d_word_slots : nullptr;
    t.word_buckets = words ? word_buckets : 0;
    t.tok_len = d_tok_len;
    return t;
  }

  void free_scratch() {
    dfree(b.flags);
    dfree(b.staging);
    dfree(b.tile_cnt);
    dfree(b.tile_first);
    dfree(b.sum1);
    dfree(b.sum2);
    dfree(b.ws_sym);
    dfree(b.ws_rk);
    dfree(b.ws_sel);
    dfree(d_text);
    dfree(d_ids);
    hfree(h_text);
    hfree(h_ids);
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
        hipMalloc((void**)&d_text, c + 64) != hipSuccess ||
        hipMalloc((void**)&d_ids, (c + 64) * sizeof(int32_t)) != hipSuccess ||
        hipHostMalloc((void**)&h_text, c + 64, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&h_ids, (c + 64) * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      free_scratch();
      return TOK_E_NOMEM;
    }
    b.ctr = d_ctr;
    cap = c;
    return TOK_OK;
  }

  int ensure_docs(uint64_t n_docs) {
    if (n_docs + 1 <= doc_cap && d_doc) return TOK_OK;
    (void)hipStreamSynchronize(stream);
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

  void mark(int i, hipStream_t s) {
    if (prof) (void)hipEventRecord(ev[i], s);
  }

  // Enqueue the pipeline over d_text[0..n) and wait for it.  out_flags: stop
  // after pre-tokenization, with the flag words written there.
  int run(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, int32_t* out,
          uint64_t out_cap, uint64_t* out_off, hipStream_t s, bool words, uint16_t* out_flags,
          uint32_t* total) {
    Bufs bb = b;
    if (out_flags) bb.flags = out_flags;
    bb.gen = ++gen;
    const Tables t = tables(words);
    mark(0, s);
    if (n == 0) {  // only a batch of empty documents gets here
      launch_empty_batch(bb, doc_off, n_docs, out_off, s);
    } else {
      launch_pretok(text, n, doc_off, n_docs, pattern, bb, s);
      mark(1, s);
      if (!out_flags) {
        launch_pieces(text, n, t, bb, doc_off, n_docs, out_off, s);
        mark(2, s);
        launch_assemble(n, bb, out, out_cap, doc_off, n_docs, out_off, s);
        mark(3, s);
      }
    }
    HIP_OK(hipGetLastError());
    HIP_OK(hipStreamSynchronize(s));
    if (prof) {
      const int last = n == 0 ? 0 : out_flags ? 1 : kStages;
      for (int i = 0; i < kStages; ++i) {
        float ms = 0.f;
        if (i < last && hipEventElapsedTime(&ms, ev[i], ev[i + 1]) != hipSuccess) ms = 0.f;
        stage_ms[i] = i < last ? ms : 0.f;
      }
    }
    const volatile Counters* c = h_ctr;
    if (c->err_docs == bb.gen) return TOK_E_ARG;
    if (c->err_utf8 == bb.gen) return TOK_E_UTF8;
    if (out_flags) return TOK_OK;
    if (c->done != bb.gen) return TOK_E_DEVICE;
    if (total) *total = c->total;
    return TOK_OK;
  }

  // Run only the merge stages over pieces given by host-built flag words (the
  // load-time self-encoding check of vocabulary strings).
  int run_pieces(const uint8_t* h_bytes, uint64_t n, const std::vector<uint16_t>& flags,
                 std::vector<int32_t>& ids) {
    int rc = ensure(n);
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
    launch_assemble(n, bb, d_ids, n, nullptr, 0, nullptr, stream);
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
    free_scratch();
    dfree(d_merge_slots);
    dfree(d_pair_rank);
    dfree(d_word_slots);
    dfree(d_tok_len);
    dfree(d_doc);
    dfree(d_outoff);
    hfree(h_doc);
    hfree(h_ctr);
    for (auto& e : ev)
      if (e) (void)hipEventDestroy(e);
    if (stream) (void)hipStreamDestroy(stream);
  }
};

namespace {

// Build the whole-piece table from the vocabulary strings of 2..13 bytes
// that the merge kernels encode to their own single token.
int build_word_table(tok_ctx* ctx, const std::vector<std::vector<uint8_t>>& tok) {
  std::vector<uint32_t> cand;
  std::vector<uint8_t> blob;
  std::vector<uint16_t> flags;
  for (uint32_t id = 256; id < tok.size(); ++id) {
    const size_t L = tok[id].size();
    if (L < 2 || L > (size_t)kWordMax) continue;
    const uint64_t pos = blob.size();
    if (flags.size() * kChunk <= pos) flags.resize(pos / kChunk + 1, 0);
    flags[pos / kChunk] |= (uint16_t)(1u << (pos % kChunk));
    blob.insert(blob.end(), tok[id].begin(), tok[id].end());
    cand.push_back(id);
  }
  if (cand.empty()) return TOK_OK;
  flags.resize((blob.size() + kChunk - 1) / kChunk + 8, 0);
  std::vector<int32_t> ids;
  int rc = ctx->run_pieces(blob.data(), blob.size(), flags, ids);
  if (rc) return rc;
  std::vector<uint32_t> self;
  size_t k = 0;
  for (uint32_t id : cand) {
    const size_t L = tok[id].size();
    size_t got = 0, used = 0;
    bool one = k < ids.size() && ids[k] == (int32_t)id;
    while (got < L && k < ids.size()) {
      got += ctx->tok_len[(uint32_t)ids[k++]];
      ++used;
    }
    if (got != L) return TOK_E_DEVICE;  // token lengths must tile each string
    if (one && used == 1) self.push_back(id);
  }
  ctx->n_whole = (uint32_t)self.size();
  ctx->n_not_self = (uint32_t)(cand.size() - self.size());
  if (self.empty()) return TOK_OK;
  const uint64_t slots = std::max<uint64_t>(next_pow2(2 * self.size()), 64);
  const uint32_t bmask = (uint32_t)(slots / kBucket - 1);
  std::vector<uint64_t> tab(2 * slots, 0);
  for (uint32_t id : self) {
    const auto& s = tok[id];
    uint64_t a = 0, bb = 0;
    for (size_t i = 0; i < s.size() && i < 8; ++i) a |= (uint64_t)s[i] << (8 * i);
    for (size_t i = 8; i < s.size(); ++i) bb |= (uint64_t)s[i] << (8 * (i - 8));
    bb |= (uint64_t)s.size() << 40;
    uint32_t h = word_hash(a, bb) & bmask;
    for (bool placed = false; !placed; h = (h + 1) & bmask) {
      for (uint32_t j = 0; j < kBucket && !placed; ++j) {
        const size_t at = ((size_t)h * kBucket + j) * 2;
        if (tab[at + 1] == 0) {
          tab[at] = a;
          tab[at + 1] = bb | ((uint64_t)id << 44);
          placed = true;
        }
      }
    }
  }
  HIP_OK(hipMalloc((void**)&ctx->d_word_slots, tab.size() * 8));
  HIP_OK(hipMemcpy(ctx->d_word_slots, tab.data(), tab.size() * 8, hipMemcpyHostToDevice));
  ctx->word_buckets = bmask;
  return TOK_OK;
}

}  // namespace

extern "C" {

const char* tok_strerror(int code) {
  switch (code) {
    case TOK_OK: return "ok";
    case TOK_E_ARG: return "invalid argument";
    case TOK_E_BADMERGES: return "invalid merge list";
    case TOK_E_PATTERN: return "unsupported pre-tokenizer pattern";
    case TOK_E_UTF8: return "malformed UTF-8 input";
    case TOK_E_CAPACITY: return "output buffer too small";
    case TOK_E_TOOLONG: return "input too long";
    case TOK_E_DEVICE: return "HIP device error";
    case TOK_E_NOMEM: return "out of memory";
    case TOK_E_SESSION: return "session IDs do not match the old text";
    default: return "unknown error";
  }
}

int tok_load(const uint32_t* merges, size_t n_merges, int pattern, int device, tok_ctx** out) {
  if (!out || (!merges && n_merges)) return TOK_E_ARG;
  *out = nullptr;
  if (pattern != TOK_PAT_GPT2 && pattern != TOK_PAT_LLAMA3) return TOK_E_PATTERN;
  if (n_merges > TOK_MAX_MERGES) return TOK_E_BADMERGES;
  // operands precede their merge, and each ordered pair has one rank
  // open addressing over buckets of kBucket slots, at most half full; a key
  // lives in the first bucket of its probe sequence with a free slot, taking
  // the bucket's first free slot (lookups stop at a bucket with a free slot)
  const uint64_t slots = std::max<uint64_t>(next_pow2(2 * n_merges), 1024);
  const uint32_t bmask = (uint32_t)(slots / kBucket - 1);
  std::vector<uint64_t> mtab(slots, kEmptySlot);
  std::vector<uint32_t> pr(65536, kNoRank);
  std::vector<std::vector<uint8_t>> tok(256 + n_merges);
  for (uint32_t i = 0; i < 256; ++i) tok[i] = {(uint8_t)i};
  for (size_t r = 0; r < n_merges; ++r) {
    const uint32_t a = merges[2 * r], bb = merges[2 * r + 1];
    if (a >= 256 + r || bb >= 256 + r) return TOK_E_BADMERGES;
    const uint64_t key = ((uint64_t)a << 20) | bb;
    uint32_t h = merge_hash(a, bb) & bmask;
    for (bool placed = false; !placed; h = (h + 1) & bmask) {
      for (uint32_t j = 0; j < kBucket && !placed; ++j) {
        uint64_t& slot = mtab[(size_t)h * kBucket + j];
        if (slot == kEmptySlot) {
          slot = (key << 24) | r;
          placed = true;
        } else if ((slot >> 24) == key) {
          return TOK_E_BADMERGES;  // the same ordered pair twice
        }
      }
    }
    if ((a | bb) < 256) pr[(a << 8) | bb] = (uint32_t)r;
    tok[256 + r] = tok[a];
    tok[256 + r].insert(tok[256 + r].end(), tok[bb].begin(), tok[bb].end());
  }
  tok_ctx* ctx = new (std::nothrow) tok_ctx();
  if (!ctx) return TOK_E_NOMEM;
  ctx->device = device;
  ctx->pattern = pattern;
  ctx->n_merges = (uint32_t)n_merges;
  ctx->tok_len.resize(tok.size());
  for (size_t i = 0; i < tok.size(); ++i) {
    ctx->tok_len[i] = (uint32_t)tok[i].size();
    ctx->max_tok_len = std::max(ctx->max_tok_len, ctx->tok_len[i]);
  }
  uint64_t h = 0xCBF29CE484222325ull;  // FNV-1a over pattern and merges
  auto fnv = [&](const void* p, size_t n) {
    const uint8_t* c = (const uint8_t*)p;
    for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001B3ull;
  };
  const uint32_t pat32 = (uint32_t)pattern;
  fnv(&pat32, 4);
  if (n_merges) fnv(merges, n_merges * 8);
  ctx->config_hash = h;

  DeviceGuard g(device);
  int rc = TOK_E_DEVICE;
  do {
    if (hipSetDevice(device) != hipSuccess) break;
    if (hipStreamCreateWithFlags(&ctx->stream, hipStreamNonBlocking) != hipSuccess) break;
    bool ok = true;
    for (auto& e : ctx->ev) ok = ok && hipEventCreate(&e) == hipSuccess;
    if (!ok) break;
    if (hipMalloc((void**)&ctx->d_merge_slots, slots * 8) != hipSuccess ||
        hipMalloc((void**)&ctx->d_pair_rank, pr.size() * 4) != hipSuccess ||
        hipMalloc((void**)&ctx->d_tok_len, ctx->tok_len.size() * 4) != hipSuccess ||
        hipHostMalloc((void**)&ctx->h_ctr, sizeof(Counters), hipHostMallocMapped) != hipSuccess) {
      rc = TOK_E_NOMEM;
      break;
    }
    if (hipMemcpy(ctx->d_merge_slots, mtab.data(), slots * 8, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ctx->d_pair_rank, pr.data(), pr.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ctx->d_tok_len, ctx->tok_len.data(), ctx->tok_len.size() * 4, hipMemcpyHostToDevice) !=
            hipSuccess ||
        hipHostGetDevicePointer((void**)&ctx->d_ctr, ctx->h_ctr, 0) != hipSuccess)
      break;
    std::memset(ctx->h_ctr, 0, sizeof(Counters));
    ctx->b.ctr = ctx->d_ctr;
    ctx->merge_buckets = bmask;
    rc = build_word_table(ctx, tok);
  } while (false);
  if (rc != TOK_OK) {
    (void)hipGetLastError();
    delete ctx;
    return rc;
  }
  *out = ctx;
  return TOK_OK;
}

void tok_free(tok_ctx* ctx) {
  if (!ctx) return;
  DeviceGuard g(ctx->device);
  delete ctx;
}

int tok_encode_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, int32_t* d_ids, size_t cap,
                   size_t* n_out, void* stream) {
  if (!ctx || !n_out || (!d_text && len) || (!d_ids && cap)) return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if (len == 0) return TOK_OK;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len);
  if (rc) return rc;
  hipStream_t s = stream ? (hipStream_t)stream : ctx->stream;
  uint32_t total = 0;
  rc = ctx->run(d_text, len, nullptr, 0, d_ids, cap, nullptr, s, true, nullptr, &total);
  if (rc) return rc;
  *n_out = total;
  return total > cap ? TOK_E_CAPACITY : TOK_OK;
}

int tok_encode(tok_ctx* ctx, const uint8_t* text, size_t len, int32_t* ids, size_t cap, size_t* n_out) {
  if (!ctx || !n_out || (!text && len) || (!ids && cap)) return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if (len == 0) return TOK_OK;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len);
  if (rc) return rc;
  hipStream_t s = ctx->stream;
  std::memcpy(ctx->h_text, text, len);
  HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, len, hipMemcpyHostToDevice, s));
  uint32_t total = 0;
  rc = ctx->run(ctx->d_text, len, nullptr, 0, ctx->d_ids, len, nullptr, s, true, nullptr, &total);
  if (rc) return rc;
  *n_out = total;
  if (total > cap) return TOK_E_CAPACITY;
  HIP_OK(hipMemcpyAsync(ctx->h_ids, ctx->d_ids, (size_t)total * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipStreamSynchronize(s));
  std::memcpy(ids, ctx->h_ids, (size_t)total * 4);
  return TOK_OK;
}

int tok_encode_batch_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, const uint64_t* d_doc_off,
                         size_t n_docs, int32_t* d_ids, size_t cap, uint64_t* d_out_off, size_t* n_out,
                         void* stream) {
  if (!ctx || !n_out || !d_doc_off || !d_out_off || n_docs == 0 || n_docs >= 0xFFFFFFFFu ||
      (!d_text && len) || (!d_ids && cap))
    return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len ? len : 1);
  if (rc) return rc;
  hipStream_t s = stream ? (hipStream_t)stream : ctx->stream;
  uint32_t total = 0;
  rc = ctx->run(d_text, len, d_doc_off, (uint32_t)n_docs, d_ids, cap, d_out_off, s, true, nullptr, &total);
  if (rc) return rc;
  *n_out = total;
  return total > cap ? TOK_E_CAPACITY : TOK_OK;
}

int tok_encode_batch(tok_ctx* ctx, const uint8_t* text, const uint64_t* doc_off, size_t n_docs,
                     int32_t* ids, size_t cap, uint64_t* out_off) {
  if (!ctx || !doc_off || !out_off || n_docs == 0 || n_docs >= 0xFFFFFFFFu) return TOK_E_ARG;
  if (doc_off[0] != 0) return TOK_E_ARG;
  for (size_t d = 0; d < n_docs; ++d)
    if (doc_off[d + 1] < doc_off[d]) return TOK_E_ARG;
  const uint64_t len = doc_off[n_docs];
  if ((!text && len) || (!ids && cap)) return TOK_E_ARG;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len ? len : 1);
  if (rc) return rc;
  rc = ctx->ensure_docs(n_docs);
  if (rc) return rc;
  hipStream_t s = ctx->stream;
  if (len) {
    std::memcpy(ctx->h_text, text, len);
    HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, len, hipMemcpyHostToDevice, s));
  }
  std::memcpy(ctx->h_doc, doc_off, (n_docs + 1) * 8);
  HIP_OK(hipMemcpyAsync(ctx->d_doc, ctx->h_doc, (n_docs + 1) * 8, hipMemcpyHostToDevice, s));
  uint32_t total = 0;
  rc = ctx->run(ctx->d_text, len, ctx->d_doc, (uint32_t)n_docs, ctx->d_ids, len, ctx->d_outoff, s, true,
                nullptr, &total);
  if (rc) return rc;
  HIP_OK(hipMemcpyAsync(ctx->h_doc, ctx->d_outoff, (n_docs + 1) * 8, hipMemcpyDeviceToHost, s));
  if (total <= cap && total)
    HIP_OK(hipMemcpyAsync(ctx->h_ids, ctx->d_ids, (size_t)total * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipStreamSynchronize(s));
  std::memcpy(out_off, ctx->h_doc, (n_docs + 1) * 8);
  if (total > cap) return TOK_E_CAPACITY;
  if (total) std::memcpy(ids, ctx->h_ids, (size_t)total * 4);
  return TOK_OK;
}

int tok_pretokenize_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, const uint64_t* d_doc_off,
                        size_t n_docs, uint16_t* d_flags, void* stream) {
  if (!ctx || (!d_text && len) || (!d_flags && len) || (d_doc_off && n_docs == 0) ||
      n_docs >= 0xFFFFFFFFu)
    return TOK_E_ARG;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if (len == 0) return TOK_OK;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len);
  if (rc) return rc;
  hipStream_t s = stream ? (hipStream_t)stream : ctx->stream;
  return ctx->run(d_text, len, d_doc_off, (uint32_t)(d_doc_off ? n_docs : 0), nullptr, 0, nullptr, s, true,
                  d_flags, nullptr);
}

int tok_get_info(const tok_ctx* ctx, tok_info* info) {
  if (!ctx || !info) return TOK_E_ARG;
  info->pattern = (uint32_t)ctx->pattern;
  info->n_merges = ctx->n_merges;
  info->vocab_size = 256 + ctx->n_merges;
  info->max_token_len = ctx->max_tok_len;
  info->n_whole = ctx->n_whole;
  info->n_not_self = ctx->n_not_self;
  info->config_hash = ctx->config_hash;
  return TOK_OK;
}

size_t tok_token_lengths(const tok_ctx* ctx, uint32_t* len_out, size_t n) {
  if (!ctx) return 0;
  const size_t v = ctx->tok_len.size();
  if (len_out) std::memcpy(len_out, ctx->tok_len.data(), std::min(n, v) * 4);
  return v;
}

int tok_set_profiling(tok_ctx* ctx, int on) {
  if (!ctx) return TOK_E_ARG;
  ctx->prof = on != 0;
  return TOK_OK;
}

int tok_stage_ms(const tok_ctx* ctx, float* ms, int n) {
  if (!ctx || !ms || n < 0) return 0;
  const int k = std::min(n, kStages);
  for (int i = 0; i < k; ++i) ms[i] = ctx->stage_ms[i];
  return k;
}

}  // extern "C"
