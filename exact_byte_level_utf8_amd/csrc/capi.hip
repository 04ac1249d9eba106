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

#include "ctx.h"

using namespace tok;

namespace {

// Build the whole-piece tables from the vocabulary strings of 2..28 bytes
// that the merge kernels encode to their own single token: 2..13-byte keys in
// 16-byte slots, 14..28-byte keys in 32-byte slots.
int build_word_table(tok_ctx* ctx, const std::vector<std::vector<uint8_t>>& tok) {
  std::vector<uint32_t> cand;
  std::vector<uint8_t> blob;
  std::vector<uint16_t> flags;
  for (uint32_t id = 256; id < tok.size(); ++id) {
    const size_t L = tok[id].size();
    if (L < 2 || L > (size_t)kLongMax) continue;
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
  std::vector<uint32_t> self_short, self_long;
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
    if (one && used == 1) (L <= (size_t)kWordMax ? self_short : self_long).push_back(id);
  }
  ctx->n_whole = (uint32_t)(self_short.size() + self_long.size());
  ctx->n_not_self = (uint32_t)(cand.size() - ctx->n_whole);
  auto key_bytes = [&](const std::vector<uint8_t>& s, size_t from, size_t to) {
    uint64_t v = 0;
    for (size_t i = from; i < s.size() && i < to; ++i) v |= (uint64_t)s[i] << (8 * (i - from));
    return v;
  };
  if (!self_short.empty()) {
    const uint64_t slots = std::max<uint64_t>(next_pow2(2 * self_short.size()), 64);
    const uint32_t bmask = (uint32_t)(slots / kBucket - 1);
    std::vector<uint64_t> tab(2 * slots, 0);
    for (uint32_t id : self_short) {
      const auto& s = tok[id];
      const uint64_t a = key_bytes(s, 0, 8), bb = key_bytes(s, 8, 13) | ((uint64_t)s.size() << 40);
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
  }
  if (!self_long.empty()) {
    const uint64_t slots = std::max<uint64_t>(next_pow2(2 * self_long.size()), 64);
    const uint32_t bmask = (uint32_t)(slots / kBucket - 1);
    std::vector<uint64_t> tab(4 * slots, 0);
    for (uint32_t id : self_long) {
      const auto& s = tok[id];
      const uint64_t k0 = key_bytes(s, 0, 8), k1 = key_bytes(s, 8, 16), k2 = key_bytes(s, 16, 24);
      const uint64_t k3 = key_bytes(s, 24, 28) | ((uint64_t)s.size() << 32);
      uint32_t h = long_hash(k0, k1, k2, k3) & bmask;
      for (bool placed = false; !placed; h = (h + 1) & bmask) {
        for (uint32_t j = 0; j < kBucket && !placed; ++j) {
          const size_t at = ((size_t)h * kBucket + j) * 4;
          if (tab[at + 3] == 0) {
            tab[at] = k0;
            tab[at + 1] = k1;
            tab[at + 2] = k2;
            tab[at + 3] = k3 | ((uint64_t)id << 37);
            placed = true;
          }
        }
      }
    }
    HIP_OK(hipMalloc((void**)&ctx->d_long_slots, tab.size() * 8));
    HIP_OK(hipMemcpy(ctx->d_long_slots, tab.data(), tab.size() * 8, hipMemcpyHostToDevice));
    ctx->long_buckets = bmask;
  }
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

void tok_opts_default(tok_opts* opts) {
  if (!opts) return;
  *opts = tok_opts{};
  opts->device = 0;
  opts->initial_bytes = 0;
  opts->repair_window = 512;
  opts->repair_doublings = 5;
  opts->repair_margin = 8;
  opts->handoff_wait_us = 1000000;
}

int tok_load(const uint32_t* merges, size_t n_merges, int pattern, const tok_opts* opts, tok_ctx** out) {
  if (!out || (!merges && n_merges)) return TOK_E_ARG;
  *out = nullptr;
  tok_opts o;
  tok_opts_default(&o);
  if (opts) o = *opts;
  if (o.device < 0 || o.repair_window < 1 || o.repair_window > (1u << 24) || o.repair_doublings > 24 ||
      o.repair_margin > (1u << 20) || o.initial_bytes > TOK_MAX_BYTES || o.handoff_wait_us > 10000000u)
    return TOK_E_ARG;
  const int device = o.device;
  if (pattern != TOK_PAT_GPT2 && pattern != TOK_PAT_LLAMA3 && pattern != TOK_PAT_O200K) return TOK_E_PATTERN;
  if (n_merges > TOK_MAX_MERGES) return TOK_E_BADMERGES;
  // operands precede their merge, and each ordered pair has one rank
  // open addressing over buckets of kBucket slots, at most half full (denser
  // tables send more lookups of absent pairs on to a second bucket, and the
  // merge rounds wait on those loads); a key lives in the first bucket of its
  // probe sequence with a free slot, taking the bucket's first free slot
  // (lookups stop at a bucket with a free slot)
  const uint64_t slots = std::max<uint64_t>(next_pow2(2 * n_merges), 1024);
  const uint32_t nbk = (uint32_t)(slots / kBucket);
  std::vector<uint64_t> mtab(slots, kEmptySlot);
  std::vector<uint32_t> pr(65536, kNoRank);
  // per token: lowest rank of a merge taking it as right operand (x), as
  // left operand (y); kNoRank for none
  std::vector<uint32_t> tmin(2 * (256 + n_merges), kNoRank);
  std::vector<std::vector<uint8_t>> tok(256 + n_merges);
  for (uint32_t i = 0; i < 256; ++i) tok[i] = {(uint8_t)i};
  // byte pairs that some token spans, one bit per (first << 8 | second): the
  // junction of each merge (the pairs inside its operands are set already)
  std::vector<uint32_t> join(kUnitTabWords, 0u);  // the unit table: pairs, two-byte tokens, three-byte strings
  for (size_t r = 0; r < n_merges; ++r) {
    const uint32_t a = merges[2 * r], bb = merges[2 * r + 1];
    if (a >= 256 + r || bb >= 256 + r) return TOK_E_BADMERGES;
    const uint64_t key = ((uint64_t)a << 20) | bb;
    uint32_t h = merge_bucket(a, bb, nbk);
    for (bool placed = false; !placed; h = next_bucket(h, nbk)) {
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
    tmin[2 * (size_t)bb] = std::min(tmin[2 * (size_t)bb], (uint32_t)r);
    tmin[2 * (size_t)a + 1] = std::min(tmin[2 * (size_t)a + 1], (uint32_t)r);
    const uint32_t jp = ((uint32_t)tok[a].back() << 8) | tok[bb].front();
    join[jp >> 5] |= 1u << (jp & 31u);
    tok[256 + r] = tok[a];
    tok[256 + r].insert(tok[256 + r].end(), tok[bb].begin(), tok[bb].end());
  }
  // the rest of the unit table: two-byte tokens, and every three-byte string
  // inside a token (hashed)
  for (size_t t = 256; t < tok.size(); ++t) {
    const std::vector<uint8_t>& b = tok[t];
    if (b.size() == 2) {
      const uint32_t k = ((uint32_t)b[0] << 8) | b[1];
      join[kJoinWords + (k >> 5)] |= 1u << (k & 31u);
    }
    for (size_t i = 0; i + 2 < b.size(); ++i) {
      const uint32_t h = tri_slot((uint32_t)b[i] | (uint32_t)b[i + 1] << 8 | (uint32_t)b[i + 2] << 16);
      join[2 * kJoinWords + (h >> 5)] |= 1u << (h & 31u);
    }
  }
  // the same ranks, 16 bits each in one word per token: the rank shifted
  // right so that every rank fits below 0xFFFF (which stands for none).  A
  // floor only makes the shelter test stricter, so merging stays exact.
  uint32_t min_shift = 0;
  while (n_merges && ((uint64_t)(n_merges - 1) >> min_shift) >= 0xFFFFu) ++min_shift;
  std::vector<uint32_t> tmin16(256 + n_merges);
  for (size_t t = 0; t < tmin16.size(); ++t) {
    auto q = [&](uint32_t r) { return r == kNoRank ? 0xFFFFu : r >> min_shift; };
    tmin16[t] = (q(tmin[2 * t]) << 16) | q(tmin[2 * t + 1]);
  }
  tok_ctx* ctx = new (std::nothrow) tok_ctx();
  if (!ctx) return TOK_E_NOMEM;
  ctx->device = device;
  ctx->pattern = pattern;
  ctx->repair_window = o.repair_window;
  ctx->repair_doublings = o.repair_doublings;
  ctx->repair_margin = o.repair_margin;
  ctx->n_merges = (uint32_t)n_merges;
  ctx->min_shift = min_shift;
  ctx->tok_len.resize(tok.size());
  ctx->tok_off.resize(tok.size() + 1);
  ctx->tok_off[0] = 0;
  for (size_t i = 0; i < tok.size(); ++i) {
    ctx->tok_len[i] = (uint32_t)tok[i].size();
    ctx->max_tok_len = std::max(ctx->max_tok_len, ctx->tok_len[i]);
    ctx->tok_off[i + 1] = ctx->tok_off[i] + tok[i].size();
  }
  ctx->tok_bytes.reserve(ctx->tok_off.back());
  for (const auto& t : tok) ctx->tok_bytes.insert(ctx->tok_bytes.end(), t.begin(), t.end());
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
    // a blocking stream: ordered with the legacy default stream, on which
    // callers that pass no stream usually produced the input
    if (hipStreamCreate(&ctx->stream) != hipSuccess) break;
    bool ok = true;
    // timing-only events: no system-scope fence (no cache write-back and
    // invalidation around the timed kernels)
    for (int i = 0; i < kStages; ++i)
      ok = ok && hipEventCreateWithFlags(&ctx->ev0[i], hipEventDisableSystemFence) == hipSuccess &&
           hipEventCreateWithFlags(&ctx->ev1[i], hipEventDisableSystemFence) == hipSuccess;
    if (!ok) break;
    if (hipMalloc((void**)&ctx->d_merge_slots, slots * 8) != hipSuccess ||
        hipMalloc((void**)&ctx->d_pair_rank, pr.size() * 4) != hipSuccess ||
        hipMalloc((void**)&ctx->d_tok_len, ctx->tok_len.size() * 4) != hipSuccess ||
        hipMalloc((void**)&ctx->d_tok_min, tmin16.size() * 4) != hipSuccess ||
        hipMalloc((void**)&ctx->d_unit_tab, join.size() * 4) != hipSuccess ||
        hipMalloc((void**)&ctx->d_hand_tick, kHandTickWords * 8) != hipSuccess ||
        hipHostMalloc((void**)&ctx->h_ctr, sizeof(Counters), hipHostMallocMapped) != hipSuccess) {
      rc = TOK_E_NOMEM;
      break;
    }
    if (hipMemcpy(ctx->d_merge_slots, mtab.data(), slots * 8, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ctx->d_pair_rank, pr.data(), pr.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ctx->d_tok_len, ctx->tok_len.data(), ctx->tok_len.size() * 4, hipMemcpyHostToDevice) !=
            hipSuccess ||
        hipMemcpy(ctx->d_tok_min, tmin16.data(), tmin16.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ctx->d_unit_tab, join.data(), join.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(ctx->d_hand_tick, 0, kHandTickWords * 8) != hipSuccess ||
        hipHostGetDevicePointer((void**)&ctx->d_ctr, ctx->h_ctr, 0) != hipSuccess)
      break;
    // the hand-over wait in wall-clock ticks (the clock's rate is in kHz)
    int clock_khz = 0;
    if (hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, device) != hipSuccess || clock_khz <= 0)
      break;
    ctx->b.hand_tick = ctx->d_hand_tick;
    ctx->b.hand_wait = (uint64_t)o.handoff_wait_us * (uint64_t)clock_khz / 1000u;
    std::memset(ctx->h_ctr, 0, sizeof(Counters));
    // the no-allocation entry point's array: its address on this device, once
    // per device (a failed lookup only disables that entry point)
    (void)noalloc_scratch(device);
    ctx->b.ctr = ctx->d_ctr;
    ctx->merge_buckets = nbk;
    rc = build_word_table(ctx, tok);
    if (rc == TOK_OK && o.initial_bytes) rc = ctx->ensure(o.initial_bytes);
  } while (false);
  if (rc != TOK_OK) {
    (void)hipGetLastError();
    delete ctx;
    return rc;
  }
  *out = ctx;
  return TOK_OK;
}

int tok_fill_scratch(tok_ctx* ctx, int value) {
  if (!ctx || value < 0 || value > 255) return TOK_E_ARG;
  DeviceGuard g(ctx->device);
  return ctx->fill_scratch((uint8_t)value);
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
  rc = ctx->n_lit ? ctx->run_added(d_text, len, nullptr, 0, d_ids, cap, nullptr, s, &total)
                  : ctx->run(d_text, len, nullptr, 0, d_ids, nullptr, cap, nullptr, s, true, nullptr, &total);
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
  if (!rc) rc = ctx->ensure_host();
  if (rc) return rc;
  hipStream_t s = ctx->stream;
  std::memcpy(ctx->h_text, text, len);
  HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, len, hipMemcpyHostToDevice, s));
  uint32_t total = 0;
  rc = ctx->n_lit ? ctx->run_added(ctx->d_text, len, nullptr, 0, ctx->d_ids, len, nullptr, s, &total)
                  : ctx->run(ctx->d_text, len, nullptr, 0, ctx->d_ids, nullptr, len, nullptr, s, true, nullptr, &total);
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
  rc = ctx->n_lit && len ? ctx->run_added(d_text, len, d_doc_off, (uint32_t)n_docs, d_ids, cap, d_out_off, s, &total)
                         : ctx->run(d_text, len, d_doc_off, (uint32_t)n_docs, d_ids, nullptr, cap, d_out_off, s, true,
                                    nullptr, &total);
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
  if (!rc) rc = ctx->ensure_host();
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
  rc = ctx->n_lit && len ? ctx->run_added(ctx->d_text, len, ctx->d_doc, (uint32_t)n_docs, ctx->d_ids, len,
                                           ctx->d_outoff, s, &total)
                         : ctx->run(ctx->d_text, len, ctx->d_doc, (uint32_t)n_docs, ctx->d_ids, nullptr, len,
                                    ctx->d_outoff, s, true, nullptr, &total);
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

int tok_encode_spans_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, const uint64_t* d_doc_off,
                         size_t n_docs, int32_t* d_ids, uint32_t* d_spans, size_t cap, uint64_t* d_out_off,
                         size_t* n_out, void* stream) {
  if (!ctx || !n_out || (!d_text && len) || (cap && (!d_ids || !d_spans)) || n_docs >= 0xFFFFFFFFu ||
      (d_doc_off && (n_docs == 0 || !d_out_off)))
    return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if (len == 0 && !d_doc_off) return TOK_OK;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len ? len : 1);
  if (rc) return rc;
  hipStream_t s = stream ? (hipStream_t)stream : ctx->stream;
  uint32_t total = 0;
  rc = ctx->n_lit && len ? ctx->run_added(d_text, len, d_doc_off, d_doc_off ? (uint32_t)n_docs : 0, d_ids, cap,
                                           d_doc_off ? d_out_off : nullptr, s, &total, d_spans)
                  : ctx->run(d_text, len, d_doc_off, d_doc_off ? (uint32_t)n_docs : 0, d_ids, d_spans, cap,
                             d_doc_off ? d_out_off : nullptr, s, true, nullptr, &total);
  if (rc) return rc;
  *n_out = total;
  return total > cap ? TOK_E_CAPACITY : TOK_OK;
}

int tok_encode_spans(tok_ctx* ctx, const uint8_t* text, size_t len, int32_t* ids, uint32_t* spans, size_t cap,
                     size_t* n_out) {
  if (!ctx || !n_out || (!text && len) || (cap && (!ids || !spans))) return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if (len == 0) return TOK_OK;
  DeviceGuard g(ctx->device);
  int rc = ctx->ensure(len);
  if (!rc) rc = ctx->ensure_host();
  if (!rc) rc = ctx->ensure_spans();
  if (rc) return rc;
  hipStream_t s = ctx->stream;
  std::memcpy(ctx->h_text, text, len);
  HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, len, hipMemcpyHostToDevice, s));
  uint32_t total = 0;
  rc = ctx->n_lit ? ctx->run_added(ctx->d_text, len, nullptr, 0, ctx->d_ids, len, nullptr, s, &total, ctx->d_spans)
                  : ctx->run(ctx->d_text, len, nullptr, 0, ctx->d_ids, ctx->d_spans, len, nullptr, s, true, nullptr,
                             &total);
  if (rc) return rc;
  *n_out = total;
  if (total > cap) return TOK_E_CAPACITY;
  HIP_OK(hipMemcpyAsync(ctx->h_ids, ctx->d_ids, (size_t)total * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipMemcpyAsync(ctx->h_spans, ctx->d_spans, (size_t)total * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipStreamSynchronize(s));
  std::memcpy(ids, ctx->h_ids, (size_t)total * 4);
  std::memcpy(spans, ctx->h_spans, (size_t)total * 4);
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
  return ctx->run(d_text, len, d_doc_off, (uint32_t)(d_doc_off ? n_docs : 0), nullptr, nullptr, 0, nullptr, s, true,
                  d_flags, nullptr);
}

int tok_set_added_tokens(tok_ctx* ctx, const uint8_t* bytes, const uint64_t* off, size_t n, const int32_t* ids) {
  if (!ctx || (n && (!bytes || !off || !ids)) || n > kLitMaxCount) return TOK_E_ARG;
  DeviceGuard g(ctx->device);
  (void)hipStreamSynchronize(ctx->stream);
  ctx->free_lit_tables();
  if (n == 0) return TOK_OK;
  if (off[0] != 0) return TOK_E_ARG;
  std::vector<std::vector<uint8_t>> lit(n);
  for (size_t i = 0; i < n; ++i) {
    if (off[i + 1] <= off[i] || off[i + 1] - off[i] > (uint64_t)kLitMax || ids[i] < 0) return TOK_E_ARG;
    lit[i].assign(bytes + off[i], bytes + off[i + 1]);
  }
  // each literal is whole UTF-8 (so it starts and ends on code-point
  // boundaries of any valid text), and no string is given twice
  for (const auto& x : lit) {
    size_t i = 0;
    while (i < x.size()) {
      const uint32_t b0 = x[i];
      const uint32_t len = b0 < 0x80 ? 1 : (b0 >= 0xC2 && b0 < 0xE0) ? 2 : (b0 >= 0xE0 && b0 < 0xF0) ? 3
                                                                       : (b0 >= 0xF0 && b0 < 0xF5) ? 4 : 0;
      if (!len || i + len > x.size()) return TOK_E_UTF8;
      uint32_t cp = b0 & (0x7Fu >> len);
      for (uint32_t k = 1; k < len; ++k) {
        if ((x[i + k] & 0xC0) != 0x80) return TOK_E_UTF8;
        cp = (cp << 6) | (x[i + k] & 0x3Fu);
      }
      if ((len == 3 && (cp < 0x800 || (cp >= 0xD800 && cp < 0xE000))) || (len == 4 && (cp < 0x10000 || cp > 0x10FFFF)))
        return TOK_E_UTF8;
      i += len;
    }
  }
  {
    std::vector<size_t> idx(n);
    for (size_t i = 0; i < n; ++i) idx[i] = i;
    std::sort(idx.begin(), idx.end(), [&](size_t a, size_t c) { return lit[a] < lit[c]; });
    for (size_t i = 1; i < n; ++i)
      if (lit[idx[i]] == lit[idx[i - 1]]) return TOK_E_ARG;
  }
  std::vector<uint32_t> first(8, 0), key2(65536, 0);
  std::vector<int32_t> key1(256, -1);
  std::vector<uint16_t> order;
  std::vector<std::vector<uint16_t>> groups(65536);
  for (size_t i = 0; i < n; ++i) {
    const uint32_t b0 = lit[i][0];
    first[b0 >> 5] |= 1u << (b0 & 31u);
    if (lit[i].size() == 1) key1[b0] = (int32_t)i;
    else groups[b0 | ((uint32_t)lit[i][1] << 8)].push_back((uint16_t)i);
  }
  for (uint32_t k = 0; k < 65536; ++k) {
    auto& gk = groups[k];
    if (gk.empty()) continue;
    std::sort(gk.begin(), gk.end(), [&](uint16_t a, uint16_t c) { return lit[a].size() > lit[c].size(); });
    key2[k] = ((uint32_t)order.size() << 16) | (uint32_t)gk.size();
    order.insert(order.end(), gk.begin(), gk.end());
  }
  std::vector<uint8_t> blob;
  std::vector<uint32_t> loff(n + 1, 0);
  for (size_t i = 0; i < n; ++i) {
    blob.insert(blob.end(), lit[i].begin(), lit[i].end());
    loff[i + 1] = (uint32_t)blob.size();
  }
  blob.resize(blob.size() + 72, 0);  // the match kernel reads whole words up to 8 bytes past a literal
  std::vector<uint64_t> by_id(n);
  for (size_t i = 0; i < n; ++i) by_id[i] = ((uint64_t)(uint32_t)ids[i] << 32) | i;
  std::sort(by_id.begin(), by_id.end());
  if (hipMalloc((void**)&ctx->d_lit_by_id, n * 8) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_bytes, blob.size()) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_off, loff.size() * 4) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_ids, n * 4) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_key2, key2.size() * 4) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_order, std::max<size_t>(order.size(), 1) * 2) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_key1, key1.size() * 4) != hipSuccess ||
      hipMalloc((void**)&ctx->d_lit_first, first.size() * 4) != hipSuccess) {
    (void)hipGetLastError();
    ctx->free_lit_tables();
    return TOK_E_NOMEM;
  }
  if (hipMemcpy(ctx->d_lit_by_id, by_id.data(), n * 8, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->d_lit_bytes, blob.data(), blob.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->d_lit_off, loff.data(), loff.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->d_lit_ids, ids, n * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->d_lit_key2, key2.data(), key2.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      (order.size() && hipMemcpy(ctx->d_lit_order, order.data(), order.size() * 2, hipMemcpyHostToDevice) != hipSuccess) ||
      hipMemcpy(ctx->d_lit_key1, key1.data(), key1.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->d_lit_first, first.data(), first.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    ctx->free_lit_tables();
    return TOK_E_DEVICE;
  }
  ctx->n_lit = (uint32_t)n;
  ctx->lit_str = lit;
  ctx->lit_id.assign(ids, ids + n);
  ctx->lit_by_first.assign(256, {});
  ctx->lit_max_len = 0;
  for (size_t i = 0; i < n; ++i) {
    ctx->lit_by_first[lit[i][0]].push_back((uint32_t)i);
    ctx->lit_max_len = std::max(ctx->lit_max_len, (uint32_t)lit[i].size());
  }
  std::vector<int32_t> sorted_ids(ids, ids + n);
  std::sort(sorted_ids.begin(), sorted_ids.end());
  ctx->lit_ids_clash = sorted_ids[0] < (int32_t)ctx->tok_len.size() ||
                       std::adjacent_find(sorted_ids.begin(), sorted_ids.end()) != sorted_ids.end();
  return TOK_OK;
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

int tok_set_graph(tok_ctx* ctx, int on) {
  if (!ctx || on < 0 || on > 1) return TOK_E_ARG;
  DeviceGuard g(ctx->device);
  (void)hipStreamSynchronize(ctx->stream);
  ctx->graph_mode = on == 1;
  if (!ctx->graph_mode) ctx->drop_graphs();
  return TOK_OK;
}

size_t tok_graph_count(const tok_ctx* ctx) { return ctx ? ctx->graphs.size() : 0; }

int tok_set_profiling(tok_ctx* ctx, int stages) {
  if (!ctx || stages < 0) return TOK_E_ARG;
  ctx->prof = (uint32_t)stages & TOK_STAGES_ALL;
  return TOK_OK;
}

int tok_stage_ms(const tok_ctx* ctx, float* ms, int n) {
  if (!ctx || !ms || n < 0) return 0;
  const int k = std::min(n, kStages);
  for (int i = 0; i < k; ++i) ms[i] = ctx->stage_ms[i];
  return k;
}

}  // extern "C"
