// Append repair: tok_repair, and its splice certificate tok_sync_boundary.
//
// A session keeps the IDs of its text A.  When text B is appended, only a
// window at the seam is encoded again: the last w code points of A plus B
// (TokTier, section 3, windowed repair; Delta Tokenizer, reference-identical
// tokenization of session deltas).  The fresh records (byte offset, ID) of the
// window are matched against the stored records; a run of equal records is
// accepted if it contains a stable pre-tokenization boundary, and the result
// is the stored IDs up to the end of that run followed by the fresh IDs after
// it (TokTier, Appendix A: Definition A.4 splice certificate, Theorem A.5,
// Corollary A.6 -- splicing at the end of the equal run is interchangeable
// with splicing at the boundary inside it).  If no run qualifies the window
// doubles, at most five times, and then the whole text is encoded.  A miss
// costs work, never a different ID.
//
// The stable boundary used here is a synchronizing transition (sync_rules.h).
//
// Work per call is O(w + |B|): the stored IDs are walked back from the end
// through the token byte lengths, never from the start of the session.
#include "ctx.h"
#include "pretok_rules.h"
#include "sync_rules.h"

namespace {

#define TOK_CLS_QUAL static
#include "uniclass.inc"
#include "uniclass_case.inc"
#undef TOK_CLS_QUAL

uint32_t host_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
  if (cp < TOK_CLS_LOW) return (kClsLow[cp >> 2] >> (2 * (cp & 3u))) & 3u;
  if (cp >= 0x110000) return kO;
  const uint32_t blk = kClsBlock[cp >> 8];
  return (kClsBits[blk * 64 + ((cp & 255u) >> 2)] >> (2 * (cp & 3u))) & 3u;
}

uint32_t host_case(uint32_t cp) {
  if (cp < TOK_CLS_LOW) return (kCaseLow[cp >> 1] >> (4 * (cp & 1u))) & 15u;
  if (cp >= 0x110000) return 6u;
  const uint32_t blk = kCaseBlock[cp >> 8];
  return (kCaseBits[blk * 128 + ((cp & 255u) >> 1)] >> (4 * (cp & 1u))) & 15u;
}

bool is_cont(uint8_t b) { return (b & 0xC0) == 0x80; }

// Code point whose lead byte is t[i] (the text is valid UTF-8 around i).
uint32_t cp_at(const uint8_t* t, uint64_t n, uint64_t i) {
  const uint32_t b0 = t[i];
  if (b0 < 0x80) return b0;
  const uint32_t len = b0 >= 0xF0 ? 4 : b0 >= 0xE0 ? 3 : 2;
  uint32_t cp = b0 & (0x7Fu >> len);
  for (uint32_t k = 1; k < len && i + k < n; ++k) cp = (cp << 6) | (t[i + k] & 0x3Fu);
  return cp;
}

// Lead byte of the code point that ends just before byte i (i > 0).
uint64_t prev_lead(const uint8_t* t, uint64_t i) {
  uint64_t j = i - 1;
  while (j > 0 && is_cont(t[j])) --j;
  return j;
}

// Byte offset of the w-th code point before byte `end` (0 if there are fewer).
uint64_t back_code_points(const uint8_t* t, uint64_t end, uint64_t w) {
  uint64_t i = end, seen = 0;
  while (i > 0 && seen < w) {
    --i;
    if (!is_cont(t[i])) ++seen;
  }
  return i;
}

// Byte offset of the code point that lies w code points after byte `start`
// (`end` if there are fewer).
uint64_t fwd_code_points(const uint8_t* t, uint64_t start, uint64_t end, uint64_t w) {
  uint64_t i = start, seen = 0;
  while (i < end) {
    if (!is_cont(t[i])) {
      if (seen == w) return i;
      ++seen;
    }
    ++i;
  }
  return end;
}

bool sync_transition(int pattern, uint32_t x, uint32_t y) {
  if (pattern == TOK_PAT_O200K) return sync_transition_case(x, host_case(x), y, host_case(y));
  return sync_transition_of(pattern == TOK_PAT_GPT2, x, host_class(x), y, host_class(y));
}

struct Rec {
  uint64_t off;  // byte offset of the token in the text
  size_t idx;    // index in its sequence (session or window)
  int32_t id;
};

}  // namespace

extern "C" {

int tok_sync_boundary(int pattern, uint32_t prev_cp, uint32_t cp) {
  if (pattern != TOK_PAT_GPT2 && pattern != TOK_PAT_LLAMA3 && pattern != TOK_PAT_O200K) return 0;
  return sync_transition(pattern, prev_cp, cp) ? 1 : 0;
}

int tok_repair(tok_ctx* ctx, int32_t* session_ids, size_t n_session, size_t cap, const uint8_t* text,
               size_t old_len, size_t new_len, size_t* n_out, tok_repair_info* info) {
  if (!ctx || !n_out || (!text && new_len) || (!session_ids && (cap || n_session)) || old_len > new_len ||
      n_session > cap)
    return TOK_E_ARG;
  *n_out = 0;
  tok_repair_info scratch{};
  tok_repair_info& inf = info ? *info : scratch;
  inf = tok_repair_info{};
  if (new_len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if ((old_len == 0) != (n_session == 0)) return TOK_E_SESSION;
  if (ctx->n_lit && ctx->lit_ids_clash) {  // an ID that names two strings: no walk-back; encode the whole text
    inf.full = 1;
    return tok_encode(ctx, text, new_len, session_ids, cap, n_out);
  }
  if (new_len == old_len) {  // nothing appended: the stored IDs are the answer
    *n_out = n_session;
    inf.kept = n_session;
    inf.splice_byte = old_len;
    return TOK_OK;
  }

  // the bytes of an ID: a vocabulary token, or an added-token literal (their
  // IDs are distinct here); false for an ID that is neither
  const size_t vocab = ctx->tok_len.size();
  auto token_str = [&](int32_t id, const uint8_t** b, uint32_t* L) -> bool {
    if (id >= 0 && (size_t)id < vocab) {
      *b = &ctx->tok_bytes[ctx->tok_off[(size_t)id]];
      *L = ctx->tok_len[(size_t)id];
      return true;
    }
    for (size_t i = 0; i < ctx->lit_id.size(); ++i)
      if (ctx->lit_id[i] == id) {
        *b = ctx->lit_str[i].data();
        *L = (uint32_t)ctx->lit_str[i].size();
        return true;
      }
    return false;
  };
  auto token_len = [&](int32_t id) -> uint32_t {
    const uint8_t* b = nullptr;
    uint32_t L = 0;
    return token_str(id, &b, &L) ? L : 0u;
  };
  // an added-token literal occurrence (taken or not) that covers bytes b - 1
  // and b: no cut may fall inside one (Delta Tokenizer, section 3, the cut
  // guard over every occurrence of every special-token string)
  auto inside_literal = [&](uint64_t b) -> bool {
    if (!ctx->n_lit) return false;
    const uint64_t from = b > ctx->lit_max_len ? b - ctx->lit_max_len + 1 : 0;
    for (uint64_t p = from; p < b; ++p)
      for (uint32_t li : ctx->lit_by_first[text[p]]) {
        const auto& x = ctx->lit_str[li];
        if (p + x.size() > b && p + x.size() <= new_len && std::memcmp(text + p, x.data(), x.size()) == 0)
          return true;
      }
    return false;
  };
  const uint32_t longest = std::max(ctx->max_tok_len, ctx->lit_max_len);

  // stored records, walked back from the end of the session as far as needed
  std::vector<Rec> stored;  // in reverse order of offset
  uint64_t pos = old_len;
  size_t j = n_session;
  auto walk_to = [&](uint64_t target) -> int {
    while (pos > target && j > 0) {
      const int32_t id = session_ids[j - 1];
      const uint8_t* tb = nullptr;
      uint32_t L = 0;
      if (!token_str(id, &tb, &L) || L > pos) return TOK_E_SESSION;
      pos -= L;
      --j;
      if (std::memcmp(tb, text + pos, L) != 0) return TOK_E_SESSION;
      stored.push_back(Rec{pos, j, id});
    }
    return pos > target ? TOK_E_SESSION : TOK_OK;  // the IDs must cover the stored text
  };

  std::vector<int32_t> fresh;
  uint64_t w = ctx->repair_window;
  for (uint32_t widen = 0; widen <= ctx->repair_doublings; ++widen, w *= 2) {
    inf.widenings = widen;
    const uint64_t ws = back_code_points(text, old_len, w);
    if (ws == 0) break;  // the window would be the whole text
    int rc = walk_to(ws);
    if (rc) return rc;
    const uint64_t wlen = new_len - ws;
    fresh.resize(wlen);
    size_t nf = 0;
    rc = tok_encode(ctx, text + ws, wlen, fresh.data(), wlen, &nf);
    if (rc) return rc;
    const uint64_t margin = fwd_code_points(text, ws, new_len, ctx->repair_margin);

    // match stored records (offset >= ws) against the window's records
    size_t si = stored.size();  // stored[si - 1] is the first stored record at or after ws
    while (si > 0 && stored[si - 1].off < ws) --si;
    uint64_t fo = ws;  // offset of fresh[k]
    size_t k = 0;
    bool found = false;
    size_t keep_s = 0, keep_f = 0;
    uint64_t splice = 0;
    while (si > 0 && k < nf) {
      const Rec& s = stored[si - 1];
      if (s.off < fo) {
        --si;
        continue;
      }
      if (fo < s.off) {
        fo += token_len(fresh[k++]);
        continue;
      }
      if (s.id != fresh[k]) {
        --si;
        fo += token_len(fresh[k++]);
        continue;
      }
      // an equal run starts here; extend it
      const uint64_t r0 = s.off;
      uint64_t r1 = r0;
      size_t m = 0;
      bool certified = false;
      size_t last_s = 0, last_f = 0;
      while (si > 0 && k < nf && stored[si - 1].off == fo && stored[si - 1].id == fresh[k]) {
        const uint64_t b = fo;
        if (b >= margin && b < old_len &&
            sync_transition(ctx->pattern, cp_at(text, new_len, prev_lead(text, b)), cp_at(text, new_len, b)) &&
            !inside_literal(b))
          certified = true;
        last_s = stored[si - 1].idx;
        last_f = k;
        r1 = fo + token_len(fresh[k]);
        fo = r1;
        ++k;
        --si;
        ++m;
      }
      const bool gates = m >= 2 && r1 - r0 > longest;
      if (certified && gates) {  // keep the last certified run
        found = true;
        keep_s = last_s + 1;
        keep_f = last_f + 1;
        splice = r1;
      }
    }
    if (!found) continue;
    const size_t total = keep_s + (nf - keep_f);
    *n_out = total;
    inf.window_start = ws;
    inf.splice_byte = splice;
    inf.kept = keep_s;
    if (total > cap) return TOK_E_CAPACITY;
    std::memcpy(session_ids + keep_s, fresh.data() + keep_f, (nf - keep_f) * sizeof(int32_t));
    return TOK_OK;
  }

  // no certified splice: encode the whole text
  inf.full = 1;
  return tok_encode(ctx, text, new_len, session_ids, cap, n_out);
}

int tok_repair_dev(tok_ctx* ctx, int32_t* d_session_ids, size_t n_session, size_t cap, const uint8_t* text,
                   size_t old_len, size_t new_len, size_t* n_out, tok_repair_info* info) {
  if (!ctx || !n_out || (!text && new_len) || (!d_session_ids && (cap || n_session)) || old_len > new_len ||
      n_session > cap)
    return TOK_E_ARG;
  *n_out = 0;
  tok_repair_info scratch{};
  tok_repair_info& inf = info ? *info : scratch;
  inf = tok_repair_info{};
  if (new_len > TOK_MAX_BYTES) return TOK_E_TOOLONG;
  if ((old_len == 0) != (n_session == 0)) return TOK_E_SESSION;
  if (new_len == old_len) {
    *n_out = n_session;
    inf.kept = n_session;
    inf.splice_byte = old_len;
    return TOK_OK;
  }
  DeviceGuard g(ctx->device);
  hipStream_t s = ctx->stream;
  volatile Counters* c = ctx->h_ctr;
  if (!ctx->n_lit || !ctx->lit_ids_clash) {
    int rc = ctx->ensure_tok_bytes();
    if (rc) return rc;
    // the window reaches back the longest token or literal before its start
    // (the straddling stored token, the literal cut guard), word-aligned
    const uint32_t longest = std::max(ctx->max_tok_len, ctx->n_lit ? ctx->lit_max_len : 0u);
    const uint64_t pad = (longest + 3u) & ~3ull;
    uint64_t w = ctx->repair_window;
    for (uint32_t widen = 0; widen <= ctx->repair_doublings; ++widen, w *= 2) {
      inf.widenings = widen;
      const uint64_t ws = back_code_points(text, old_len, w);
      if (ws == 0) break;  // the window would be the whole text
      const uint64_t ws0 = ws > pad ? ws - pad : 0;
      const uint64_t margin = fwd_code_points(text, ws, new_len, ctx->repair_margin);
      const uint64_t wlen = new_len - ws;
      rc = ctx->ensure(new_len - ws0);
      if (!rc) rc = ctx->ensure_host();
      if (!rc) rc = ctx->ensure_spans();
      if (rc) return rc;
      std::memcpy(ctx->h_text, text + ws0, new_len - ws0);
      HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, new_len - ws0, hipMemcpyHostToDevice, s));
      const uint64_t call = ++ctx->gen;
      if (ctx->n_lit) {
        rc = ctx->ensure_lit_bufs(1);
        if (rc) return rc;
        ctx->enqueue_added(ctx->d_text + (ws - ws0), wlen, nullptr, 0, ctx->d_ids, wlen, nullptr, s, call,
                           ctx->d_spans);
      } else {
        Bufs bb = ctx->b;
        bb.gen = call;
        ctx->enqueue(ctx->d_text + (ws - ws0), wlen, nullptr, 0, ctx->d_ids, ctx->d_spans, wlen, nullptr, s, bb,
                     true, nullptr);
      }
      RepairArgs a{};
      a.win = ctx->d_text;
      a.ws0 = ws0;
      a.ws = ws;
      a.margin = margin;
      a.old_len = old_len;
      a.new_len = new_len;
      a.fresh = ctx->d_ids;
      a.fspan = ctx->d_spans;
      a.fresh_total = &ctx->d_ctr->total;
      a.session = d_session_ids;
      a.n_session = n_session;
      a.cap = cap;
      a.tok_len = ctx->d_tok_len;
      a.tok_bytes = ctx->d_tok_bytes;
      a.tok_off = ctx->d_tok_off;
      a.vocab = (uint32_t)ctx->tok_len.size();
      a.max_tok_len = longest;
      a.L = ctx->literals();
      a.pattern = ctx->pattern;
      // free once the window encode is done: 6 words of splice parameters,
      // then the stored offsets (at most one per window byte; the buffer
      // holds the capacity plus 64 words)
      a.splice = (uint64_t*)ctx->b.ws_rk;
      a.st_off = ctx->b.ws_rk + 6;
      a.max_fresh = new_len - ws;
      a.out = &ctx->d_ctr->rp;
      a.err_utf8 = &ctx->d_ctr->err_utf8;
      a.err_docs = &ctx->d_ctr->err_docs;
      a.gen = call;
      launch_repair_match(a, s);
      HIP_OK(hipGetLastError());
      HIP_OK(hipStreamSynchronize(s));
      if (c->rp.gen != call) return TOK_E_DEVICE;
      const uint32_t st = c->rp.status;
      if (c->err_utf8 == call) return TOK_E_UTF8;  // the match kernel wrote nothing (kRepairEncodeError)
      if (c->err_docs == call || st == kRepairEncodeError) return TOK_E_DEVICE;
      if (c->done != call || (ctx->n_lit && c->ins_done != call)) return TOK_E_DEVICE;
      if (st == kRepairSession) return TOK_E_SESSION;
      if (st == kRepairNone) continue;
      *n_out = c->rp.total;
      inf.window_start = ws;
      inf.splice_byte = c->rp.splice;
      inf.kept = c->rp.kept;
      return st == kRepairSpliced ? TOK_OK : TOK_E_CAPACITY;
    }
  }
  // no certified splice (or literals set): encode the whole text, then
  // replace the session if it fits
  inf.full = 1;
  int rc = ctx->ensure(new_len);
  if (!rc) rc = ctx->ensure_host();
  if (rc) return rc;
  std::memcpy(ctx->h_text, text, new_len);
  HIP_OK(hipMemcpyAsync(ctx->d_text, ctx->h_text, new_len, hipMemcpyHostToDevice, s));
  uint32_t total = 0;
  rc = ctx->n_lit ? ctx->run_added(ctx->d_text, new_len, nullptr, 0, ctx->d_ids, new_len, nullptr, s, &total)
                  : ctx->run(ctx->d_text, new_len, nullptr, 0, ctx->d_ids, nullptr, new_len, nullptr, s, true, nullptr,
                             &total);
  if (rc) return rc;
  *n_out = total;
  if (total > cap) return TOK_E_CAPACITY;
  HIP_OK(hipMemcpyAsync(d_session_ids, ctx->d_ids, (size_t)total * 4, hipMemcpyDeviceToDevice, s));
  HIP_OK(hipStreamSynchronize(s));
  return TOK_OK;
}

}  // extern "C"
