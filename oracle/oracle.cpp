// CPU oracle for exact byte-level BPE encoding.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may load this library.  It shares no code, no
// header and no table with the GPU library; it is plain, scalar,
// single-threaded and deliberately slow, so that each step can be checked by
// eye against its definition:
//
//   encode(x) = concatenation, over the pieces p of pretok(x) in order, of
//               bpe(bytes(p))
//
// (TokTier, Appendix A, Definition A.2 and Lemma A.3: the front end yields
// ordered pieces, the model stage encodes each piece on its own and the IDs
// concatenate; GraphTok, section 3, "Exactness requires the complete ordered
// token sequence").
//
//   C-1 decode UTF-8, rejecting malformed input;
//   C-2 classify code points (L letter, N number, W whitespace, O other)
//       with the frozen table in unicode_classes.inc (and, for the
//       case-splitting family, letters by case and marks from
//       unicode_subclasses.inc);
//   C-3 pre-tokenize with a direct leftmost-first matcher that tries the
//       pattern's alternatives in order at a cursor and moves the cursor to the
//       end of the first match (TokTier, section 4, "Removing the sequential
//       regex scan": each match begins where the previous one ended);
//   C-4 textbook BPE per piece: start from the piece's bytes (IDs 0..255);
//       while some adjacent pair has a merge rank, merge the leftmost
//       occurrence of the lowest-rank pair into ID 256 + rank (GraphTok,
//       section 3, "BPE is parallel across pre-tokens but ordered within
//       them"; section 4, lowest rank wins, leftmost on equal rank);
//   C-5 concatenate.
//
// Readings where the pages leave a step open: merge ranks are keyed by the
// ordered ID pair; byte b has ID b and merge r creates ID 256 + r; the
// contraction apostrophe is U+0027 only; "newline" in the Llama-3 style means
// CR or LF only; whitespace lookahead succeeds at the end of the text.
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "unicode_classes.inc"
#include "unicode_subclasses.inc"

namespace {

enum { CL = 0, CN = 1, CW = 2, CO = 3 };
enum { PAT_GPT2 = 0, PAT_LLAMA3 = 1, PAT_O200K = 2 };
// letters by case and marks (the case-splitting family): U = Lu or Lt,
// D = Ll, C = Lm or Lo, M = marks; SN / SW / SO: numbers, whitespace, others
enum { SU = 0, SD = 1, SC = 2, SM = 3, SN = 4, SW = 5, SO = 6 };
enum { ORC_OK = 0, ORC_UTF8 = 1, ORC_CAP = 2, ORC_ARG = 3 };

// ---------------------------------------------------------------- C-2 classes
int class_of(uint32_t cp) {
  size_t lo = 0, hi = kOrcNumRanges;
  while (lo < hi) {  // first range with hi >= cp
    size_t mid = (lo + hi) / 2;
    if (kOrcRanges[mid][1] < cp) lo = mid + 1;
    else hi = mid;
  }
  if (lo < kOrcNumRanges && kOrcRanges[lo][0] <= cp && cp <= kOrcRanges[lo][1])
    return int(kOrcRanges[lo][2]);
  return CO;
}

int subclass_of(uint32_t cp) {
  size_t lo = 0, hi = kOrcNumSubRanges;
  while (lo < hi) {
    size_t mid = (lo + hi) / 2;
    if (kOrcSubRanges[mid][1] < cp) lo = mid + 1;
    else hi = mid;
  }
  if (lo < kOrcNumSubRanges && kOrcSubRanges[lo][0] <= cp && cp <= kOrcSubRanges[lo][1])
    return int(kOrcSubRanges[lo][2]);
  const int c = class_of(cp);
  return c == CN ? SN : c == CW ? SW : SO;  // a letter always has a case class above
}

// case-insensitive equality with an ASCII lowercase letter
bool fold_eq(uint32_t cp, char letter) {
  for (size_t i = 0; i < kOrcNumFold; ++i)
    if (kOrcFold[i][0] == uint32_t(letter) && kOrcFold[i][1] == cp) return true;
  return false;
}

// ---------------------------------------------------------------- C-1 decode
// Well-formed UTF-8 (Unicode Table 3-7): no overlongs, no surrogates, nothing
// above U+10FFFF, no truncated sequences.
bool decode_utf8(const uint8_t* s, size_t n, std::vector<uint32_t>& cps,
                 std::vector<size_t>& offs) {
  size_t i = 0;
  while (i < n) {
    uint8_t b0 = s[i];
    uint32_t cp;
    size_t len;
    if (b0 < 0x80) {
      cp = b0;
      len = 1;
    } else if (b0 >= 0xC2 && b0 <= 0xDF) {
      len = 2;
      cp = b0 & 0x1F;
    } else if (b0 >= 0xE0 && b0 <= 0xEF) {
      len = 3;
      cp = b0 & 0x0F;
    } else if (b0 >= 0xF0 && b0 <= 0xF4) {
      len = 4;
      cp = b0 & 0x07;
    } else {
      return false;
    }
    if (i + len > n) return false;
    for (size_t k = 1; k < len; ++k) {
      uint8_t b = s[i + k];
      if ((b & 0xC0) != 0x80) return false;
      cp = (cp << 6) | (b & 0x3F);
    }
    if (len == 3 && (cp < 0x800 || (cp >= 0xD800 && cp <= 0xDFFF))) return false;
    if (len == 4 && (cp < 0x10000 || cp > 0x10FFFF)) return false;
    cps.push_back(cp);
    offs.push_back(i);
    i += len;
  }
  offs.push_back(n);
  return true;
}

// ---------------------------------------------------------------- C-3 matcher
struct Text {
  std::vector<uint32_t> cp;
  std::vector<int> cls;
  std::vector<int> sub;  // subclass_of, for the case-splitting family only
  size_t n() const { return cp.size(); }
};

size_t run_of(const Text& t, size_t p, int c) {  // end of the maximal class-c run from p
  while (p < t.n() && t.cls[p] == c) ++p;
  return p;
}

bool is_crlf(uint32_t c) { return c == 0x0D || c == 0x0A; }

const char* const kContractions[] = {"s", "t", "re", "ve", "m", "ll", "d"};

// 's|'t|'re|'ve|'m|'ll|'d, case-sensitive or case-insensitive
size_t match_contraction(const Text& t, size_t p, bool fold) {
  if (t.cp[p] != 0x27) return 0;
  for (const char* c : kContractions) {
    size_t k = strlen(c);
    if (p + 1 + k > t.n()) continue;
    bool ok = true;
    for (size_t j = 0; j < k && ok; ++j) {
      uint32_t x = t.cp[p + 1 + j];
      ok = fold ? fold_eq(x, c[j]) : (x == uint32_t(c[j]));
    }
    if (ok) return p + 1 + k;
  }
  return 0;
}

// " ?X+" for a class X: greedy optional U+0020, then a maximal X-run
size_t match_space_run(const Text& t, size_t p, int x) {
  if (t.cp[p] == 0x20 && p + 1 < t.n() && t.cls[p + 1] == x) return run_of(t, p + 1, x);
  if (t.cls[p] == x) return run_of(t, p, x);
  return 0;
}

// "\s+(?!\S)": greedy whitespace, backtracking until the next char is not
// non-whitespace (end of text counts as "not followed by non-whitespace")
size_t match_ws_lookahead(const Text& t, size_t p) {
  if (t.cls[p] != CW) return 0;
  size_t e = run_of(t, p, CW);
  for (size_t q = e; q >= p + 1; --q)
    if (q == t.n() || t.cls[q] == CW) return q;
  return 0;
}

// "\s+"
size_t match_ws(const Text& t, size_t p) { return t.cls[p] == CW ? run_of(t, p, CW) : 0; }

// GPT-2 style:
//   's|'t|'re|'ve|'m|'ll|'d | ?\p{L}+ | ?\p{N}+ | ?[^\s\p{L}\p{N}]+ | \s+(?!\S) | \s+
size_t gpt2_next(const Text& t, size_t p) {
  size_t q;
  if ((q = match_contraction(t, p, false))) return q;
  if ((q = match_space_run(t, p, CL))) return q;
  if ((q = match_space_run(t, p, CN))) return q;
  if ((q = match_space_run(t, p, CO))) return q;
  if ((q = match_ws_lookahead(t, p))) return q;
  if ((q = match_ws(t, p))) return q;
  return 0;
}

// Llama-3 style:
//   (?i:'s|'t|'re|'ve|'m|'ll|'d) | [^\r\n\p{L}\p{N}]?\p{L}+ | \p{N}{1,3}
//   | ?[^\s\p{L}\p{N}]+[\r\n]* | \s*[\r\n]+ | \s+(?!\S) | \s+
size_t llama3_next(const Text& t, size_t p) {
  const size_t n = t.n();
  size_t q;
  if ((q = match_contraction(t, p, true))) return q;
  // [^\r\n\p{L}\p{N}]?\p{L}+
  {
    bool pre = !is_crlf(t.cp[p]) && t.cls[p] != CL && t.cls[p] != CN;
    if (pre && p + 1 < n && t.cls[p + 1] == CL) return run_of(t, p + 1, CL);
    if (t.cls[p] == CL) return run_of(t, p, CL);
  }
  // \p{N}{1,3}
  if (t.cls[p] == CN) {
    q = p;
    while (q < n && q < p + 3 && t.cls[q] == CN) ++q;
    return q;
  }
  // " ?[^\s\p{L}\p{N}]+[\r\n]*"
  if ((q = match_space_run(t, p, CO))) {
    while (q < n && is_crlf(t.cp[q])) ++q;
    return q;
  }
  // \s*[\r\n]+ : greedy \s*, backtracking until [\r\n]+ can match
  if (t.cls[p] == CW) {
    size_t e = run_of(t, p, CW);
    for (size_t k = e + 1; k-- > p;) {
      if (k < n && is_crlf(t.cp[k])) {
        q = k;
        while (q < n && is_crlf(t.cp[q])) ++q;
        return q;
      }
    }
  }
  if ((q = match_ws_lookahead(t, p))) return q;
  if ((q = match_ws(t, p))) return q;
  return 0;
}

// Case-splitting (o200k-style) family, as read from TokTier, section 4
// "Removing the sequential regex scan": the Llama-3-style alternatives, with
// the letter alternative split at case boundaries, marks joining letters,
// and the contractions moved to an optional suffix of a letter piece:
//   P? H* T+ S? | P? H+ T* S? | N{1,3} | " "?[^\s L N]+[\r\n]* | \s*[\r\n]+
//   | \s+(?!\S) | \s+
// with H = U|C|M (upper, caseless, marks), T = D|C|M (lower, caseless,
// marks), P = one char that is not CR, LF, a letter or a number, and S =
// (?i:'s|'t|'re|'ve|'m|'ll|'d).  Each alternative is matched as a
// backtracking engine would: the optional prefix is tried first taken, then
// not; H* gives back one char at a time until T+ can start.
bool in_h(int k) { return k == SU || k == SC || k == SM; }
bool in_t(int k) { return k == SD || k == SC || k == SM; }
bool in_p(const Text& t, size_t i) { return !is_crlf(t.cp[i]) && t.cls[i] != CL && t.cls[i] != CN; }

// optional contraction suffix at q (case-insensitive), greedy
size_t contraction_suffix(const Text& t, size_t q) {
  if (q < t.n()) {
    size_t e = match_contraction(t, q, true);
    if (e) return e;
  }
  return q;
}

// P? H* T+ S? from cursor p; 0 if it does not match
size_t match_split_lower(const Text& t, size_t p) {
  const size_t n = t.n();
  for (int pre = 1; pre >= 0; --pre) {
    if (pre && !in_p(t, p)) continue;
    const size_t q = p + pre;
    size_t h = q;
    while (h < n && in_h(t.sub[h])) ++h;
    for (size_t x = h + 1; x-- > q;) {  // H* takes [q, x); T+ starts at x
      if (x < n && in_t(t.sub[x])) {
        size_t e = x;
        while (e < n && in_t(t.sub[e])) ++e;
        return contraction_suffix(t, e);
      }
    }
  }
  return 0;
}

// P? H+ T* S? from cursor p; 0 if it does not match
size_t match_split_upper(const Text& t, size_t p) {
  const size_t n = t.n();
  for (int pre = 1; pre >= 0; --pre) {
    if (pre && !in_p(t, p)) continue;
    const size_t q = p + pre;
    if (q >= n || !in_h(t.sub[q])) continue;
    size_t h = q;
    while (h < n && in_h(t.sub[h])) ++h;
    size_t e = h;
    while (e < n && in_t(t.sub[e])) ++e;
    return contraction_suffix(t, e);
  }
  return 0;
}

size_t o200k_next(const Text& t, size_t p) {
  const size_t n = t.n();
  size_t q;
  if ((q = match_split_lower(t, p))) return q;
  if ((q = match_split_upper(t, p))) return q;
  // \p{N}{1,3}
  if (t.cls[p] == CN) {
    q = p;
    while (q < n && q < p + 3 && t.cls[q] == CN) ++q;
    return q;
  }
  // " ?[^\s\p{L}\p{N}]+[\r\n]*": marks are not letters, so they count here
  if ((q = match_space_run(t, p, CO))) {
    while (q < n && is_crlf(t.cp[q])) ++q;
    return q;
  }
  // \s*[\r\n]+
  if (t.cls[p] == CW) {
    size_t e = run_of(t, p, CW);
    for (size_t k = e + 1; k-- > p;) {
      if (k < n && is_crlf(t.cp[k])) {
        q = k;
        while (q < n && is_crlf(t.cp[q])) ++q;
        return q;
      }
    }
  }
  if ((q = match_ws_lookahead(t, p))) return q;
  if ((q = match_ws(t, p))) return q;
  return 0;
}

// Pieces as code-point index boundaries [b_0=0, b_1, ..., b_m = n].
std::vector<size_t> pretokenize(const Text& t, int pattern) {
  std::vector<size_t> starts;
  size_t p = 0;
  while (p < t.n()) {
    starts.push_back(p);
    size_t q = pattern == PAT_GPT2 ? gpt2_next(t, p) : pattern == PAT_LLAMA3 ? llama3_next(t, p) : o200k_next(t, p);
    if (q <= p) q = p + 1;  // unreachable: every class has an alternative
    p = q;
  }
  return starts;
}

// C-2 for a decoded text: classes, and for the case-splitting family the
// letter-case and mark subclasses
void classify(Text& t, int pattern) {
  t.cls.resize(t.cp.size());
  for (size_t i = 0; i < t.cp.size(); ++i) t.cls[i] = class_of(t.cp[i]);
  if (pattern == PAT_O200K) {
    t.sub.resize(t.cp.size());
    for (size_t i = 0; i < t.cp.size(); ++i) t.sub[i] = subclass_of(t.cp[i]);
  }
}

// ---------------------------------------------------------------- C-4 BPE
struct Oracle {
  int pattern;
  std::map<std::pair<uint32_t, uint32_t>, uint32_t> rank;  // (left, right) -> rank
};

// Textbook BPE of one piece.  at, when given, receives the byte offset within
// the piece where each output token starts: a merged token starts where its
// left operand did (the span export of TokTier, section 7: per-token byte
// offsets next to the IDs).
void bpe(const Oracle& o, const uint8_t* b, size_t n, std::vector<int32_t>& out,
         std::vector<size_t>* at = nullptr) {
  std::vector<uint32_t> sym(b, b + n);
  std::vector<size_t> start(n);
  for (size_t i = 0; i < n; ++i) start[i] = i;
  for (;;) {
    size_t best_j = 0;
    uint32_t best_r = UINT32_MAX;
    for (size_t j = 0; j + 1 < sym.size(); ++j) {
      auto it = o.rank.find({sym[j], sym[j + 1]});
      if (it != o.rank.end() && it->second < best_r) {  // strict: leftmost wins ties
        best_r = it->second;
        best_j = j;
      }
    }
    if (best_r == UINT32_MAX) break;
    sym[best_j] = 256u + best_r;
    sym.erase(sym.begin() + long(best_j) + 1);
    start.erase(start.begin() + long(best_j) + 1);
  }
  for (uint32_t s : sym) out.push_back(int32_t(s));
  if (at) at->insert(at->end(), start.begin(), start.end());
}

// spans, when given, receives each token's first byte, counted from s.
int encode_one(const Oracle& o, const uint8_t* s, size_t n, std::vector<int32_t>& out,
               std::vector<uint64_t>* spans = nullptr) {
  Text t;
  std::vector<size_t> offs;
  if (!decode_utf8(s, n, t.cp, offs)) return ORC_UTF8;
  classify(t, o.pattern);
  std::vector<size_t> st = pretokenize(t, o.pattern);
  std::vector<size_t> at;
  for (size_t k = 0; k < st.size(); ++k) {
    size_t a = offs[st[k]];
    size_t e = offs[k + 1 < st.size() ? st[k + 1] : t.cp.size()];
    at.clear();
    bpe(o, s + a, e - a, out, spans ? &at : nullptr);
    if (spans)
      for (size_t x : at) spans->push_back(a + x);
  }
  return ORC_OK;
}

}  // namespace

extern "C" {

int orc_class(uint32_t cp) { return class_of(cp); }

// Classes of the code points lo .. lo + n - 1, one byte each.
void orc_class_range(uint32_t lo, uint32_t n, uint8_t* out) {
  for (uint32_t i = 0; i < n; ++i) out[i] = uint8_t(class_of(lo + i));
}

// Subclasses (U=0 D=1 C=2 M=3 N=4 W=5 O=6) of the code points lo .. lo + n - 1.
void orc_subclass_range(uint32_t lo, uint32_t n, uint8_t* out) {
  for (uint32_t i = 0; i < n; ++i) out[i] = uint8_t(subclass_of(lo + i));
}

// merges: n x (left, right); operands must precede their merge; pairs unique.
void* orc_new(const uint32_t* merges, size_t n, int pattern, int* err) {
  *err = ORC_ARG;
  if (pattern != PAT_GPT2 && pattern != PAT_LLAMA3 && pattern != PAT_O200K) return nullptr;
  Oracle* o = new Oracle();
  o->pattern = pattern;
  for (size_t r = 0; r < n; ++r) {
    uint32_t a = merges[2 * r], b = merges[2 * r + 1];
    if (a >= 256 + r || b >= 256 + r || o->rank.count({a, b})) {
      delete o;
      return nullptr;
    }
    o->rank[{a, b}] = uint32_t(r);
  }
  *err = ORC_OK;
  return o;
}

void orc_free(void* h) { delete static_cast<Oracle*>(h); }

// Piece start byte offsets.
int orc_pieces(void* h, const uint8_t* text, size_t len, uint64_t* starts, size_t cap, size_t* n_out) {
  const Oracle& o = *static_cast<Oracle*>(h);
  Text t;
  std::vector<size_t> offs;
  *n_out = 0;
  if (!decode_utf8(text, len, t.cp, offs)) return ORC_UTF8;
  classify(t, o.pattern);
  std::vector<size_t> st = pretokenize(t, o.pattern);
  *n_out = st.size();
  if (st.size() > cap) return ORC_CAP;
  for (size_t k = 0; k < st.size(); ++k) starts[k] = offs[st[k]];
  return ORC_OK;
}

// BPE of one piece given as raw bytes (no pre-tokenization).
int orc_bpe(void* h, const uint8_t* bytes, size_t len, int32_t* ids, size_t cap, size_t* n_out) {
  std::vector<int32_t> out;
  bpe(*static_cast<Oracle*>(h), bytes, len, out);
  *n_out = out.size();
  if (out.size() > cap) return ORC_CAP;
  if (!out.empty()) memcpy(ids, out.data(), out.size() * 4);
  return ORC_OK;
}

int orc_encode(void* h, const uint8_t* text, size_t len, int32_t* ids, size_t cap, size_t* n_out) {
  std::vector<int32_t> out;
  *n_out = 0;
  int rc = encode_one(*static_cast<Oracle*>(h), text, len, out);
  if (rc) return rc;
  *n_out = out.size();
  if (out.size() > cap) return ORC_CAP;
  if (!out.empty()) memcpy(ids, out.data(), out.size() * 4);
  return ORC_OK;
}

// Each document [doc_off[i], doc_off[i+1]) is encoded on its own.  spans
// (optional, cap entries): each token's first byte in text.
int orc_encode_batch_spans(void* h, const uint8_t* text, const uint64_t* doc_off, size_t n_docs,
                           int32_t* ids, uint64_t* spans, size_t cap, uint64_t* out_off) {
  std::vector<int32_t> out;
  std::vector<uint64_t> sp;
  out_off[0] = 0;
  for (size_t d = 0; d < n_docs; ++d) {
    if (doc_off[d + 1] < doc_off[d]) return ORC_ARG;
    const size_t before = sp.size();
    int rc = encode_one(*static_cast<Oracle*>(h), text + doc_off[d], doc_off[d + 1] - doc_off[d], out,
                        spans ? &sp : nullptr);
    if (rc) return rc;
    for (size_t k = before; k < sp.size(); ++k) sp[k] += doc_off[d];
    out_off[d + 1] = out.size();
  }
  if (out.size() > cap) return ORC_CAP;
  if (!out.empty()) memcpy(ids, out.data(), out.size() * 4);
  if (spans && !sp.empty()) memcpy(spans, sp.data(), sp.size() * 8);
  return ORC_OK;
}

int orc_encode_batch(void* h, const uint8_t* text, const uint64_t* doc_off, size_t n_docs,
                     int32_t* ids, size_t cap, uint64_t* out_off) {
  return orc_encode_batch_spans(h, text, doc_off, n_docs, ids, nullptr, cap, out_off);
}

// Added-token literals (TokTier, section 4 "Single-request path": a
// leftmost-longest literal pass extracts the added tokens before the
// tokenizer family handles the remaining segments; GraphTok, section 4
// "Design": added entries take precedence over pre-tokenization and only the
// unmatched regions reach it).  Literal i is lit[lit_off[i] .. lit_off[i+1])
// with ID lit_id[i].  A cursor walks the text byte by byte: where one or more
// literals match, the longest is taken, its ID emitted and the cursor moved
// past it; the text between two taken literals is one segment, encoded on its
// own by encode_one.  Malformed UTF-8 anywhere rejects the whole text.
int orc_encode_added(void* h, const uint8_t* lit, const uint64_t* lit_off, size_t n_lit, const int32_t* lit_id,
                     const uint8_t* text, size_t len, int32_t* ids, size_t cap, size_t* n_out) {
  const Oracle& o = *static_cast<Oracle*>(h);
  *n_out = 0;
  {
    Text t;
    std::vector<size_t> offs;
    if (!decode_utf8(text, len, t.cp, offs)) return ORC_UTF8;
  }
  std::vector<int32_t> out;
  size_t seg = 0, p = 0;
  while (p < len) {
    size_t best_len = 0;
    int32_t best_id = 0;
    for (size_t i = 0; i < n_lit; ++i) {
      const size_t L = lit_off[i + 1] - lit_off[i];
      if (L > best_len && p + L <= len && memcmp(text + p, lit + lit_off[i], L) == 0) {
        best_len = L;
        best_id = lit_id[i];
      }
    }
    if (best_len == 0) {
      ++p;
      continue;
    }
    int rc = encode_one(o, text + seg, p - seg, out);
    if (rc) return rc;
    out.push_back(best_id);
    p += best_len;
    seg = p;
  }
  int rc = encode_one(o, text + seg, len - seg, out);
  if (rc) return rc;
  *n_out = out.size();
  if (out.size() > cap) return ORC_CAP;
  if (!out.empty()) memcpy(ids, out.data(), out.size() * 4);
  return ORC_OK;
}

}  // extern "C"
