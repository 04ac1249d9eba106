// CPU build of the pre-tokenization rules in pretok_rules.h, for the tests.
//
// The kernel evaluates piece_start_* per code point with run aggregates that
// come from wave/workgroup scans; here the same rule functions and the same
// scan elements run sequentially over a whole text, so the tests can check the
// rules and the scan algebra against the oracle's direct matcher on the CPU.
// Not part of the tokenizer: the library never calls it.
//
// Built with g++ (no HIP): TOK_CLS_QUAL is empty, so the class table compiles
// as ordinary constant arrays.
#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <vector>

#define TOK_HD
#define TOK_CLS_QUAL
#include "pretok_rules.h"
#include "seg_rules.h"
#include "uniclass.inc"
#include "uniclass_case.inc"

namespace {

using namespace tok;

uint32_t table_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
  if (cp < TOK_CLS_LOW) return (kClsLow[cp >> 2] >> (2 * (cp & 3u))) & 3u;
  const uint32_t blk = kClsBlock[cp >> 8];
  return (kClsBits[blk * 64 + ((cp & 255u) >> 2)] >> (2 * (cp & 3u))) & 3u;
}

uint32_t fold_extra(uint32_t cp) {
  for (int i = 0; i < TOK_NFOLD_EXTRA; ++i)
    if (kFoldExtra[i][0] == cp) return ascii_letter_code(kFoldExtra[i][1]);
  return 0;
}

uint32_t table_case(uint32_t cp) {
  if (cp < TOK_CLS_LOW) return (kCaseLow[cp >> 1] >> (4 * (cp & 1u))) & 15u;
  const uint32_t blk = kCaseBlock[cp >> 8];
  return (kCaseBits[blk * 128 + ((cp & 255u) >> 1)] >> (4 * (cp & 1u))) & 15u;
}

// Byte-indexed text for the segment matcher: info words at code point starts.
struct HostAcc {
  const std::vector<uint32_t>* q;
  size_t n;
  uint32_t at(uint64_t i) const { return i >= n ? (uint32_t)seg::kQEnd : (*q)[i]; }
};

// The case-splitting family the way the kernel does it: 1 KiB tiles; in each
// tile, segments from the last synchronizing cut at or before its first code
// point and from every cut inside it, each matched from its cut until the
// cursor reaches another cut or the tile's end.
int case_pieces(const uint8_t* s, size_t n, const std::vector<char>& docstart, std::vector<uint64_t>& out) {
  std::vector<uint32_t> q(n, 0);
  std::vector<uint64_t> leads;
  for (size_t i = 0; i < n;) {
    const uint8_t b = s[i];
    const uint32_t len = b < 0x80 ? 1 : b >= 0xF0 ? 4 : b >= 0xE0 ? 3 : 2;
    if ((b & 0xC0) == 0x80 || i + len > n) return 1;
    uint32_t cp = len == 1 ? b : len == 2 ? (b & 0x1Fu) : len == 3 ? (b & 0x0Fu) : (b & 0x07u);
    for (uint32_t k = 1; k < len; ++k) cp = (cp << 6) | (s[i + k] & 0x3Fu);
    q[i] = seg::make_q(cp, table_case(cp), len, seg::fold_code(cp, fold_extra(cp)));
    if (docstart[i]) q[i] |= seg::kQDocStart;
    leads.push_back(i);
    i += len;
  }
  std::vector<char> cut(n, 0);
  for (size_t k = 0; k < leads.size(); ++k) {
    const uint64_t j = leads[k];
    cut[j] = k == 0 || docstart[j] || seg::sync_at(q[leads[k - 1]], q[j]);
  }
  HostAcc acc{&q, n};
  std::vector<char> start(n, 0);
  constexpr size_t kTile = 1024;
  for (size_t t0 = 0; t0 < n; t0 += kTile) {
    const size_t t1 = std::min(n, t0 + kTile);
    size_t first = t0;
    while (first < t1 && !(q[first] & seg::kQLead)) ++first;
    if (first == t1) continue;
    size_t a0 = first;
    while (!cut[a0]) {
      --a0;
      while (!(q[a0] & seg::kQLead)) --a0;
    }
    std::vector<size_t> segs{a0};
    for (size_t j = first + 1; j < t1; ++j)
      if ((q[j] & seg::kQLead) && cut[j]) segs.push_back(j);
    for (size_t a : segs) {
      uint64_t p = a;
      for (;;) {
        if (p >= t0) start[p] = 1;
        seg::Matcher<HostAcc> m{acc, p};
        const uint64_t e = m.piece_end();
        if (e <= p) return 2;  // no progress: a matcher bug
        p = e;
        if (p >= t1 || cut[p]) break;
      }
    }
  }
  for (size_t i = 0; i < n; ++i)
    if (start[i]) out.push_back(i);
  return 0;
}

}  // namespace

extern "C" int rules_cpu_class(uint32_t cp) { return (int)table_class(cp); }

// Letter-case classes (U=0 D=1 C=2 M=3 N=4 W=5 O=6) of lo .. lo + n - 1.
extern "C" void rules_cpu_case_range(uint32_t lo, uint32_t n, uint8_t* out) {
  for (uint32_t i = 0; i < n; ++i) out[i] = (uint8_t)table_case(lo + i);
}

// The case-splitting family's synchronizing transition (the library's rule).
extern "C" int rules_cpu_sync_case(uint32_t x, uint32_t y) {
  return tok::sync_transition_case(x, table_case(x), y, table_case(y)) ? 1 : 0;
}

// Classes of the code points lo .. lo + n - 1, one byte each.
extern "C" void rules_cpu_class_range(uint32_t lo, uint32_t n, uint8_t* out) {
  for (uint32_t i = 0; i < n; ++i) out[i] = (uint8_t)table_class(lo + i);
}

// The contraction-letter code of a non-ASCII code point (0: none), from the
// fold table the kernels use.
extern "C" int rules_cpu_fold_extra(uint32_t cp) { return (int)fold_extra(cp); }

// The contraction-letter code of an ASCII lowercase letter (0: not one).
extern "C" int rules_cpu_letter_code(uint32_t cp) { return (int)ascii_letter_code(cp); }

// Piece-start byte offsets of valid UTF-8 text (documents split at doc_off,
// n_docs + 1 offsets, or one document when doc_off is null).  Returns 0, or 1
// on malformed input (this harness only decodes; it does not fully validate).
extern "C" int rules_cpu_pieces(const uint8_t* s, size_t n, const uint64_t* doc_off, size_t n_docs,
                                int pattern, uint64_t* starts, size_t cap, size_t* n_out) {
  std::vector<uint32_t> info;
  std::vector<size_t> pos;
  std::vector<char> docstart(n + 1, 0);
  if (doc_off) {
    for (size_t d = 0; d <= n_docs; ++d)
      if (doc_off[d] <= n) docstart[doc_off[d]] = 1;
  } else {
    docstart[0] = 1;
  }
  docstart[n] = 1;
  if (pattern == 2) {
    std::vector<uint64_t> st;
    const int rc = case_pieces(s, n, docstart, st);
    if (rc) return rc;
    *n_out = st.size();
    for (size_t k = 0; k < st.size() && k < cap; ++k) starts[k] = st[k];
    return 0;
  }
  for (size_t i = 0; i < n;) {
    const uint8_t b = s[i];
    uint32_t len = b < 0x80 ? 1 : b >= 0xF0 ? 4 : b >= 0xE0 ? 3 : 2;
    if ((b & 0xC0) == 0x80 || i + len > n) return 1;
    uint32_t cp = len == 1 ? b : len == 2 ? (b & 0x1Fu) : len == 3 ? (b & 0x0Fu) : (b & 0x07u);
    for (uint32_t k = 1; k < len; ++k) cp = (cp << 6) | (s[i + k] & 0x3Fu);
    uint32_t in = make_info(cp, table_class(cp), len, fold_extra(cp));
    if (docstart[i]) in |= kIDocStart;
    if (docstart[i + len]) in |= kILastInDoc;
    info.push_back(in);
    pos.push_back(i);
    i += len;
  }
  const size_t m = info.size();
  auto at = [&](size_t j, size_t back) -> uint32_t {  // code point back steps before j, same doc
    for (size_t b = 0; b < back; ++b) {
      if (info[j] & kIDocStart) return kNone;
      --j;
    }
    return info[j];
  };
  std::vector<uint32_t> fstate(m), hstate(m);
  uint32_t st = 0;
  for (size_t j = 0; j < m; ++j) {
    fstate[j] = st;
    st = fwd_apply(fwd_elem(info[j]), st);
  }
  uint32_t h = 0;
  for (size_t j = m; j-- > 0;) {
    hstate[j] = h;
    h = bwd_apply(bwd_elem(info[j]), h);
  }
  size_t cnt = 0;
  for (size_t j = 0; j < m; ++j) {
    const uint32_t c = info[j];
    const uint32_t p1 = at(j, 1), p2 = is_none(p1) ? kNone : at(j - 1, 1);
    const uint32_t p3 = is_none(p2) ? kNone : at(j - 2, 1), p4 = is_none(p3) ? kNone : at(j - 3, 1);
    const uint32_t n1 = (c & kILastInDoc) ? kNone : info[j + 1];
    bool start = pattern == 0
                     ? piece_start_gpt2(c, p1, p2, p3, p4, n1)
                     : piece_start_llama3(c, p1, p2, p3, p4, n1, fstate[j] & 3u, (fstate[j] >> 2) & 1u,
                                          hstate[j] & 1u);
    if (start) {
      if (cnt < cap) starts[cnt] = pos[j];
      ++cnt;
    }
  }
  *n_out = cnt;
  return 0;
}

#include "bpe_util.h"

// The round selection of the long-piece merge kernel, exposed for tests.
extern "C" uint64_t rules_cpu_select(uint64_t m, uint32_t carry) { return tok::select_leftmost(m, carry); }
