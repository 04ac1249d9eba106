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
#include <cstddef>
#include <cstdint>
#include <vector>

#define TOK_HD
#define TOK_CLS_QUAL
#include "pretok_rules.h"
#include "uniclass.inc"

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

}  // namespace

extern "C" int rules_cpu_class(uint32_t cp) { return (int)table_class(cp); }

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
