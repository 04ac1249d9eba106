// Run-local piece-start rules of the two pre-tokenizer families.
//
// The leftmost-first regex of a GPT-family pre-tokenizer advances from one
// match to the next; evaluated per code point it becomes a predicate that
// needs only the classes of a few neighbours plus, for the Llama-3 style,
// three run aggregates (TokTier, "Exact GPU Tokenization", run decomposition
// over four classes with bounded lookback and per-run aggregates; GraphTok,
// section 4 "Parallel tokenizer frontends", a boundary predicate per code
// point plus prefix scans for in-run offsets, with the Llama-3 digit rule:
// a digit starts a piece iff its offset in the digit run is a multiple of 3).
//
// This header holds only per-code-point logic (no memory access), so the same
// functions run in the pre-tokenization kernel and in a CPU build used by the
// tests.  A code point is described by one 32-bit info word (kI* bits); the
// value kNone stands for "no code point here" (before a document's start or
// after its end).
#pragma once

#include <stdint.h>

#ifndef TOK_HD
#define TOK_HD __host__ __device__
#endif

namespace tok {

// info word bits
enum : uint32_t {
  kIClass = 3u,          // bits 0-1: L=0 N=1 W=2 O=3
  kILead = 1u << 2,      // byte begins a code point
  kICrlf = 1u << 3,      // U+000D or U+000A
  kISpace = 1u << 4,     // U+0020
  kIApos = 1u << 5,      // U+0027
  kIDocStart = 1u << 6,  // a document starts at this byte
  kIOutside = 1u << 7,   // byte position outside [0, N)
  kIExactShift = 8,      // bits 8-11: letter code, case-sensitive (s t r e v m l d = 1..8)
  kIFoldShift = 12,      // bits 12-15: letter code under simple case folding
  kIUndecoded = 1u << 16,  // lead whose continuation bytes lie outside the loaded window
  kILenShift = 17,         // bits 17-19: UTF-8 length of the code point
  kILastInDoc = 1u << 20,  // the next code point starts another document (or the text ends)
  kIPrevShift = 21,        // bits 21-23: bytes back to the previous code point of the document (0: none)
};
constexpr uint32_t kNone = 0xFFFFFFFFu;

enum : uint32_t { kCodeS = 1, kCodeT, kCodeR, kCodeE, kCodeV, kCodeM, kCodeL, kCodeD };

TOK_HD inline uint32_t cls_of(uint32_t i) { return i & kIClass; }
TOK_HD inline bool is_none(uint32_t i) { return i == kNone; }
TOK_HD inline bool has(uint32_t i, uint32_t bit) { return i != kNone && (i & bit); }
TOK_HD inline uint32_t exact_code(uint32_t i) { return (i >> kIExactShift) & 15u; }
TOK_HD inline uint32_t fold_code(uint32_t i) { return (i >> kIFoldShift) & 15u; }

// Letter codes of 'a'..'z' as nibbles: letters a..p in kLetterLo, q..z in
// kLetterHi (0 = not a contraction letter).
constexpr uint64_t letter_nibbles(char first, char last) {
  uint64_t v = 0;
  for (char ch = first; ch <= last; ++ch) {
    const uint64_t code = ch == 's' ? kCodeS : ch == 't' ? kCodeT : ch == 'r' ? kCodeR : ch == 'e' ? kCodeE
                        : ch == 'v' ? kCodeV : ch == 'm' ? kCodeM : ch == 'l' ? kCodeL : ch == 'd' ? kCodeD : 0;
    v |= code << (4 * (ch - first));
  }
  return v;
}
constexpr uint64_t kLetterLo = letter_nibbles('a', 'p'), kLetterHi = letter_nibbles('q', 'z');

// Letter code of an ASCII code point, case-sensitive (lowercase only).
TOK_HD inline uint32_t ascii_letter_code(uint32_t cp) {
  const uint32_t t = cp - 'a';
  if (t >= 26u) return 0;
  return (uint32_t)((t < 16u ? kLetterLo >> (4 * t) : kLetterHi >> (4 * (t - 16u))) & 15u);
}

// Class of an ASCII code point: letters L, digits N, TAB..CR and space W.
TOK_HD inline uint32_t ascii_class(uint32_t cp) {
  const bool l = (cp | 0x20u) - 'a' < 26u, d = cp - '0' < 10u, w = cp == ' ' || cp - 9u < 5u;
  return l ? 0u : d ? 1u : w ? 2u : 3u;
}

// Info word of one decoded code point (class from the caller's table).
TOK_HD inline uint32_t make_info(uint32_t cp, uint32_t cls, uint32_t len, uint32_t fold_extra_code) {
  uint32_t i = cls | kILead | (len << kILenShift);
  i |= (cp == 0x0D || cp == 0x0A) ? kICrlf : 0u;
  i |= cp == 0x20 ? kISpace : 0u;
  i |= cp == 0x27 ? kIApos : 0u;
  const bool ascii_letter = cp < 0x80 && (cp | 0x20u) - 'a' < 26u;
  i |= (cp < 0x80 ? ascii_letter_code(cp) : 0u) << kIExactShift;
  i |= (ascii_letter ? ascii_letter_code(cp | 0x20u) : cp < 0x80 ? 0u : fold_extra_code) << kIFoldShift;
  return i;
}

// The predicates below are flat boolean algebra (no early returns), so the
// kernel evaluates them without divergent branches.  kNone has every bit set,
// so each test that can see "no code point" checks for it first.  Bitwise &
// and | on bools are deliberate: they keep both sides evaluated, branch-free.
#if defined(__clang__)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wbitwise-instead-of-logical"
#endif

// The apostrophe after code point q (q = the code point before it, or none)
// stands alone at a piece start: its other-class run has length one (q is not
// O) and no space attaches it to the left (q is not U+0020).  Only then is
// the contraction alternative tried at the apostrophe.
TOK_HD inline bool apos_at_piece_start(uint32_t q) {
  return is_none(q) | ((cls_of(q) != 3u) & !(q & kISpace));
}

constexpr uint32_t kOneLetter = (1u << kCodeS) | (1u << kCodeT) | (1u << kCodeM) | (1u << kCodeD);
constexpr uint32_t kTwoLetter = (1u << kCodeR) | (1u << kCodeV) | (1u << kCodeL);

// Length in code points (1 or 2) of the contraction suffix that begins with
// code point a followed by b (either may be none), or 0.  The alternatives
// are tried in the order s t re ve m ll d; their first letters differ, so at
// most one applies.
TOK_HD inline uint32_t contraction_len(uint32_t a, uint32_t b, bool fold) {
  const uint32_t ca = is_none(a) ? 0u : fold ? fold_code(a) : exact_code(a);
  const uint32_t cb = is_none(b) ? 0u : fold ? fold_code(b) : exact_code(b);
  const uint32_t want = ca == kCodeL ? kCodeL : kCodeE;
  const bool one = (kOneLetter >> ca) & 1u;
  const bool two = ((kTwoLetter >> ca) & 1u) & (cb == want);
  return one ? 1u : two ? 2u : 0u;
}

// Code point j lies inside a letter run (p1 is a letter).  It starts a piece
// iff a contraction ending just before it was matched at the apostrophe that
// precedes the run: "'x" + j or "'xy" + j.
TOK_HD inline bool contraction_split(uint32_t p1, uint32_t p2, uint32_t p3, uint32_t p4, bool fold) {
  // one-letter suffix: p2 = apostrophe, p1 = the letter (p1 starts the run)
  const bool one = !is_none(p2) & ((p2 & kIApos) != 0) & apos_at_piece_start(p3) &
                   (contraction_len(p1, kNone, fold) == 1u);
  // two-letter suffix: p3 = apostrophe, p2 p1 = the letters
  const bool two = !is_none(p3) & ((p3 & kIApos) != 0) & !is_none(p2) & (cls_of(p2) == 0u) &
                   apos_at_piece_start(p4) & (contraction_len(p2, p1, fold) == 2u);
  return one | two;
}

// GPT-2 style: 's|'t|'re|'ve|'m|'ll|'d | ?L+ | ?N+ | ?[^\s L N]+ | \s+(?!\S) | \s+
// c = this code point, p1..p4 = the previous ones, n1 = the next one.
TOK_HD inline bool piece_start_gpt2(uint32_t c, uint32_t p1, uint32_t p2, uint32_t p3, uint32_t p4,
                                    uint32_t n1) {
  const uint32_t k = cls_of(c), k1 = cls_of(p1);
  // whitespace: a run [s, e) is one piece at the end of the text, else
  // [s, e-1) and then e-1 alone (the lookahead gives back one char)
  const bool w = (k1 != 2u) | (!is_none(n1) & (cls_of(n1) != 2u));
  // inside a letter, digit or other run
  const bool same = (k == 0u) & contraction_split(p1, p2, p3, p4, false);
  // run start: an immediately preceding U+0020 attaches to the run, and the
  // letters after a stand-alone apostrophe belong to its contraction
  const bool contr = (k == 0u) & ((p1 & kIApos) != 0) & apos_at_piece_start(p2) &
                     (contraction_len(c, n1, false) != 0u);
  const bool start = !(p1 & kISpace) & !contr;
  return is_none(p1) | (k == 2u ? w : k1 == k ? same : start);
}

// Llama-3 style:
//   (?i:'s|'t|'re|'ve|'m|'ll|'d) | [^\r\n L N]?L+ | N{1,3} | ?[^\s L N]+[\r\n]*
//   | \s*[\r\n]+ | \s+(?!\S) | \s+
// nmod3: digits immediately before c in its digit run, mod 3.
// g: the whitespace run up to c holds only CR/LF so far and follows an O code
//    point (then the O piece's [\r\n]* has absorbed that prefix).
// h: a CR or LF follows c inside its whitespace run.
TOK_HD inline bool piece_start_llama3(uint32_t c, uint32_t p1, uint32_t p2, uint32_t p3, uint32_t p4,
                                      uint32_t n1, uint32_t nmod3, bool g, bool h) {
  const uint32_t k = cls_of(c), k1 = cls_of(p1);
  const bool crlf1 = (p1 & kICrlf) != 0;
  // digits: groups of three from the run start
  const bool d = nmod3 == 0u;
  // letters: one non-CR/LF space char before the run is its optional prefix,
  // and so is a lone O char at a piece start (or its contraction)
  const bool l = k1 == 0u ? contraction_split(p1, p2, p3, p4, true)
                          : (crlf1 | (k1 == 1u)) ? true : k1 == 2u ? false : !apos_at_piece_start(p2);
  // other: U+0020 before the run attaches to it
  const bool o = (k1 != 3u) & !(p1 & kISpace);
  // whitespace: after O the CR/LF block joins the O piece; \s*[\r\n]+ runs to
  // the last CR/LF of the run; then the first char after it, or the run's
  // entry point; e-1 before a non-space run
  const bool w = (c & kICrlf) ? (k1 != 2u) & (k1 != 3u)
                              : (k1 != 2u) | (crlf1 ? (is_none(n1) | !h | g)
                                                     : (!is_none(n1) & (cls_of(n1) != 2u)));
  return is_none(p1) | (k == 0u ? l : k == 1u ? d : k == 2u ? w : o);
}

#if defined(__clang__)
#pragma clang diagnostic pop
#endif

// ---- run aggregates of the Llama-3 style as scans over (reset, value) maps --
//
// forward element, bits: 0 rn, 1-2 an (digits, mod 3), 3 rg, 4 vg
// state (n, g) -> (rn ? an : (n + an) % 3, rg ? vg : (g & vg))
constexpr uint32_t kFwdId = 1u << 4;

TOK_HD inline uint32_t fwd_elem(uint32_t i) {
  const uint32_t k = cls_of(i);
  const bool ds = i & kIDocStart;
  uint32_t rn, an, rg, vg;
  if (k == 1) { rn = ds; an = 1; } else { rn = 1; an = 0; }
  if (k == 2) { rg = ds; vg = ds ? 0u : ((i & kICrlf) ? 1u : 0u); }
  else { rg = 1; vg = (k == 3); }
  return rn | (an << 1) | (rg << 3) | (vg << 4);
}

// f then g
TOK_HD inline uint32_t fwd_comp(uint32_t f, uint32_t g) {
  const uint32_t rn = (f | g) & 1u;
  const uint32_t an = (g & 1u) ? ((g >> 1) & 3u) : ((((f >> 1) & 3u) + ((g >> 1) & 3u)) % 3u);
  const uint32_t rg = ((f | g) >> 3) & 1u;
  const uint32_t vg = ((g >> 3) & 1u) ? ((g >> 4) & 1u) : (((f >> 4) & (g >> 4)) & 1u);
  return rn | (an << 1) | (rg << 3) | (vg << 4);
}

TOK_HD inline bool fwd_resolved(uint32_t e) { return (e & 1u) && (e & 8u); }

// state packed as n | g << 2
TOK_HD inline uint32_t fwd_apply(uint32_t e, uint32_t st) {
  const uint32_t n = st & 3u, g = (st >> 2) & 1u;
  const uint32_t n2 = (e & 1u) ? ((e >> 1) & 3u) : ((n + ((e >> 1) & 3u)) % 3u);
  const uint32_t g2 = (e & 8u) ? ((e >> 4) & 1u) : (g & (e >> 4) & 1u);
  return n2 | (g2 << 2);
}

// backward element, bits: 0 rh, 1 vh; state h -> rh ? vh : (h | vh)
// (h: "a CR/LF lies to the right inside the current whitespace run")
constexpr uint32_t kBwdId = 0u;

TOK_HD inline uint32_t bwd_elem(uint32_t i) {
  if (cls_of(i) != 2) return 1u;  // reset to false
  const uint32_t rh = (i & kILastInDoc) ? 1u : 0u;
  const uint32_t vh = (i & kICrlf) ? 1u : 0u;
  return rh | (vh << 1);
}

// segment l followed (to its right) by segment r
TOK_HD inline uint32_t bwd_comp(uint32_t l, uint32_t r) {
  const uint32_t rh = (l | r) & 1u;
  const uint32_t vh = (l & 1u) ? ((l >> 1) & 1u) : (((r | l) >> 1) & 1u);
  return rh | (vh << 1);
}

TOK_HD inline uint32_t bwd_apply(uint32_t e, uint32_t h) {
  return (e & 1u) ? ((e >> 1) & 1u) : ((h | (e >> 1)) & 1u);
}

}  // namespace tok
