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
};
constexpr uint32_t kNone = 0xFFFFFFFFu;

enum : uint32_t { kCodeS = 1, kCodeT, kCodeR, kCodeE, kCodeV, kCodeM, kCodeL, kCodeD };

TOK_HD inline uint32_t cls_of(uint32_t i) { return i & kIClass; }
TOK_HD inline bool is_none(uint32_t i) { return i == kNone; }
TOK_HD inline bool has(uint32_t i, uint32_t bit) { return i != kNone && (i & bit); }
TOK_HD inline uint32_t exact_code(uint32_t i) { return (i >> kIExactShift) & 15u; }
TOK_HD inline uint32_t fold_code(uint32_t i) { return (i >> kIFoldShift) & 15u; }

// Letter code of an ASCII code point, case-sensitive (lowercase only).
TOK_HD inline uint32_t ascii_letter_code(uint32_t cp) {
  switch (cp) {
    case 's': return kCodeS;
    case 't': return kCodeT;
    case 'r': return kCodeR;
    case 'e': return kCodeE;
    case 'v': return kCodeV;
    case 'm': return kCodeM;
    case 'l': return kCodeL;
    case 'd': return kCodeD;
    default: return 0;
  }
}

// Class of an ASCII code point: letters L, digits N, TAB..CR and space W.
TOK_HD inline uint32_t ascii_class(uint32_t cp) {
  if ((cp | 0x20u) - 'a' < 26u) return 0;  // L
  if (cp - '0' < 10u) return 1;            // N
  if (cp == ' ' || (cp >= 9 && cp <= 13)) return 2;  // W
  return 3;                                 // O
}

// Info word of one decoded code point (class from the caller's table).
TOK_HD inline uint32_t make_info(uint32_t cp, uint32_t cls, uint32_t len, uint32_t fold_extra_code) {
  uint32_t i = cls | kILead | (len << kILenShift);
  if (cp == 0x0D || cp == 0x0A) i |= kICrlf;
  if (cp == 0x20) i |= kISpace;
  if (cp == 0x27) i |= kIApos;
  if (cp < 0x80) {
    uint32_t ex = ascii_letter_code(cp);
    uint32_t fo = ascii_letter_code(cp | 0x20u);
    if ((cp | 0x20u) - 'a' >= 26u) fo = 0;
    i |= ex << kIExactShift;
    i |= fo << kIFoldShift;
  } else {
    i |= fold_extra_code << kIFoldShift;
  }
  return i;
}

// The apostrophe before code point q (q = the code point before the
// apostrophe, or none) stands alone at a piece start: its other-class run has
// length one (q is not O) and no space attaches it to the left (q is not
// U+0020).  Only then is the contraction alternative tried at the apostrophe.
TOK_HD inline bool apos_at_piece_start(uint32_t q) {
  return is_none(q) || (cls_of(q) != 3 && !(q & kISpace));
}

// Length in code points (1 or 2) of the contraction suffix that begins with
// code point a followed by b (b may be none), or 0.  The alternatives are
// tried in the order s t re ve m ll d; their first letters differ, so at most
// one applies.
TOK_HD inline uint32_t contraction_len(uint32_t a, uint32_t b, bool fold) {
  uint32_t ca = fold ? fold_code(a) : exact_code(a);
  switch (ca) {
    case kCodeS: case kCodeT: case kCodeM: case kCodeD: return 1;
    case kCodeR: case kCodeV: case kCodeL: {
      if (is_none(b)) return 0;
      uint32_t cb = fold ? fold_code(b) : exact_code(b);
      uint32_t want = ca == kCodeL ? kCodeL : kCodeE;
      return cb == want ? 2 : 0;
    }
    default: return 0;
  }
}

// Code point j lies inside a letter run (p1 is a letter).  It starts a piece
// iff a contraction ending just before it was matched at the apostrophe that
// precedes the run: "'x" + j or "'xy" + j.
TOK_HD inline bool contraction_split(uint32_t p1, uint32_t p2, uint32_t p3, uint32_t p4, bool fold) {
  // one-letter suffix: p2 = apostrophe, p1 = the letter (p1 starts the run)
  if (has(p2, kIApos) && apos_at_piece_start(p3) && contraction_len(p1, kNone, fold) == 1)
    return true;
  // two-letter suffix: p3 = apostrophe, p2 p1 = the letters
  if (has(p3, kIApos) && !is_none(p2) && cls_of(p2) == 0 && apos_at_piece_start(p4) &&
      contraction_len(p2, p1, fold) == 2)
    return true;
  return false;
}

// GPT-2 style: 's|'t|'re|'ve|'m|'ll|'d | ?L+ | ?N+ | ?[^\s L N]+ | \s+(?!\S) | \s+
// c = this code point, p1..p4 = the previous ones, n1 = the next one.
TOK_HD inline bool piece_start_gpt2(uint32_t c, uint32_t p1, uint32_t p2, uint32_t p3, uint32_t p4,
                                    uint32_t n1) {
  if (is_none(p1)) return true;  // document start
  const uint32_t k = cls_of(c), k1 = cls_of(p1);
  if (k == 2) {
    // a whitespace run [s, e) is one piece at the end of the text, else
    // [s, e-1) and then e-1 alone (the lookahead gives back one char)
    if (k1 != 2) return true;
    return !is_none(n1) && cls_of(n1) != 2;
  }
  if (k1 == k) {  // inside a letter, digit or other run
    return k == 0 && contraction_split(p1, p2, p3, p4, false);
  }
  // run start: an immediately preceding U+0020 attaches to the run
  if (p1 & kISpace) return false;
  if (k == 0 && (p1 & kIApos) && apos_at_piece_start(p2) && contraction_len(c, n1, false))
    return false;  // the letters belong to the contraction piece
  return true;
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
  if (is_none(p1)) return true;
  const uint32_t k = cls_of(c), k1 = cls_of(p1);
  switch (k) {
    case 1:  // digits: groups of three from the run start
      return nmod3 == 0;
    case 0:  // letters
      if (k1 == 0) return contraction_split(p1, p2, p3, p4, true);
      if ((p1 & kICrlf) || k1 == 1) return true;
      if (k1 == 2) return false;  // one non-CR/LF space char is the optional prefix
      // k1 == O: a lone O char at a piece start is the prefix (or a contraction)
      return !apos_at_piece_start(p2);
    case 3:  // other
      if (k1 == 3) return false;
      return !(p1 & kISpace);
    default:  // whitespace
      if (c & kICrlf) {
        if (k1 != 2) return k1 != 3;  // after O the CR/LF block joins the O piece
        return false;                 // \s*[\r\n]+ runs to the last CR/LF of the run
      }
      if (k1 != 2) return true;
      // first char after the last CR/LF of the run, or the run's entry point
      if (p1 & kICrlf) return is_none(n1) || !h || g;
      return !is_none(n1) && cls_of(n1) != 2;  // e-1 before a non-space run
  }
}

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
