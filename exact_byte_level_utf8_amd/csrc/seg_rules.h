// Pre-tokenization of the case-splitting (o200k-style) family by segments.
//
// TokTier, section 4 "Removing the sequential regex scan", describes this
// lineage as the cl100k/Llama-3 rules plus a case-boundary rule inside letter
// runs, a contraction path, and a narrow fallback for marks.  Here the family
// is: an optional prefix char P (not CR, LF, a letter or a number), then
// either H* T+ or H+ T* (H = upper-case or caseless letters or marks, T =
// lower-case or caseless letters or marks), then an optional case-insensitive
// contraction suffix; digit groups of 1-3; an optional space, a run of other
// chars and marks, and trailing CR/LF; whitespace up to the last CR/LF of its
// run; whitespace not followed by non-whitespace; whitespace.
//
// Instead of a per-code-point predicate with run aggregates, the text is cut
// at synchronizing transitions (sync_rules.h: for every left context, a piece
// starts there, the pieces after it are those of the text from there alone,
// and the pieces before it do not depend on the text after it).  Between two
// such cuts the pieces are found by matching the alternatives in order from
// the cut, one piece after another.  Cuts come at nearly every word edge, so
// a segment is short, and each segment is independent of every other.
//
// This header holds the matching logic only; the text is read through an
// accessor (a.at(p): the info word of the code point at byte p), so the same
// code runs in the pre-tokenization kernel and in a CPU build for the tests.
#pragma once

#include <stdint.h>

#include "sync_rules.h"

#ifndef TOK_HD
#define TOK_HD __host__ __device__
#endif
// the matcher's steps are inlined into the one loop that calls them
#define TOK_SEG_INLINE __attribute__((always_inline)) inline

namespace tok {
namespace seg {

// letter-case classes
enum : uint32_t { kSU = 0, kSD = 1, kSC = 2, kSM = 3, kSN = 4, kSW = 5, kSO = 6 };

// info word of the code point at a byte
enum : uint32_t {
  kQSub = 7u,             // bits 0-2: letter-case class
  kQLead = 1u << 3,       // a code point starts at this byte
  kQLenShift = 4,         // bits 4-6: its UTF-8 length
  kQCrlf = 1u << 7,       // U+000D or U+000A
  kQSpace = 1u << 8,      // U+0020
  kQApos = 1u << 9,       // U+0027
  kQFoldShift = 10,       // bits 10-13: contraction letter under case folding (s t r e v m l d = 1..8)
  kQDocStart = 1u << 14,  // a document starts at this byte
  kQEnd = 1u << 15,       // no code point: past the text
  kQCpShift = 16,         // bits 16-31: the code point if below U+10000, else 0xFFFF
};
enum : uint32_t { kFS = 1, kFT, kFR, kFE, kFV, kFM, kFL, kFD };

TOK_HD inline uint32_t sub_of(uint32_t q) { return q & kQSub; }
TOK_HD inline uint32_t len_of(uint32_t q) { return (q >> kQLenShift) & 7u; }
TOK_HD inline uint32_t fold_of(uint32_t q) { return (q >> kQFoldShift) & 15u; }
TOK_HD inline bool in_h(uint32_t s) { return s == kSU || s == kSC || s == kSM; }
TOK_HD inline bool in_t(uint32_t s) { return s == kSD || s == kSC || s == kSM; }
TOK_HD inline bool in_om(uint32_t s) { return s == kSO || s == kSM; }
// the optional prefix char of a letter piece: not CR, LF, a letter or a number
TOK_HD inline bool is_prefix(uint32_t q) { return !(q & kQCrlf) && sub_of(q) >= kSM && sub_of(q) != kSN; }

// Letter-case class of an ASCII code point (b < 0x80) without the table:
// A-Z upper, a-z lower, 0-9 numbers, TAB..CR and space whitespace, the rest
// other (the table's values there; a test checks all 128).  Selects only.
TOK_HD inline uint32_t ascii_case(uint32_t b) {
  const bool letter = (b | 0x20u) - 'a' < 26u, digit = b - '0' < 10u, ws = b - 9u < 5u || b == 0x20u;
  const uint32_t other = digit ? (uint32_t)kSN : ws ? (uint32_t)kSW : (uint32_t)kSO;
  return letter ? (b < 'a' ? (uint32_t)kSU : (uint32_t)kSD) : other;
}

// Info word of a decoded code point.
TOK_HD inline uint32_t make_q(uint32_t cp, uint32_t sub, uint32_t len, uint32_t fold) {
  uint32_t q = sub | kQLead | (len << kQLenShift) | (fold << kQFoldShift);
  q |= (cp == 0x0D || cp == 0x0A) ? kQCrlf : 0u;
  q |= cp == 0x20 ? kQSpace : 0u;
  q |= cp == 0x27 ? kQApos : 0u;
  q |= (cp < 0xFFFFu ? cp : 0xFFFFu) << kQCpShift;
  return q;
}

// Contraction-letter codes of a..p and q..z as nibbles.
constexpr uint64_t contraction_nibbles(char first, char last) {
  uint64_t v = 0;
  for (char ch = first; ch <= last; ++ch) {
    const uint64_t code = ch == 's' ? kFS : ch == 't' ? kFT : ch == 'r' ? kFR : ch == 'e' ? kFE
                        : ch == 'v' ? kFV : ch == 'm' ? kFM : ch == 'l' ? kFL : ch == 'd' ? kFD : 0;
    v |= code << (4 * (ch - first));
  }
  return v;
}
constexpr uint64_t kFoldLo = contraction_nibbles('a', 'p'), kFoldHi = contraction_nibbles('q', 'z');

// Contraction letter of a code point under simple case folding (ASCII letters
// either case; fold_extra: the code for a non-ASCII code point that folds to
// one of them, else 0).  Selects only.
TOK_HD inline uint32_t fold_code(uint32_t cp, uint32_t fold_extra) {
  const uint32_t t = (cp | 0x20u) - 'a';
  const uint32_t ascii = (uint32_t)((t < 16u ? kFoldLo >> (4 * (t & 15u)) : kFoldHi >> (4 * ((t - 16u) & 15u))) & 15u);
  return cp >= 0x80 ? fold_extra : t < 26u ? ascii : 0u;
}

// Kinds of code point for the matcher's runs: the letter-case class, with
// CR and LF (whitespace) apart, and the sets the pattern's loops take.
enum : uint32_t { kKCrlf = 7 };
enum : uint32_t {
  kMaskH = (1u << kSU) | (1u << kSC) | (1u << kSM),      // upper, caseless, marks
  kMaskT = (1u << kSD) | (1u << kSC) | (1u << kSM),      // lower, caseless, marks
  kMaskOM = (1u << kSO) | (1u << kSM),                   // other chars and marks
  kMaskW = (1u << kSW) | (1u << kKCrlf),                 // whitespace
  kMaskCrlf = 1u << kKCrlf,                              // CR, LF
};
TOK_HD inline uint32_t kind_of(uint32_t q) { return (q & kQCrlf) ? (uint32_t)kKCrlf : sub_of(q); }

constexpr uint64_t kNoPos = ~0ull;

// A run of code points whose kinds lie in a set, from a code point start h:
// stop = the first code point start at or after h that ends it (past the
// text, a document start past the cursor, or a kind outside the set); tend =
// the byte after the last code point in [h, stop) whose kind lies in a second
// set (kNoPos if none); last = the first byte of the last code point in
// [h, stop) (kNoPos if the run is empty).
struct Run {
  uint64_t stop, tend, last;
};

// The run, one code point at a time through the accessor's at().
template <typename Acc>
TOK_HD TOK_SEG_INLINE Run run_serial(const Acc& a, uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) {
  Run r{h, kNoPos, kNoPos};
  for (;;) {
    const uint32_t v = a.at(r.stop);
    if ((v & kQEnd) || (r.stop > p && (v & kQDocStart)) || !((mask >> kind_of(v)) & 1u)) return r;
    r.last = r.stop;
    r.stop += len_of(v);
    if ((tmask >> kind_of(v)) & 1u) r.tend = r.stop;
  }
}

// The same run, a stretch of one kind at a time: the accessor also gives
// run_end(i), the first code point start after the code point at i where the
// kind changes, a document starts or the text ends (or the end of what the
// accessor can read), and prev_lead(i), the first byte of the code point
// before i.  A run of one kind costs one step however long it is.
template <typename Acc>
TOK_HD TOK_SEG_INLINE Run run_jump(const Acc& a, uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) {
  uint64_t stop = h, tend = kNoPos;
  for (;;) {
    const uint32_t v = a.at(stop);
    if ((v & kQEnd) || (stop > p && (v & kQDocStart)) || !((mask >> kind_of(v)) & 1u)) break;
    const uint64_t e = a.run_end(stop);
    if ((tmask >> kind_of(v)) & 1u) tend = e;
    stop = e;
  }
  return Run{stop, tend, stop > h ? a.prev_lead(stop) : kNoPos};
}

// The pieces of a segment are matched from a cursor p.  Within a match,
// any position past p where a document starts, or past the text, ends the
// text (documents are hard boundaries).  The accessor gives the info word of
// a byte (at) and the extent of a run (run, as run_serial defines it); every
// loop of the pattern is one run, so an accessor that finds long runs in
// parallel matches long pieces in parallel.
template <typename Acc>
struct Matcher {
  const Acc a;  // held by value, so a device accessor stays in registers
  uint64_t p;  // the cursor: the current piece's first byte

  TOK_HD TOK_SEG_INLINE uint32_t q(uint64_t i) const {
    const uint32_t v = a.at(i);
    return (i > p && (v & kQDocStart)) ? kQEnd : v;
  }
  TOK_HD static bool end(uint32_t v) { return (v & kQEnd) != 0; }
  TOK_HD TOK_SEG_INLINE Run run(uint64_t h, uint32_t mask, uint32_t tmask = 0) const {
    return a.run(p, h, mask, tmask);
  }

  // optional contraction suffix at e: 's 't 're 've 'm 'll 'd, any case
  TOK_HD TOK_SEG_INLINE uint64_t suffix(uint64_t e) const {
    const uint32_t v = q(e);
    if (end(v) || !(v & kQApos)) return e;
    const uint64_t e1 = e + 1;
    const uint32_t v1 = q(e1);
    if (end(v1)) return e;
    const uint32_t f1 = fold_of(v1);
    const uint64_t e2 = e1 + len_of(v1);
    if (f1 == kFS || f1 == kFT || f1 == kFM || f1 == kFD) return e2;
    if (f1 == kFR || f1 == kFV || f1 == kFL) {
      const uint32_t v2 = q(e2);
      if (end(v2)) return e;
      const uint32_t f2 = fold_of(v2);
      if ((f1 == kFL && f2 == kFL) || (f1 != kFL && f2 == kFE)) return e2 + len_of(v2);
    }
    return e;
  }

  // First byte after the piece that starts at the cursor.
  TOK_HD TOK_SEG_INLINE uint64_t piece_end() const {
    const uint32_t v0 = q(p);
    const uint32_t s0 = sub_of(v0);
    const uint64_t n0 = p + len_of(v0);
    // P? H* T+ S?: the prefix taken if possible, then H* as long as it goes;
    // T+ starts at the first char after H* that is in T, else at the last
    // char of the H* stretch that is also in T
    for (int pre = 1; pre >= 0; --pre) {
      if (pre && !is_prefix(v0)) continue;
      const Run h = run(pre ? n0 : p, kMaskH, kMaskT);
      const uint32_t vh = q(h.stop);
      if (!end(vh) && in_t(sub_of(vh))) return suffix(run(h.stop, kMaskT).stop);
      if (h.tend != kNoPos) return suffix(h.tend);
    }
    // P? H+ T* S?
    for (int pre = 1; pre >= 0; --pre) {
      if (pre && !is_prefix(v0)) continue;
      const uint64_t h0 = pre ? n0 : p;
      const uint32_t vh = q(h0);
      if (end(vh) || !in_h(sub_of(vh))) continue;
      return suffix(run(run(h0, kMaskH).stop, kMaskT).stop);
    }
    // digits in groups of one to three
    if (s0 == kSN) {
      uint64_t e = p;
      uint32_t ve = v0;
      for (int k = 0; k < 3 && !end(ve) && sub_of(ve) == kSN; ++k) {
        e += len_of(ve);
        ve = q(e);
      }
      return e;
    }
    // an optional space, other chars and marks, then CR/LF
    {
      uint64_t e = kNoPos;
      if ((v0 & kQSpace) && !end(q(n0)) && in_om(sub_of(q(n0)))) e = n0;
      else if (in_om(s0)) e = p;
      if (e != kNoPos) return run(run(e, kMaskOM).stop, kMaskCrlf).stop;
    }
    // whitespace: up to its last CR/LF; else not followed by non-whitespace;
    // else all of it
    const Run w = run(p, kMaskW, kMaskCrlf);
    if (w.tend != kNoPos) return w.tend;  // CR and LF are one byte each
    if (end(q(w.stop))) return w.stop;
    return w.last != kNoPos && w.last > p ? w.last : w.stop;
  }
};

// The same matches as one forward scan, for a matcher that runs in lockstep
// with others (a wave's lanes): each step reads one code point (or crosses
// one stretch of one kind) and moves a small state machine, so every lane
// does the same work per step whatever alternative its piece takes.  The
// pattern's loops never need to look back, except for two things the scan
// carries along: the end of the last letter in both H and T (where H* T+
// falls back to when T+ finds nothing after H*), and the end of the last
// CR/LF of a whitespace run.  A piece that starts with a mark (a prefix char
// and a letter at once) is left to Matcher.
enum : uint32_t { kKEnd = 8, kKFar = 9 };  // kinds past kind_of's: no code point; past the readable text
enum : uint32_t {
  kStStart,  // at the piece's first code point
  kStPreO,   // after a prefix char that is an other char
  kStPreW,   // after a prefix char that is whitespace (sp: U+0020)
  kStH,      // H* (a: end of the last code point in H and T, or none)
  kStT,      // T+
  kStSuf,    // the contraction suffix at e: its apostrophe
  kStSuf1,   // its first letter
  kStSuf2,   // its second letter (a: the first one's code)
  kStOM,     // other chars and marks
  kStCrlf,   // CR/LF after them
  kStW,      // whitespace (a: end of the last CR/LF, or none)
  kStDig,    // digits (a: how many so far)
};
enum : uint32_t { kScanGo, kScanPiece, kScanFar, kScanHard };

template <typename P>
struct Scan {
  P x;          // the code point the next step reads; after kScanPiece, the piece's end
  P p;          // the piece's first byte
  P a;          // per stage, as above
  P e;          // a letter piece's end before its suffix
  uint32_t st;  // stage
  uint32_t sp;  // the piece's first code point is U+0020
};

// A step as an action word for each (stage, kind): the next stage, how the
// cursor moves, how the stage's position a changes, the outcome, and a few
// cases that look at more than the kind (the apostrophe, the contraction
// letters, the digit count, the ends of letter and whitespace runs).  A
// stage that a step enters takes the stretch at the cursor at once when it
// can, and a run that ends checks the suffix's apostrophe at its end when
// that is where the cursor is, so a typical piece takes three steps.
enum : uint32_t {
  kAxKeep = 0u << 4, kAxLen = 1u << 4, kAxRun = 2u << 4, kAxE = 3u << 4,       // x stays, x += len, x = r, x = e
  kAaKeep = 0u << 6, kAaNone = 1u << 6, kAaRun = 2u << 6, kAaOne = 3u << 6,    // a stays, none, r, 1
  kArGo = 0u << 8, kArPiece = 1u << 8, kArFar = 2u << 8, kArHard = 3u << 8,    // the outcome
  kAfSpO = 1u << 10,   // PreW before an other char: other chars after a space, else the piece ends
  kAfExit = 1u << 11,  // end of H* or T+ (e = a if set, else x), then the suffix from e
  kAfApos = 1u << 12,  // the suffix's apostrophe, or the piece ends at e
  kAfSuf1 = 1u << 13,  // the suffix's first letter
  kAfSuf2 = 1u << 14,  // its second letter
  kAfWEnd = 1u << 15,  // end of a whitespace run
  kAfDig = 1u << 16,   // one more digit, if fewer than three so far
};
constexpr int kScanStages = 12, kScanKinds = 16;  // action table: stage * kScanKinds + kind

TOK_HD constexpr TOK_SEG_INLINE uint32_t scan_action(uint32_t st, uint32_t k) {
  if (k == kKFar) return kArFar;
  if (k > kKFar) return kArHard;  // no such kind
  // entering a letter piece at the cursor: H* takes U, C and M (C and M
  // are in T as well); a lower-case letter starts T+
  const uint32_t letter = (k == kSU)                ? (kStH | kAxRun | kAaNone)
                          : (k == kSC || k == kSM) ? (kStH | kAxRun | kAaRun)
                          : (k == kSD)             ? (kStT | kAxRun | kAaNone)
                                                   : 0u;
  switch (st) {
    case kStStart:
      if (k == kSM) return kArHard;  // a mark is a prefix char and a letter: the matcher's
      if (letter) return letter;
      if (k == kSN) return kStDig | kAxLen | kAaOne;
      if (k == kSO) return kStPreO | kAxLen;
      if (k == kSW) return kStPreW | kAxLen;
      if (k == kKCrlf) return kStW | kAxRun | kAaRun;
      return kArHard;  // no code point
    case kStPreO:  // a letter piece with the prefix, else other chars from the piece's start
      if (letter) return letter;
      if (k == kSO) return kStOM | kAxRun;
      if (k == kKCrlf) return kStCrlf | kAxRun;
      return kArPiece;
    case kStPreW:  // a letter piece with the prefix, a space before other chars, else whitespace
      if (letter) return letter;
      if (k == kSO) return kStOM | kAxRun | kAfSpO;
      if (k == kSW) return kStW | kAxRun | kAaNone;
      if (k == kKCrlf) return kStW | kAxRun | kAaRun;
      return kArPiece;  // the whitespace run is the prefix char alone
    case kStH:
      if (k == kSU) return kStH | kAxRun;
      if (k == kSC || k == kSM) return kStH | kAxRun | kAaRun;
      if (k == kSD) return kStT | kAxRun | kAaNone;
      return kAfExit;
    case kStT:
      if (k == kSD || k == kSC || k == kSM) return kStT | kAxRun;
      return kAfExit;
    case kStSuf:
      return k == kSO ? (uint32_t)kAfApos : (kAxE | kArPiece);
    case kStSuf1:
      return k < kKEnd ? (uint32_t)kAfSuf1 : (kAxE | kArPiece);
    case kStSuf2:
      return k < kKEnd ? (uint32_t)kAfSuf2 : (kAxE | kArPiece);
    case kStOM:
      if (k == kSO || k == kSM) return kStOM | kAxRun;
      if (k == kKCrlf) return kStCrlf | kAxRun;
      return kArPiece;
    case kStCrlf:
      return k == kKCrlf ? (kStCrlf | kAxRun) : (uint32_t)kArPiece;
    case kStW:
      if (k == kKCrlf) return kStW | kAxRun | kAaRun;  // CR and LF are one byte each
      if (k == kSW) return kStW | kAxRun;
      return kAfWEnd;
    case kStDig:
      return k == kSN ? (kStDig | kAfDig) : (uint32_t)kArPiece;
    default:
      return kArHard;
  }
}

// Applies action act to s.  v: the info word at s.x; k: its kind (kind_of,
// or kKEnd past the text or at a document start after s.p, or kKFar past
// what the reader holds); r: the end of the stretch of one kind that starts
// at s.x (capped at what the reader holds); pl: the first byte of the code
// point before s.x.  Returns kScanGo (step again), kScanPiece (s.x: where
// the piece ends), kScanFar (the piece at s.p needs the text past the
// reader) or kScanHard (the piece at s.p starts with a mark).  Written as
// selects only, so lanes in different stages take the same instructions.
template <typename P>
TOK_HD TOK_SEG_INLINE uint32_t scan_apply(Scan<P>& s, uint32_t act, uint32_t v, uint32_t k, P r, P pl) {
  constexpr P kNone = ~P(0);
  const P x = s.x, len = (P)len_of(v);
  const uint32_t xop = act & (3u << 4), aop = act & (3u << 6);
  uint32_t st = act & 15u, res = (act >> 8) & 3u;
  // two independent selects per field (the codes' low and high bits)
  const P x_lo = (xop & kAxLen) ? x + len : x, x_hi = (xop & kAxLen) ? s.e : r;
  P nx = (xop & kAxRun) ? x_hi : x_lo;
  const P a_lo = (aop & kAaNone) ? kNone : s.a, a_hi = (aop & kAaNone) ? P(1) : r;
  P na = (aop & kAaRun) ? a_hi : a_lo;
  P ne = s.e;
  const bool apos = k == kSO && (v & kQApos) != 0;
  if (act & kAfSpO) {  // a space before other chars, else the prefix char alone
    nx = s.sp ? nx : x;
    res = s.sp ? res : (uint32_t)kScanPiece;
  }
  // end of H* or T+: the piece reaches e; a suffix may follow
  if (act & kAfExit) {
    const P e = s.a != kNone ? s.a : x;
    const bool here = e == x;
    ne = e;
    nx = here ? (apos ? x + 1 : x) : e;
    st = here ? (uint32_t)kStSuf1 : (uint32_t)kStSuf;
    res = (here && !apos) ? (uint32_t)kScanPiece : (uint32_t)kScanGo;
  }
  // the suffix after an apostrophe that is not where the run ended, and its
  // letters under case folding: rare, so apart from the rest
  if (act & (kAfApos | kAfSuf1 | kAfSuf2)) {
    const uint32_t f = fold_of(v);
    const bool one = f == kFS || f == kFT || f == kFM || f == kFD, two = f == kFR || f == kFV || f == kFL;
    const bool fin = s.a == kFL ? f == kFL : f == kFE;
    if (act & kAfApos) {
      nx = apos ? x + 1 : s.e;
      st = kStSuf1;
      res = apos ? (uint32_t)kScanGo : (uint32_t)kScanPiece;
    }
    if (act & kAfSuf1) {
      nx = (one || two) ? x + len : s.e;
      na = two ? (P)f : na;
      st = kStSuf2;
      res = two ? (uint32_t)kScanGo : (uint32_t)kScanPiece;
    }
    if (act & kAfSuf2) {
      nx = fin ? x + len : s.e;
      res = kScanPiece;
    }
  }
  // end of a whitespace run: up to its last CR/LF; else all of it at the
  // text's end; else all but its last code point, if that leaves one
  if (act & kAfWEnd) {
    nx = s.a != kNone ? s.a : (k != kKEnd && pl > s.p) ? pl : x;
    res = kScanPiece;
  }
  // digits in groups of at most three
  if (act & kAfDig) {
    const bool more = s.a < 3;
    na = more ? s.a + 1 : s.a;
    nx = more ? x + len : x;
    res = more ? (uint32_t)kScanGo : (uint32_t)kScanPiece;
  }
  s.x = nx;
  s.a = na;
  s.e = ne;
  s.st = st;
  return res;
}

// One step: the action for the stage and kind, applied.
template <typename P>
TOK_HD TOK_SEG_INLINE uint32_t scan_step(Scan<P>& s, uint32_t v, uint32_t k, P r, P pl) {
  if (s.st == kStStart) s.sp = (v & kQSpace) != 0;
  return scan_apply(s, scan_action(s.st, k), v, k, r, pl);
}

// Synchronizing transition from the code point with info x to the one with
// info y (both decoded, both in one document).
TOK_HD inline bool sync_at(uint32_t x, uint32_t y) {
  return sync_transition_case(x >> kQCpShift, sub_of(x), y >> kQCpShift, sub_of(y));
}

}  // namespace seg
}  // namespace tok
