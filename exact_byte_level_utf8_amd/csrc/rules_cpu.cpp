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
  seg::Run run(uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) const {
    return seg::run_serial(*this, p, h, mask, tmask);
  }
};

// The same text seen through a tile's loaded window: a read at or past wend
// marks the match as needing the text beyond the window.  Runs go a stretch
// of one kind at a time (rend: the text's run ends, cut at the window's end),
// as the kernel's per-thread matches do.
struct WinAcc {
  const std::vector<uint32_t>* q;
  const std::vector<uint64_t>* rend;
  size_t n;
  uint64_t wend;
  mutable bool far = false;
  uint32_t at(uint64_t i) const {
    if (i >= n) return seg::kQEnd;
    if (i >= wend) {
      far = true;
      return seg::kQEnd;
    }
    return (*q)[i];
  }
  uint64_t run_end(uint64_t i) const { return std::min<uint64_t>((*rend)[i], wend); }
  uint64_t prev_lead(uint64_t i) const {
    uint64_t k = i - 1;
    while (!((*q)[k] & seg::kQLead)) --k;
    return k;
  }
  seg::Run run(uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) const {
    return seg::run_jump(*this, p, h, mask, tmask);
  }
};

// The case-splitting family the way the kernel does it, tile by tile (1 KiB
// tiles, a window of 16 bytes before and 236 valid bytes after each).  A
// tile matches the segments that start at its cuts, each until the cursor
// reaches another cut or the tile's end, reading only its window (by the
// forward scan, with the matcher from a piece that starts with a mark); a match
// that needs more is finished by the unbounded matcher (the kernel's
// workgroup-wide one).  The cursor past the tile's end (the first piece
// start at or after it) goes to the next tile, which continues the segment
// running into it from there: directly if that start is past its first cut,
// else by matching forward, where the piece starts already found from up to
// four of the tile's first code points (speculatively, before the
// predecessor's cursor was known) are taken over as soon as the cursor meets
// one of them.  fallback: ignore the predecessor and find the segment's cut
// by walking back (the kernel's path when a wait runs out).
int case_pieces(const uint8_t* s, size_t n, const std::vector<char>& docstart, std::vector<uint64_t>& out,
                bool fallback) {
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
  std::vector<char> cut(n + 1, 0);
  for (size_t k = 0; k < leads.size(); ++k) {
    const uint64_t j = leads[k];
    cut[j] = k == 0 || docstart[j] || seg::sync_at(q[leads[k - 1]], q[j]);
  }
  // run ends: the next code point start where the kind changes, a document
  // starts or the text ends
  std::vector<uint64_t> rend(n + 1, n);
  {
    uint64_t next = n;
    for (size_t k = leads.size(); k-- > 0;) {
      const uint64_t j = leads[k];
      rend[j] = next;
      if (k == 0 || docstart[j] || seg::kind_of(q[j]) != seg::kind_of(q[leads[k - 1]])) next = j;
    }
  }
  const HostAcc full{&q, n};
  std::vector<char> start(n, 0);
  constexpr size_t kTile = 1024, kLeft = 16, kWin = 1280, kCand = 4;
  uint64_t carry = 0;  // the first piece start at or after the previous tile's end
  for (size_t t0 = 0; t0 < n; t0 += kTile) {
    const size_t t1 = std::min(n, t0 + kTile);
    const WinAcc win{&q, &rend, n, t0 - kLeft + kWin - 4};  // window [t0 - 16, t0 + 1264), decoded up to 4 bytes short
    size_t first = t0;
    while (first < t1 && !(q[first] & seg::kQLead)) ++first;
    size_t first_cut = first;
    while (first_cut < t1 && !((q[first_cut] & seg::kQLead) && cut[first_cut])) ++first_cut;
    // match from a piece start until a cut or the tile's end; returns the
    // cursor there, or kNoPos if the window did not suffice (mark: the
    // starts found, which stay valid)
    auto walk = [&](uint64_t p, const auto& acc, std::vector<char>& mark, bool& far) -> uint64_t {
      far = false;
      for (;;) {
        if (p >= t0 && p < t1) mark[p - t0] = 1;
        seg::Matcher<std::decay_t<decltype(acc)>> m{acc, p};
        m.a.far = false;
        const uint64_t e = m.piece_end();
        if (m.a.far) {  // the matcher holds its own copy of the accessor
          far = true;
          return p;
        }
        if (e <= p) return seg::kNoPos - 1;  // no progress: a matcher bug
        p = e;
        if (p >= t1 || cut[p]) return p;
      }
    };
    // the kernel's per-thread match: the forward scan (seg::scan_step), one
    // code point or one stretch of one kind per step; from a piece that
    // starts with a mark the matcher takes the rest of the segment
    auto walk_scan = [&](uint64_t p, std::vector<char>& mark, bool& far) -> uint64_t {
      far = false;
      const uint64_t wend = win.wend;
      if (p >= t0 && p < t1) mark[p - t0] = 1;
      seg::Scan<uint64_t> sc{p, p, 0, 0, seg::kStStart, 0};
      for (;;) {
        const uint64_t x = sc.x;
        uint32_t v = 0, k;
        uint64_t r = x, pl = x;
        if (x >= n) {
          k = seg::kKEnd;
        } else if (x >= wend) {
          k = seg::kKFar;
        } else {
          v = q[x];
          k = ((v & seg::kQEnd) || (x > sc.p && (v & seg::kQDocStart))) ? (uint32_t)seg::kKEnd : seg::kind_of(v);
          r = std::min<uint64_t>(rend[x], wend);
          if (x > 0) {
            pl = x - 1;
            while (!(q[pl] & seg::kQLead)) --pl;
          }
        }
        const uint32_t res = seg::scan_step(sc, v, k, r, pl);
        if (res == seg::kScanGo) continue;
        if (res == seg::kScanFar) {
          far = true;
          return sc.p;
        }
        if (res == seg::kScanHard) {
          WinAcc w = win;
          return walk(sc.p, w, mark, far);
        }
        const uint64_t e = sc.x;
        if (e <= sc.p) return seg::kNoPos - 1;  // no progress: a scan bug
        if (e >= t1 || cut[e]) return e;
        mark[e - t0] = 1;
        sc = seg::Scan<uint64_t>{e, e, 0, 0, seg::kStStart, 0};
      }
    };
    struct Unbounded {  // the unbounded matcher behind the WinAcc interface
      const HostAcc* f;
      mutable bool far = false;
      uint32_t at(uint64_t i) const { return f->at(i); }
      seg::Run run(uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) const { return f->run(p, h, mask, tmask); }
    };
    const Unbounded unb{&full};
    std::vector<char> tmark(t1 - t0, 0);
    auto walk_any = [&](uint64_t p, std::vector<char>& mark) -> uint64_t {
      bool far = false;
      uint64_t r = walk_scan(p, mark, far);
      if (r == seg::kNoPos - 1) return r;
      if (far) r = walk(r, unb, mark, far);
      return r;
    };
    // the segments that start at the tile's cuts
    uint64_t exit = seg::kNoPos;
    for (size_t j = first_cut; j < t1; ++j) {
      if (!((q[j] & seg::kQLead) && cut[j])) continue;
      const uint64_t r = walk_any(j, tmark);
      if (r == seg::kNoPos - 1) return 2;
      if (r >= t1) exit = r;
    }
    // the segment running into the tile
    if (first < first_cut) {
      // speculative matches from the first code points
      std::vector<std::vector<char>> cmark;
      std::vector<uint64_t> cstart, cexit;
      for (size_t j = first; j < first_cut && cstart.size() < kCand; ++j) {
        if (!(q[j] & seg::kQLead)) continue;
        std::vector<char> mk(t1 - t0, 0);
        bool far = false;
        const uint64_t r = walk_scan(j, mk, far);
        if (r == seg::kNoPos - 1) return 2;
        if (far) continue;  // a candidate that needs the text past the window is dropped
        cmark.push_back(mk);
        cstart.push_back(j);
        cexit.push_back(r);
      }
      uint64_t R = carry;
      if (fallback) {
        // walk back to the segment's cut, then forward to the first piece
        // start at or after t0
        uint64_t c = first;
        while (!cut[c]) {
          --c;
          while (!(q[c] & seg::kQLead)) --c;
        }
        uint64_t p = c;
        while (p < t0) {
          const seg::Matcher<HostAcc> m{full, p};
          const uint64_t e = m.piece_end();
          if (e <= p) return 2;
          p = e;
        }
        R = p;
      }
      uint64_t in_exit = R;
      if (R < first_cut) {
        uint64_t p = R;
        for (;;) {
          size_t hit = cstart.size();
          for (size_t c = 0; c < cstart.size() && hit == cstart.size(); ++c)
            if (cmark[c][p - t0]) hit = c;
          if (hit < cstart.size()) {
            for (size_t i = p - t0; i < t1 - t0; ++i) tmark[i] |= cmark[hit][i];
            in_exit = cexit[hit];
            break;
          }
          // one piece, through the window if it suffices
          tmark[p - t0] = 1;
          seg::Matcher<WinAcc> m{win, p};
          m.a.far = false;
          uint64_t e = m.piece_end();
          if (m.a.far) {
            const seg::Matcher<HostAcc> mf{full, p};
            e = mf.piece_end();
          }
          if (e <= p) return 2;
          p = e;
          if (p >= t1 || cut[p]) {
            in_exit = p;
            break;
          }
        }
      }
      if (first_cut == t1) exit = in_exit;
    } else if (first == t1) {
      exit = carry;  // no code point starts in the tile
    }
    for (size_t i = 0; i < t1 - t0; ++i)
      if (tmark[i]) start[t0 + i] = 1;
    carry = exit;
  }
  for (size_t i = 0; i < n; ++i)
    if (start[i]) out.push_back(i);
  return 0;
}

}  // namespace

// The forward scan of the case-splitting family alone (seg::scan_step) over
// a whole text of one document, with no window and no fallback: the piece
// starts in order, until the first piece the scan leaves to the matcher (one
// that starts with a mark).  Returns the number of starts found, and in
// *hard_at that piece's first byte (n if the scan matched the whole text);
// -1 on malformed input or a step that does not advance.
extern "C" long rules_cpu_scan_pieces(const uint8_t* s, size_t n, uint64_t* starts, size_t cap, uint64_t* hard_at) {
  std::vector<uint32_t> q(n, 0);
  std::vector<uint64_t> leads;
  for (size_t i = 0; i < n;) {
    const uint8_t b = s[i];
    const uint32_t len = b < 0x80 ? 1 : b >= 0xF0 ? 4 : b >= 0xE0 ? 3 : 2;
    if ((b & 0xC0) == 0x80 || i + len > n) return -1;
    uint32_t cp = len == 1 ? b : len == 2 ? (b & 0x1Fu) : len == 3 ? (b & 0x0Fu) : (b & 0x07u);
    for (uint32_t k = 1; k < len; ++k) cp = (cp << 6) | (s[i + k] & 0x3Fu);
    q[i] = seg::make_q(cp, table_case(cp), len, seg::fold_code(cp, fold_extra(cp)));
    leads.push_back(i);
    i += len;
  }
  if (n) q[0] |= seg::kQDocStart;
  // where each stretch of one kind ends
  std::vector<uint64_t> rend(n + 1, n);
  uint64_t next = n;
  for (size_t k = leads.size(); k-- > 0;) {
    const uint64_t j = leads[k];
    rend[j] = next;
    if (k == 0 || seg::kind_of(q[j]) != seg::kind_of(q[leads[k - 1]])) next = j;
  }
  size_t count = 0;
  *hard_at = n;
  uint64_t p = 0;
  while (p < n) {
    if (count < cap) starts[count] = p;
    ++count;
    seg::Scan<uint64_t> sc{p, p, 0, 0, seg::kStStart, 0};
    for (int steps = 0;; ++steps) {
      if (steps > (int)(4 * n + 16)) return -1;
      const uint64_t x = sc.x;
      uint32_t v = 0, k = seg::kKEnd;
      uint64_t r = x, pl = x;
      if (x < n) {
        v = q[x];
        k = (x > sc.p && (v & seg::kQDocStart)) ? (uint32_t)seg::kKEnd : seg::kind_of(v);
        r = rend[x];
        if (x > 0) {
          pl = x - 1;
          while (!(q[pl] & seg::kQLead)) --pl;
        }
      }
      const uint32_t res = seg::scan_step(sc, v, k, r, pl);
      if (res == seg::kScanGo) continue;
      if (res != seg::kScanPiece) {
        *hard_at = sc.p;
        return (long)count - 1;
      }
      break;
    }
    if (sc.x <= p) return -1;
    p = sc.x;
  }
  return (long)count;
}

extern "C" int rules_cpu_class(uint32_t cp) { return (int)table_class(cp); }

// Letter-case classes (U=0 D=1 C=2 M=3 N=4 W=5 O=6) of lo .. lo + n - 1.
extern "C" void rules_cpu_case_range(uint32_t lo, uint32_t n, uint8_t* out) {
  for (uint32_t i = 0; i < n; ++i) out[i] = (uint8_t)table_case(lo + i);
}

// The kernels' table-free letter-case class of an ASCII byte.
extern "C" int rules_cpu_ascii_case(uint32_t b) { return (int)seg::ascii_case(b); }

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
  if (pattern == 2 || pattern == 3) {  // 3: every tile takes the fallback path
    std::vector<uint64_t> st;
    const int rc = case_pieces(s, n, docstart, st, pattern == 3);
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
