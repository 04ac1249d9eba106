// Pre-tokenization kernel: UTF-8 decode and validation, character classes,
// run aggregates and the piece-start predicate, one 1 KiB tile per workgroup.
//
// Each workgroup loads its tile plus 64 bytes of context on each side into LDS
// with coalesced dword loads, decodes every code point once into an info word
// (class and the few character flags the rules test), and evaluates the
// run-local rules of pretok_rules.h at every code point of the tile (TokTier,
// "Exact GPU Tokenization"; GraphTok, section 4 "Parallel tokenizer
// frontends").  Positions are dealt to lanes interleaved (position j * NT +
// thread, with NT = 512 threads for grids of up to 1024 tiles and 256 above),
// so a wave touches 64 consecutive LDS entries at every step and a wave
// ballot yields four flag words at once: bit i of word c is set iff byte
// 16c + i starts a piece.  Ahead of the merge stage (a byte-pair table is
// given) a bit is also set where no token spans the pair of the byte and the
// one before it: BPE cannot join the two sides, so each merges on its own.
//
// The Llama-3 style needs three run aggregates whose runs may cross the tile
// edge.  They are (reset, value) scan elements: one workgroup pass of wave
// scans combines the tile's elements, and the carries into the tile are wave
// reductions over the LDS halos; a run longer than the halo (a long digit or
// whitespace run) falls back to reducing blocks of 16 bytes per thread from
// global memory until the run ends, which costs time only on such input and
// keeps the result exact.
#include "tok_internal.h"
#include "pretok_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"

namespace tok {
namespace {

constexpr int kPT = kPretokTile;          // tile bytes
constexpr int kWin = kPT + 2 * kHalo;     // LDS window bytes
// per-byte flags in LDS
constexpr uint8_t kBDoc = 1, kBOut = 2;

__device__ inline uint32_t dev_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
  if (cp < TOK_CLS_LOW) return (kClsLow[cp >> 2] >> (2 * (cp & 3u))) & 3u;
  if (cp >= 0x110000) return kO;
  const uint32_t blk = kClsBlock[cp >> 8];
  return (kClsBits[blk * 64 + ((cp & 255u) >> 2)] >> (2 * (cp & 3u))) & 3u;
}

__device__ inline uint32_t dev_fold_extra(uint32_t cp) {
#pragma unroll
  for (int i = 0; i < TOK_NFOLD_EXTRA; ++i)
    if (kFoldExtra[i][0] == cp) return ascii_letter_code(kFoldExtra[i][1]);
  return 0;
}

__device__ inline uint32_t utf8_len(uint32_t b) {
  return b < 0x80 ? 1u : b >= 0xF0 ? 4u : b >= 0xE0 ? 3u : 2u;
}

// Code point of the sequence b0 b1 b2 b3 of length len; continuation bits are
// taken as they are (validation is separate).
__device__ inline uint32_t utf8_cp(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, uint32_t len) {
  if (len == 1) return b0;
  if (len == 2) return ((b0 & 0x1Fu) << 6) | (b1 & 0x3Fu);
  if (len == 3) return ((b0 & 0x0Fu) << 12) | ((b1 & 0x3Fu) << 6) | (b2 & 0x3Fu);
  return ((b0 & 0x07u) << 18) | ((b1 & 0x3Fu) << 12) | ((b2 & 0x3Fu) << 6) | (b3 & 0x3Fu);
}


// Scan elements of the code points whose lead byte lies in [x, x + 16), read
// from global memory (slow path for runs longer than the halo).
__device__ void chunk_elems_global(const uint8_t* text, uint64_t n, const uint64_t* doc_off,
                                   uint32_t n_docs, int64_t x, uint32_t* fe, uint32_t* be) {
  uint32_t b[20];
  uint32_t edge = 0;  // bit i: a document starts at x + i, or x + i >= n
  if (x >= 0 && x + 20 <= (int64_t)n && (reinterpret_cast<uintptr_t>(text + x) & 3u) == 0) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(text + x);  // five loads in flight at once
    uint32_t d[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = w[i];
#pragma unroll
    for (int i = 0; i < 20; ++i) b[i] = (d[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  } else {
#pragma unroll
    for (int i = 0; i < 20; ++i) {
      const int64_t p = x + i;
      b[i] = (p >= 0 && p < (int64_t)n) ? text[p] : 0u;
      if (p >= (int64_t)n) edge |= 1u << i;
    }
  }
  if (doc_off) {
    uint32_t d = first_doc_at_or_after(doc_off, n_docs, x < 0 ? 0 : (uint64_t)x);
    for (; d <= n_docs; ++d) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= x + 20) break;
      if ((int64_t)p >= x) edge |= 1u << (uint32_t)(p - x);
    }
  } else if (x <= 0 && x + 20 > 0) {
    edge |= 1u << (uint32_t)(-x);
  }
  uint32_t f = kFwdId, k = kBwdId;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const int64_t p = x + i;
    if (p < 0 || p >= (int64_t)n || (b[i] & 0xC0) == 0x80) continue;
    const uint32_t len = utf8_len(b[i]);
    const uint32_t cp = utf8_cp(b[i], b[i + 1], b[i + 2], b[i + 3], len);
    uint32_t in = make_info(cp, dev_class(cp), len, dev_fold_extra(cp));
    if (edge & (1u << i)) in |= kIDocStart;
    if (edge & (1u << (i + len))) in |= kILastInDoc;
    f = fwd_comp(f, fwd_elem(in));
    k = bwd_comp(k, bwd_elem(in));
  }
  *fe = f;
  *be = k;
}

struct FwdOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return fwd_comp(a, b); }
};
struct BwdOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return bwd_comp(a, b); }
};

// Bytes b .. b + 3 of an LDS byte array read as one word: two aligned word
// loads and a byte funnel shift.
__device__ inline uint32_t lds_word(const uint32_t* a, uint32_t b) {
  return __builtin_amdgcn_alignbyte(a[(b >> 2) + 1], a[b >> 2], b & 3u);
}

__device__ inline bool is_cont(uint32_t byte) { return (byte & 0xC0u) == 0x80u; }

// Occupancy: 8 workgroups per CU for 8-wave workgroups, and for 4-wave ones
// of the Llama-3 style (its register spills cost less than fewer waves: 393
// -> 375 us on the 64 x 500K batch); 6 for the GPT-2 style's 4-wave ones,
// which would spill for nothing.
template <int PATTERN, int NT>
__global__ void __launch_bounds__(NT, NT >= 512 || PATTERN == 1 ? 8 : 6)
pretok_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off,
              uint32_t n_docs, const uint32_t* __restrict__ unit_tab, Bufs B) {
  mark_literals(B.lit);  // for the piece pass, when literal IDs are folded in
  constexpr int kRounds = kPT / NT;                    // tile positions per thread
  constexpr int kPer = kRounds;                        // consecutive positions per thread in the aggregate pass
  static_assert(kPer == 2 || kPer == 4, "aggregate states are packed as 2 or 4 bytes per thread");
  constexpr int kWinRounds = (kWin + NT - 1) / NT;     // window positions per thread
  // window byte k (k in [-4, kWin + 12)) lives at byte 4 + k of s_raw32 / s_fl32 (as bytes)
  constexpr int kGuard = 4, kBytes = kWin + 16;
  static_assert(kBytes % 4 == 0 && (kHalo + kGuard) % 4 == 0, "the window is loaded as aligned dwords");
  __shared__ uint32_t s_raw32[kBytes / 4];
  __shared__ uint32_t s_fl32[kBytes / 4];
  __shared__ uint32_t s_info[kWin];
  __shared__ uint32_t s_scan[NT / kWave], s_scan2[NT / kWave];
  __shared__ uint32_t s_misc[4];
  __shared__ uint32_t s_agg[PATTERN == 1 ? kPT / 4 : 1];  // Llama-3 run states, a byte per tile position
  uint8_t* s_fl = reinterpret_cast<uint8_t*>(s_fl32);

  if (B.n_docs_dev) n_docs = *B.n_docs_dev;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * kPT;
  uint16_t* __restrict__ flags = B.flags;
  // per-call set-up for the later passes: clear the group sums of the tile
  // counts, and check the batch's document offsets
  if (tid == 0) {
    const uint32_t tiles = gridDim.x;
    if (blockIdx.x < ((tiles + 63u) >> kSum1Shift)) B.sum1[blockIdx.x] = 0;
    if (blockIdx.x < ((tiles + 4095u) >> kSum2Shift)) B.sum2[blockIdx.x] = 0;
    if (doc_off && blockIdx.x == 0 && (doc_off[0] != 0 || doc_off[n_docs] != n)) report(&B.ctr->err_docs, B.gen);
  }
  if (doc_off) {
    bool bad_doc = false;
    for (uint32_t d = blockIdx.x * NT + tid; d < n_docs; d += gridDim.x * NT)
      bad_doc |= doc_off[d] > doc_off[d + 1];
    if (bad_doc) report(&B.ctr->err_docs, B.gen);
  }
  const int64_t lo = base - kHalo;
  const int64_t sn = (int64_t)n;

  // the window as dwords, every load in flight before the first wait; bytes
  // outside the text are 0 and flagged kBOut
  {
    constexpr int kWords = kBytes / 4, kR = (kWords + NT - 1) / NT;
    const bool aligned = (reinterpret_cast<uintptr_t>(text) & 3u) == 0;
    uint32_t v[kR], f[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int64_t p = lo - kGuard + 4 * (r * NT + (int)tid);
      v[r] = 0;
      f[r] = 0;
      if (aligned && p >= 0 && p + 4 <= sn) {
        v[r] = *reinterpret_cast<const uint32_t*>(text + p);
      } else {
        for (int i = 0; i < 4; ++i) {
          const bool in = p + i >= 0 && p + i < sn;
          v[r] |= in ? (uint32_t)text[p + i] << (8 * i) : 0u;
          f[r] |= in ? 0u : (uint32_t)kBOut << (8 * i);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int w = r * NT + (int)tid;
      if (w < kWords) {
        s_raw32[w] = v[r];
        s_fl32[w] = f[r];
      }
    }
  }
  if (doc_off && tid == 0) s_misc[0] = first_doc_at_or_after(doc_off, n_docs, lo < 0 ? 0 : (uint64_t)lo);
  __syncthreads();
  if (doc_off) {
    for (uint32_t d = s_misc[0] + tid; d <= n_docs; d += NT) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= lo + kWin) break;
      if ((int64_t)p >= lo && (int64_t)p < sn) s_fl[p - lo + kGuard] |= kBDoc;  // equal offsets write equal bytes
    }
  } else if (tid == 0 && lo <= 0 && sn > 0) {
    s_fl[kGuard - lo] |= kBDoc;
  }
  __syncthreads();

  // decode every window position into an info word, without branches: the
  // bytes of a position and the four before it come from word reads; class
  // lookups of all rounds (one direct table up to U+1FFFF, so emoji too) are
  // issued before any is used
  {
    // the last round covers only the window's tail: a wave wholly past the
    // window skips it (a scalar branch), instead of decoding clamped copies
    const uint32_t wv_s = __builtin_amdgcn_readfirstlane(wv);
    auto live = [&](int j) { return j + 1 < kWinRounds || (int)(wv_s * kWave) + j * NT < kWin; };
    uint32_t cps[kWinRounds], pre[kWinRounds];
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) {
      cps[j] = 0;
      pre[j] = 0;
      if (!live(j)) continue;
      const int k = min((int)(tid + j * NT), kWin - 1);  // positions past the window repeat the last one
      const uint32_t g = (uint32_t)(k + kGuard);
      const uint32_t cur = lds_word(s_raw32, g), prv = lds_word(s_raw32, g - 4u);
      const uint64_t fl = (uint64_t)lds_word(s_fl32, g) | ((uint64_t)lds_word(s_fl32, g + 4u) << 32);
      const uint32_t fprv = lds_word(s_fl32, g - 4u);
      const uint32_t b0 = cur & 0xFFu, b1 = (cur >> 8) & 0xFFu, b2 = (cur >> 16) & 0xFFu, b3 = cur >> 24;
      const uint32_t fl0 = (uint32_t)fl & 0xFFu;
      const bool lead = !(fl0 & kBOut) & !is_cont(b0);
      const uint32_t len = 1u + (b0 >= 0xC0u) + (b0 >= 0xE0u) + (b0 >= 0xF0u);
      const bool undecoded = k + (int)len >= kWin;
      const uint32_t c2 = ((b0 & 0x1Fu) << 6) | (b1 & 0x3Fu);
      const uint32_t c3 = ((b0 & 0x0Fu) << 12) | ((b1 & 0x3Fu) << 6) | (b2 & 0x3Fu);
      const uint32_t c4 = ((b0 & 0x07u) << 18) | ((b1 & 0x3Fu) << 12) | ((b2 & 0x3Fu) << 6) | (b3 & 0x3Fu);
      cps[j] = len == 1u ? b0 : len == 2u ? c2 : len == 3u ? c3 : c4;
      const bool last = ((uint32_t)(fl >> (8u * len)) & (kBDoc | kBOut)) != 0;
      // bytes back to the previous code point's lead (bytes k-1 .. k-4 are
      // prv bytes 3 .. 0); none at a document start or before the text
      const bool q1 = is_cont(prv >> 24), q2 = is_cont((prv >> 16) & 0xFFu), q3 = is_cont((prv >> 8) & 0xFFu);
      uint32_t d = !q1 ? 1u : !q2 ? 2u : !q3 ? 3u : 4u;
      const uint32_t fback = (fprv >> (8u * (4u - d))) & 0xFFu;
      if ((fl0 & kBDoc) | ((fback & kBOut) != 0)) d = 0;
      uint32_t pr = kILead | (len << kILenShift) | ((fl0 & kBDoc) ? kIDocStart : 0u) | (d << kIPrevShift);
      pr |= undecoded ? kIUndecoded : last ? kILastInDoc : 0u;
      pre[j] = lead && k == (int)(tid + j * NT) ? pr : 0u;
    }
    uint32_t cls[kWinRounds];
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) {
      cls[j] = kO;
      if (!live(j)) continue;
      const uint32_t cp = cps[j];
      const uint32_t low = kClsLow[min(cp, (uint32_t)TOK_CLS_LOW - 1u) >> 2];
      cls[j] = cp < 0x80u ? ascii_class(cp) : (low >> (2u * (cp & 3u))) & 3u;
    }
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j)
      if (live(j) && cps[j] >= (uint32_t)TOK_CLS_LOW) cls[j] = dev_class(cps[j]);  // rare: two-level table above U+1FFFF
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) {
      const int k = tid + j * NT;
      if (!live(j) || k >= kWin) continue;
      const uint32_t cp = cps[j], p = pre[j];
      uint32_t in = 0;
      if (p & kIUndecoded) in = kO | p;
      else if (p) in = make_info(cp, cls[j], 0u, dev_fold_extra(cp)) | p;
      s_info[k] = in;
    }
  }

  // UTF-8 validation of the tile's own bytes (Unicode Table 3-7, well-formed
  // byte sequences), from the lead side: every sequence that starts in the
  // tile has a lead in C2..F4 (or is ASCII), its continuation bytes in the
  // same document, the second-byte ranges of E0 ED F0 F4, and no
  // continuation byte after it; no document starts with a continuation byte.
  // Together these leave no stray or missing continuation byte anywhere.
  bool bad = false;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const uint32_t g = (uint32_t)(kHalo + tid + j * NT + kGuard);
    const uint64_t raw = (uint64_t)lds_word(s_raw32, g) | ((uint64_t)lds_word(s_raw32, g + 4u) << 32);
    // a wave whose positions and the four bytes after each are all ASCII is
    // well formed there (bytes outside the text read as 0): skip the checks
    if (__ballot((raw & 0x8080808080ull) != 0) == 0) continue;
    const uint64_t fl = (uint64_t)lds_word(s_fl32, g) | ((uint64_t)lds_word(s_fl32, g + 4u) << 32);
    const uint32_t b0 = (uint32_t)raw & 0xFFu, b1 = (uint32_t)(raw >> 8) & 0xFFu, f0 = (uint32_t)fl & 0xFFu;
    const uint32_t len = 1u + (b0 >= 0xC0u) + (b0 >= 0xE0u) + (b0 >= 0xF0u);
    bool ok = b0 < 0x80u || (b0 >= 0xC2u && b0 <= 0xF4u);
#pragma unroll
    for (uint32_t t = 1; t < 4; ++t) {
      const uint32_t bt = (uint32_t)(raw >> (8 * t)) & 0xFFu, ft = (uint32_t)(fl >> (8 * t)) & 0xFFu;
      ok &= t >= len || (is_cont(bt) && !(ft & (kBOut | kBDoc)));
    }
    ok &= !(b0 == 0xE0u && b1 < 0xA0u) & !(b0 == 0xEDu && b1 > 0x9Fu) & !(b0 == 0xF0u && b1 < 0x90u) &
          !(b0 == 0xF4u && b1 > 0x8Fu);
    const uint32_t bn = (uint32_t)(raw >> (8 * len)) & 0xFFu, fn = (uint32_t)(fl >> (8 * len)) & 0xFFu;
    ok &= (fn & (kBOut | kBDoc)) || !is_cont(bn);
    const bool cont = is_cont(b0);
    bad |= !(f0 & kBOut) && (cont ? (f0 & kBDoc) != 0 : !ok);
  }
  if (bad) report(&B.ctr->err_utf8, B.gen);
  __syncthreads();

  // Llama-3 style: run-aggregate states before (forward) and after (backward)
  // every tile position.  Thread t composes the elements of the kPer
  // consecutive positions kPer t ..; one workgroup pass turns the per-thread
  // compositions into exclusive prefixes (forward) and suffixes (backward);
  // the carries into the tile come from wave reductions over the halos, or,
  // for a run longer than a halo, from blocks of 16 bytes per thread in
  // global memory.  The
  // states go to LDS, one byte per position: n | g << 2 | h << 3.
  if (PATTERN == 1) {
    uint32_t carry_f, carry_h;
    bool fdone, bdone;
    {
      // halo carries: wave 0 composes the 64 positions left of the tile,
      // wave 1 the 64 right of it (identity past an undecoded lead)
      if (wv == 0) {
        const uint32_t in = s_info[lane];
        const uint32_t acc = __builtin_amdgcn_readlane(
            (int)wave_incl_scan((in & kILead) ? fwd_elem(in) : kFwdId, FwdOp(), kFwdId), 63);
        if (lane == 0) {
          s_misc[1] = fwd_apply(acc, 0);
          s_misc[2] = fwd_resolved(acc) || lo <= 0;
        }
      } else if (wv == 1) {
        const uint32_t in = s_info[kHalo + kPT + lane];
        const uint64_t und = __ballot((in & kIUndecoded) != 0);
        const bool past = und && lane >= (uint32_t)__builtin_ctzll(und);
        const uint32_t e = ((in & kILead) && !past) ? bwd_elem(in) : kBwdId;
        const uint32_t acc = __builtin_amdgcn_readlane((int)wave_incl_suffix(e, BwdOp(), kBwdId), 0);
        if (lane == 0) s_misc[3] = bwd_apply(acc, 0) | ((acc & 1u) << 1);
      }
    }
    __syncthreads();
    carry_f = __builtin_amdgcn_readfirstlane(s_misc[1]);
    fdone = __builtin_amdgcn_readfirstlane(s_misc[2]) != 0;
    const uint32_t m3 = __builtin_amdgcn_readfirstlane(s_misc[3]);
    carry_h = m3 & 1u;
    bdone = (m3 >> 1) & 1u;
    if (!fdone) {  // a run longer than the halo ends before the tile: reduce blocks from global memory
      uint32_t acc = kFwdId;
      for (int64_t end = base;; end -= NT * kChunk) {
        const int64_t start = end - NT * kChunk;
        uint32_t fe2, be2;
        chunk_elems_global(text, n, doc_off, n_docs, start + (int64_t)tid * kChunk, &fe2, &be2);
        uint32_t tot;
        wg_excl_scan<NT>(fe2, kFwdId, FwdOp(), s_scan, &tot);
        acc = __builtin_amdgcn_readfirstlane(fwd_comp(tot, acc));  // uniform loop exit
        if (fwd_resolved(acc) || start <= 0) break;
      }
      carry_f = fwd_apply(acc, 0);
    }
    if (!bdone) {
      uint32_t acc = kBwdId;
      for (int64_t start = base + kPT;; start += NT * kChunk) {
        uint32_t fe2, be2;
        chunk_elems_global(text, n, doc_off, n_docs, start + (int64_t)tid * kChunk, &fe2, &be2);
        uint32_t tot;
        wg_excl_suffix<NT>(be2, kBwdId, BwdOp(), s_scan, &tot);
        acc = __builtin_amdgcn_readfirstlane(bwd_comp(acc, tot));  // uniform loop exit
        if ((acc & 1u) || start + NT * kChunk >= sn) break;
      }
      carry_h = bwd_apply(acc, 0);
    }
    // per-thread compositions of kPer consecutive positions, then the
    // workgroup prefix (forward) and suffix (backward) of them
    uint32_t fe[kPer], be[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t in = s_info[kHalo + tid * kPer + i];
      fe[i] = (in & kILead) ? fwd_elem(in) : kFwdId;
      be[i] = (in & kILead) ? bwd_elem(in) : kBwdId;
    }
    uint32_t fcomp = fe[0], bcomp = be[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) {
      fcomp = fwd_comp(fcomp, fe[i]);
      bcomp = bwd_comp(bcomp, be[i]);
    }
    const uint32_t finc = wave_incl_scan(fcomp, FwdOp(), kFwdId);
    const uint32_t binc = wave_incl_suffix(bcomp, BwdOp(), kBwdId);
    if (lane == kWave - 1) s_scan[wv] = finc;
    if (lane == 0) s_scan2[wv] = binc;
    __syncthreads();
    uint32_t wbefore = kFwdId, wafter = kBwdId;
#pragma unroll
    for (uint32_t i = 0; i < (uint32_t)(NT / kWave); ++i) {
      if (i < wv) wbefore = fwd_comp(wbefore, s_scan[i]);
    }
#pragma unroll
    for (int i = NT / kWave - 1; i >= 0; --i) {
      if ((uint32_t)i > wv) wafter = bwd_comp(s_scan2[i], wafter);
    }
    const uint32_t fprev = (uint32_t)__builtin_amdgcn_update_dpp((int)kFwdId, (int)finc, 0x138, 0xF, 0xF, false);
    const uint32_t bnext = (uint32_t)__builtin_amdgcn_update_dpp((int)kBwdId, (int)binc, 0x130, 0xF, 0xF, false);
    const uint32_t pre = fwd_comp(wbefore, lane == 0 ? kFwdId : fprev);         // elements before this thread's positions
    const uint32_t suf = bwd_comp(lane == kWave - 1 ? kBwdId : bnext, wafter);  // elements after them
    // states of this thread's positions
    uint32_t st[kPer];
    uint32_t acc = pre;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      st[i] = fwd_apply(acc, carry_f);
      acc = fwd_comp(acc, fe[i]);
    }
    acc = suf;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      st[i] |= bwd_apply(acc, carry_h) << 3;
      acc = bwd_comp(be[i], acc);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) packed |= st[i] << (8 * i);
    if (kPer == 4) s_agg[tid] = packed;
    else reinterpret_cast<uint16_t*>(s_agg)[tid] = (uint16_t)packed;
    __syncthreads();
  }

  // the piece-start predicate at every tile position: the previous code
  // points come from the back distances stored in the info words (four
  // chained LDS reads), the next one from the code point's length
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int k = kHalo + tid + j * NT;
    const uint32_t c = s_info[k];
    uint32_t p[4];
    uint32_t at = (uint32_t)k, cur = c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = is_none(cur) ? 0u : (cur >> kIPrevShift) & 7u;
      at -= d;
      const uint32_t v = s_info[at];
      cur = d ? v : kNone;
      p[i] = cur;
    }
    const uint32_t len = (c >> kILenShift) & 7u;
    const uint32_t nx = s_info[k + len];
    const uint32_t n1 = (c & kILastInDoc) ? kNone : nx;
    uint32_t agg = 0;
    if (PATTERN == 1) agg = reinterpret_cast<const uint8_t*>(s_agg)[k - kHalo];
    const bool rule = PATTERN == 0 ? piece_start_gpt2(c, p[0], p[1], p[2], p[3], n1)
                                   : piece_start_llama3(c, p[0], p[1], p[2], p[3], n1, agg & 3u, (agg >> 2) & 1u,
                                                        (agg >> 3) & 1u);
    bool st = (c & kILead) && rule;
    if (unit_tab) {  // a unit of BPE also starts where no token can span the boundary
      const uint32_t g = (uint32_t)(k + kGuard) - 2u;
      const uint32_t four = lds_word(s_raw32, g), out = lds_word(s_fl32, g + 1u);  // bytes i - 2 .. i + 1
      // (ASCII pairs are left alone: a cut is never required, and byte-level
      // vocabularies join nearly every ASCII pair)
      if (!((out | (out >> 8)) & kBOut) && (four & 0x808000u)) st = st || no_token_spans(unit_tab, four);
    }
    // this wave holds 64 consecutive positions: four flag words
    const uint64_t m = __ballot(st);
    const uint64_t p0 = (uint64_t)base + (uint64_t)j * NT + wv * kWave;
    if (lane < 4) {
      const uint64_t cw = p0 / kChunk + lane;
      if (cw * kChunk < n) flags[cw] = (uint16_t)(m >> (16 * lane));
    }
  }
}

}  // namespace

void launch_pretok(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                   int pattern, const uint32_t* unit_tab, Bufs b, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t tiles = (uint32_t)((n + kPretokTile - 1) / kPretokTile);
  if (!tiles) return;
  // up to one tile per workgroup slot of the device, 8 waves per tile; larger
  // inputs use 4-wave workgroups, which pack the CUs better
  const bool small = tiles <= (uint32_t)kPretokSmallGrid;
  if (pattern == 2) {  // the case-splitting family: segments between synchronizing cuts
    launch_pretok_case(text, n, doc_off, n_docs, unit_tab, b, s, e0, e1);
  } else if (pattern == 0) {
    if (small)
      launch_on(pretok_kernel<0, 512>, dim3(tiles), dim3(512), s, e0, e1, text, n, doc_off, n_docs, unit_tab, b);
    else
      launch_on(pretok_kernel<0, 256>, dim3(tiles), dim3(256), s, e0, e1, text, n, doc_off, n_docs, unit_tab, b);
  } else {
    if (small)
      launch_on(pretok_kernel<1, 512>, dim3(tiles), dim3(512), s, e0, e1, text, n, doc_off, n_docs, unit_tab, b);
    else
      launch_on(pretok_kernel<1, 256>, dim3(tiles), dim3(256), s, e0, e1, text, n, doc_off, n_docs, unit_tab, b);
  }
}

}  // namespace tok
