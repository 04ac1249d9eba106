// Pre-tokenization of the case-splitting (o200k-style) family.
//
// TokTier, section 4 "Removing the sequential regex scan", gives this lineage
// a case-boundary rule inside letter runs, a contraction path and a narrow
// fallback for marks.  Rather than one predicate per code point, this kernel
// cuts the text at synchronizing transitions (sync_rules.h: a piece starts
// there for every left context, the pieces after it are those of the text
// from there alone, and the pieces before it do not depend on the text after
// it) and matches the pattern's alternatives from each cut (seg_rules.h).
// Cuts fall at nearly every word edge, so the segments are short and all of
// them are matched at once, one per thread.
//
// One workgroup per 1 KiB tile: the tile, 16 bytes before it and 240 after it
// are loaded into LDS and decoded (code point, letter-case class, CR/LF,
// space, apostrophe, contraction letter, document start).  The tile's own
// bytes are checked as well-formed UTF-8 (Unicode Table 3-7; no sequence may
// cross a document boundary).  The result is the same flag words as the
// other families' pre-tokenization: bit i of word c set iff byte 16c + i
// starts a piece, or, ahead of the merge stage, a unit of BPE (no token spans
// the byte pair there).
//
// Long stretches without a cut (an ideograph run, a digit string, a wall of
// whitespace) cost time linear in their length:
//  - the segment running into a tile from an earlier cut is not re-matched
//    from that cut.  Each tile publishes its cursor past its end (the first
//    piece start at or after it), and the next tile continues from there.
//    A tile with a cut of its own publishes before it waits, so only runs of
//    tiles without a cut wait on one another, each for its predecessor
//    alone.  Workgroups start in index order on each XCD, so the earliest
//    unfinished tile is always running and never waits on anything
//    unfinished; a wait is also bounded in time, after which the tile finds
//    the cursor itself (walking back to the segment's cut).  The cursors are
//    tagged with the call's number, read once per workgroup; the last
//    workgroup to read it advances it for the next call.
//  - while it waits, a tile matches speculatively from its first four code
//    points; once the handed-over cursor meets a piece start of one of these
//    matches, the rest of that match is the tile's (matching from a piece
//    start does not depend on how it was reached).
//  - every loop of the pattern is a run of code points of given kinds.  In
//    the window, a table of where each stretch of one kind ends lets a
//    thread's match cross a stretch in one step; a match that needs the text
//    past the window is finished by the whole workgroup, which finds a run's
//    end 1 KiB per step.
#include "tok_internal.h"
#include "seg_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"
#include "uniclass_case.inc"

namespace tok {
namespace {

using namespace seg;

constexpr int kCaseNT = 256;
constexpr int kCaseTile = kPretokTile;          // 1024 bytes
constexpr int kCaseLeft = 16;                   // bytes before the tile: the code point before it, for cuts and checks
constexpr int kCaseWin = 1280;                  // loaded bytes: [t0 - 16, t0 + 1264)
constexpr int kCaseValid = kCaseWin - 4;        // decoded window bytes (a lead reads the 3 bytes after it)
constexpr int kCand = 4;                        // speculative starts of the segment running into a tile
constexpr int kJobs = kCaseTile + kCand;        // segments (one per cut) and speculative starts
constexpr int kStagePer = 16;                   // bytes per thread and step of the workgroup-wide run search
constexpr int kStage = kStagePer * kCaseNT;     // bytes per step: 4 KiB
constexpr uint32_t kNotLead = 0;                // info of a continuation byte
constexpr uint32_t kNone32 = 0xFFFFFFFFu;       // no position (positions are below TOK_MAX_BYTES < 2^32)
static_assert(kCaseWin % kCaseNT == 0 && kCaseTile % 32 == 0, "window and tile shapes");

__device__ inline uint32_t case_class(uint32_t cp) {
  if (cp < 0x80) return ascii_case(cp);
  if (cp < TOK_CLS_LOW) return (kCaseLow[cp >> 1] >> (4 * (cp & 1u))) & 15u;
  if (cp >= 0x110000) return kSO;
  const uint32_t blk = kCaseBlock[cp >> 8];
  return (kCaseBits[blk * 128 + ((cp & 255u) >> 1)] >> (4 * (cp & 1u))) & 15u;
}

__device__ inline uint32_t case_fold_extra(uint32_t cp) {
#pragma unroll
  for (int i = 0; i < TOK_NFOLD_EXTRA; ++i)
    if (kFoldExtra[i][0] == cp) return fold_code((uint32_t)kFoldExtra[i][1], 0u);
  return 0;
}

__device__ inline uint32_t seq_len(uint32_t b0) { return b0 < 0x80 ? 1u : b0 >= 0xF0 ? 4u : b0 >= 0xE0 ? 3u : 2u; }

__device__ inline uint32_t decode_cp(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, uint32_t len) {
  if (len == 2) return ((b0 & 0x1Fu) << 6) | (b1 & 0x3Fu);
  if (len == 3) return ((b0 & 0x0Fu) << 12) | ((b1 & 0x3Fu) << 6) | (b2 & 0x3Fu);
  if (len == 4) return ((b0 & 0x07u) << 18) | ((b1 & 0x3Fu) << 12) | ((b2 & 0x3Fu) << 6) | (b3 & 0x3Fu);
  return b0;
}

// Info word of the code point whose bytes are b[0 .. len) (taken as given;
// validation is separate).
__device__ inline uint32_t decode_q(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, uint32_t len) {
  const uint32_t cp = decode_cp(b0, b1, b2, b3, len);
  return make_q(cp, case_class(cp), len, fold_code(cp, case_fold_extra(cp)));
}

// Info word of the code point at byte p of the text (kNotLead inside one),
// without a document-start mark.
__device__ inline uint32_t text_q(const uint8_t* text, uint64_t n, uint64_t p) {
  // all four bytes in one round trip
  const uint32_t b0 = text[p];
  const uint32_t b1 = p + 1 < n ? text[p + 1] : 0u;
  const uint32_t b2 = p + 2 < n ? text[p + 2] : 0u;
  const uint32_t b3 = p + 3 < n ? text[p + 3] : 0u;
  if ((b0 & 0xC0u) == 0x80u) return kNotLead;
  return decode_q(b0, b1, b2, b3, seq_len(b0));
}

// The value of the first active lane, as a scalar (the builtin works on
// signed 32-bit values: cast back before any widening).
__device__ __forceinline__ uint32_t uni32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  return ((uint64_t)uni32((uint32_t)(v >> 32)) << 32) | uni32((uint32_t)v);
}

struct CaseShared {
  uint8_t raw[kCaseWin + 4];
  uint16_t rend[kCaseWin];       // at a lead i: where its stretch of one kind ends (window index, at most
                                 // kCaseValid) << 2 | the byte length - 1 of the code point before i,
                                 // and bit 15: i is a cut
  uint8_t ds[kCaseWin];          // a document starts at this byte
  alignas(16) uint8_t stage[kStage + 32];  // 16-byte chunks of the text around one step of a run search
  uint32_t q[kCaseWin];          // info per window byte
  uint32_t cut[kCaseTile / 32];    // cut bit per tile byte
  uint32_t start[kCaseTile / 32];  // piece-start bit per tile byte
  uint32_t job[kJobs];           // a segment's cut; a job that needs the text past the window leaves its cursor here
  uint32_t far[(kJobs + 31) / 32];  // jobs that need the text past the window
  uint32_t hard[(kJobs + 31) / 32];  // jobs at a piece that starts with a mark (the matcher's)
  uint32_t cmask[kCand][kCaseTile / 32];  // piece starts of each speculative match
  uint32_t cstart[kCand], cexit[kCand], cok[kCand];
  uint32_t red[3 * kCaseNT / kWave];
  uint32_t act[kScanStages * kScanKinds];  // the forward scan's action per (stage, kind)
  uint64_t stage_base;           // text position of the step's first byte (kNoPos before the first run search)
  uint32_t stage_off;            // its index in stage
  uint32_t nseg, ncand, doc0, bad, first, first_cut, exit, hand, back;
};

// Workgroup-wide minimum (scratch red[0 .. 4)), and maximum of two values
// (red[4 .. 12)), for one step of a run search.  One barrier each: a step
// writes its scratch again only after the next step's staging barrier, which
// every thread reaches after reading this step's results.
__device__ inline uint32_t wg_min(CaseShared* S, uint32_t v) {
  constexpr int NW = kCaseNT / kWave;
  v = __builtin_amdgcn_readlane((int)wave_incl_scan(v, MinOp{}, kNone32), kWave - 1);
  if (lane_id() == 0) S->red[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = S->red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = min(r, S->red[i]);
  return uni32(r);
}
__device__ inline uint2 wg_max2(CaseShared* S, uint32_t a, uint32_t b) {
  constexpr int NW = kCaseNT / kWave;
  uint32_t* red = S->red + NW;
  a = __builtin_amdgcn_readlane((int)wave_incl_scan(a, MaxOp{}, 0u), kWave - 1);
  b = __builtin_amdgcn_readlane((int)wave_incl_scan(b, MaxOp{}, 0u), kWave - 1);
  if (lane_id() == 0) {
    red[threadIdx.x / kWave] = a;
    red[NW + threadIdx.x / kWave] = b;
  }
  __syncthreads();
  uint32_t ra = red[0], rb = red[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    ra = max(ra, red[i]);
    rb = max(rb, red[NW + i]);
  }
  return make_uint2(uni32(ra), uni32(rb));
}

// The run (seg_rules.h) from the code point start h, found by the whole
// workgroup, 4 KiB of text per step; lim: the end of the text as the match
// sees it (the text's end or the first document start past the cursor).
// Call from all threads with the same arguments.
__device__ Run coop_run(CaseShared* S, const uint8_t* __restrict__ text, uint64_t n, uint64_t lim, uint64_t h,
                        uint32_t mask, uint32_t tmask) {
  const uint32_t tid = threadIdx.x;
  uint32_t tend = 0, last = 0;  // a byte position + 0 / + 1; 0: none yet
  __syncthreads();  // every wave is done reading the previous step's block (CoopAcc::at)
  const uintptr_t end = (uintptr_t)(text + n);
  for (uint64_t base = h;; base += kStage) {
    // the step's bytes as aligned 16-byte chunks, one per thread (threads 0
    // and 1 take one more for the tail), a single load each: a chunk that
    // starts before the text's end holds a byte of the text, so, aligned, it
    // lies in a page the text uses; a later one is zeros.  Bytes around the
    // text's ends are read but never used.
    const uintptr_t al = (uintptr_t)(text + base) & ~(uintptr_t)15;
    const uint32_t off = (uint32_t)((uintptr_t)(text + base) - al);
    for (uint32_t c = tid; c < (uint32_t)(kStage / 16 + 2); c += kCaseNT) {
      const uintptr_t ca = al + 16u * c;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ca < end) v = *reinterpret_cast<const uint4*>(ca);
      *reinterpret_cast<uint4*>(&S->stage[16 * c]) = v;
    }
    if (tid == 0) {
      S->stage_base = base;
      S->stage_off = off;
    }
    __syncthreads();
    const uint64_t x0 = base + kStagePer * tid;
    uint32_t stop = kNone32, my_tend = 0, my_last = 0;
    // two halves of 8 bytes: their code points, every class-table read at
    // once, then the run's test in order
    for (int half = 0; half < kStagePer / 8 && stop == kNone32; ++half) {
      uint32_t cps[8], lens[8], low[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t si = off + kStagePer * tid + 8 * half + j;
        const uint32_t b0 = S->stage[si];
        lens[j] = (b0 & 0xC0u) == 0x80u ? 0u : seq_len(b0);  // 0: inside a code point
        cps[j] = decode_cp(b0, S->stage[si + 1], S->stage[si + 2], S->stage[si + 3], seq_len(b0));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) low[j] = kCaseLow[min(cps[j], (uint32_t)TOK_CLS_LOW - 1u) >> 1];
      for (int j = 0; j < 8; ++j) {
        const uint64_t x = x0 + 8 * half + j;
        if (x >= lim) {  // the first such x over all threads is max(lim, h), as a serial run finds it
          stop = (uint32_t)x;
          break;
        }
        if (!lens[j]) continue;
        const uint32_t cp = cps[j];
        const uint32_t cls = cp < 0x80 ? ascii_case(cp)
                             : cp < TOK_CLS_LOW ? (low[j] >> (4 * (cp & 1u))) & 15u
                                                : case_class(cp);
        const uint32_t k = (cp == 0x0A || cp == 0x0D) ? (uint32_t)kKCrlf : cls;
        if (!((mask >> k) & 1u)) {
          stop = (uint32_t)x;
          break;
        }
        my_last = (uint32_t)x + 1;
        if ((tmask >> k) & 1u) my_tend = (uint32_t)(x + lens[j]);
      }
    }
    const uint32_t f = wg_min(S, stop);
    if (f != kNone32 && x0 > f) my_tend = my_last = 0;  // past the run's end
    const uint2 tl = wg_max2(S, my_tend, my_last);
    tend = max(tend, tl.x);
    last = max(last, tl.y);
    if (f != kNone32) return Run{f, tend ? (uint64_t)tend : kNoPos, last ? (uint64_t)(last - 1) : kNoPos};
  }
}

// The text as a thread's own match reads it: the loaded window only; a read
// at or past its end marks the match as needing the workgroup.
struct WinAcc {
  const uint32_t* q;
  const uint16_t* rend;
  int64_t lo;
  uint64_t n;
  uint64_t wend;
  mutable bool far;
  __device__ __forceinline__ uint32_t at(uint64_t i) const {
    if (i >= n) return kQEnd;
    if (i >= wend) {
      far = true;
      return kQEnd;
    }
    return q[i - lo];
  }
  __device__ __forceinline__ uint64_t run_end(uint64_t i) const { return (uint64_t)(lo + ((rend[i - lo] >> 2) & 0x1FFFu)); }
  __device__ __forceinline__ uint64_t prev_lead(uint64_t i) const {
    int64_t k = (int64_t)i - 1 - lo;
    while (q[k] == kNotLead) --k;
    return (uint64_t)(lo + k);
  }
  __device__ __forceinline__ Run run(uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) const {
    return run_jump(*this, p, h, mask, tmask);
  }
};

// The text as the workgroup's match reads it: the window from LDS, the rest
// from global memory, runs found by coop_run.  Every value is the same in
// every lane (read as scalars), so the match's branches are uniform and the
// barriers inside coop_run are reached by all threads.
struct CoopAcc {
  CaseShared* S;
  int64_t lo;
  const uint8_t* text;
  uint64_t n;
  uint64_t lim;  // the text's end, or the first document start past the entry cursor
  __device__ __forceinline__ uint32_t at(uint64_t i) const {
    uint32_t v;
    const int64_t w = (int64_t)i - lo;
    const uint64_t sb = S->stage_base;
    if (i >= lim) {
      v = kQEnd;
    } else if (w >= 0 && w < kCaseValid) {
      v = S->q[w];
    } else if (i >= sb && i - sb < (uint64_t)kStage) {  // the last block a run search staged
      const uint32_t k = (uint32_t)(i - sb) + S->stage_off, b0 = S->stage[k];
      v = (b0 & 0xC0u) == 0x80u ? kNotLead
                                : decode_q(b0, S->stage[k + 1], S->stage[k + 2], S->stage[k + 3], seq_len(b0));
    } else {
      v = text_q(text, n, i);
    }
    return uni32(v);
  }
  __device__ __forceinline__ Run run(uint64_t p, uint64_t h, uint32_t mask, uint32_t tmask) const {
    const Run r = coop_run(S, text, n, lim, h, mask, tmask);
    return Run{uni64(r.stop), uni64(r.tend), uni64(r.last)};
  }
};

// The first document start after byte p (or the text's end).
__device__ inline uint64_t doc_limit(const uint64_t* doc_off, uint32_t n_docs, uint64_t n, uint64_t p) {
  if (!doc_off) return n;
  const uint32_t d = first_doc_at_or_after(doc_off, n_docs, p + 1);
  return uni64(d <= n_docs ? min(doc_off[d], n) : n);
}

__device__ inline void publish(const Bufs& B, uint32_t tile, uint32_t tag, uint64_t cursor) {
  __hip_atomic_store(&B.hand_state[tile], ((uint64_t)tag << 32) | (uint32_t)cursor, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(kCaseNT)
pretok_case_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off,
                   uint32_t n_docs, const uint32_t* __restrict__ unit_tab, Bufs B) {
  __shared__ CaseShared sh;
  CaseShared* S = &sh;
  mark_literals(B.lit);  // for the piece pass, when literal IDs are folded in
  if (B.n_docs_dev) n_docs = *B.n_docs_dev;
  const uint32_t tid = threadIdx.x;
  const uint32_t tiles = gridDim.x;
  const uint32_t tile = blockIdx.x;
  // the call's number (thread 0 only: it publishes and waits); the count of
  // workgroups that have read it is taken later, off the critical path
  uint64_t epoch = 0;
  if (tid == 0) {
    epoch = __hip_atomic_load(&B.hand_tick[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // per-call set-up for the later passes: clear the group sums of the tile
    // counts, and check the batch's document offsets
    if (blockIdx.x < ((tiles + 63u) >> kSum1Shift)) B.sum1[blockIdx.x] = 0;
    if (blockIdx.x < ((tiles + 4095u) >> kSum2Shift)) B.sum2[blockIdx.x] = 0;
    if (doc_off && blockIdx.x == 0 && (doc_off[0] != 0 || doc_off[n_docs] != n)) report(&B.ctr->err_docs, B.gen);
  }
  const uint32_t tag = (uint32_t)(epoch % 0xFFFFFFFFull) + 1u;  // meaningful in thread 0
  if (doc_off) {
    bool bad_doc = false;
    for (uint32_t d = blockIdx.x * kCaseNT + tid; d < n_docs; d += gridDim.x * kCaseNT)
      bad_doc |= doc_off[d] > doc_off[d + 1];
    if (bad_doc) report(&B.ctr->err_docs, B.gen);
  }
  const int64_t t0 = (int64_t)tile * kCaseTile;
  const int64_t lo = t0 - kCaseLeft;
  const int64_t t1 = min((int64_t)n, t0 + kCaseTile);
  if (tid == 0) {
    S->nseg = 0;
    S->ncand = 0;
    S->bad = 0;
    S->first_cut = (uint32_t)t1;
    S->exit = (uint32_t)t1;
    S->stage_base = kNoPos;
    S->doc0 = doc_off ? first_doc_at_or_after(doc_off, n_docs, (uint64_t)max(lo, (int64_t)0)) : 0u;
  }
#pragma unroll
  for (int r = 0; r < kCaseWin / kCaseNT; ++r) {  // all loads in flight at once
    const int i = tid + r * kCaseNT;
    const int64_t p = lo + i;
    S->raw[i] = p >= 0 && p < (int64_t)n ? text[p] : 0;
    S->ds[i] = 0;
  }
  if (tid < 4) S->raw[kCaseWin + tid] = 0;
  for (int i = tid; i < kCaseTile / 32; i += kCaseNT) {
    S->cut[i] = 0;
    S->start[i] = 0;
  }
  for (int i = tid; i < kCand * (kCaseTile / 32); i += kCaseNT) S->cmask[i / (kCaseTile / 32)][i % (kCaseTile / 32)] = 0;
  for (int i = tid; i < (kJobs + 31) / 32; i += kCaseNT) {
    S->far[i] = 0;
    S->hard[i] = 0;
  }
  for (int i = tid; i < kScanStages * kScanKinds; i += kCaseNT) S->act[i] = scan_action(i / kScanKinds, i % kScanKinds);
  __syncthreads();
  // document starts inside the window
  if (doc_off) {
    for (uint32_t d = S->doc0 + tid; d <= n_docs; d += kCaseNT) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= lo + kCaseWin || p >= n) break;
      if ((int64_t)p >= lo) S->ds[p - lo] = 1;
    }
  } else if (lo <= 0 && tid == 0) {
    S->ds[-lo] = 1;
  }
  __syncthreads();
  // decode every window byte: the code points, then all their class-table
  // reads at once (one round trip; none in a wave without a non-ASCII
  // byte), then the info words
  {
    constexpr int kPer = kCaseWin / kCaseNT;
    uint32_t cps[kPer], lens[kPer], low[kPer];
    bool hi = false, big = false;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + r * kCaseNT;
      const uint32_t b0 = S->raw[i];
      lens[r] = seq_len(b0);
      cps[r] = decode_cp(b0, S->raw[i + 1], S->raw[i + 2], S->raw[i + 3], lens[r]);
      hi |= cps[r] >= 0x80u;
      big |= cps[r] >= (uint32_t)TOK_CLS_LOW;
      low[r] = 0;
    }
    if (__ballot(hi)) {
#pragma unroll
      for (int r = 0; r < kPer; ++r) low[r] = kCaseLow[min(cps[r], (uint32_t)TOK_CLS_LOW - 1u) >> 1];
    }
    const bool any_big = __ballot(big) != 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + r * kCaseNT;
      const int64_t p = lo + i;
      const uint32_t b0 = S->raw[i], cp = cps[r];
      uint32_t cls = cp < 0x80 ? ascii_case(cp) : (low[r] >> (4 * (cp & 1u))) & 15u;
      if (any_big) cls = cp >= (uint32_t)TOK_CLS_LOW ? case_class(cp) : cls;
      const uint32_t q = make_q(cp, cls, lens[r], fold_code(cp, case_fold_extra(cp))) | (S->ds[i] ? kQDocStart : 0u);
      S->q[i] = (p < 0 || p >= (int64_t)n) ? kQEnd : (b0 & 0xC0u) == 0x80u ? kNotLead : q;
    }
  }
  // well-formed UTF-8 over the tile's own bytes (Unicode Table 3-7): a lead
  // is ASCII or C2..F4 with the right continuation bytes, all in its
  // document; a continuation byte belongs to a lead at most 3 bytes before
  // it in the same document.  A wave whose bytes are all ASCII has nothing
  // to check.
  {
    constexpr int kRounds = kCaseTile / kCaseNT;
    bool hi = false;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) hi |= S->raw[kCaseLeft + r * kCaseNT + tid] >= 0x80u;
    if (__ballot(hi)) {
      bool bad = false;
      auto cont = [](uint32_t b) { return (b & 0xC0u) == 0x80u; };
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int i = kCaseLeft + r * kCaseNT + tid;
        const int64_t p = lo + i;
        const uint32_t b0 = S->raw[i], b1 = S->raw[i + 1], b2 = S->raw[i + 2], b3 = S->raw[i + 3];
        const uint32_t r1 = S->raw[i - 1], r2 = S->raw[i - 2], r3 = S->raw[i - 3];
        // a continuation byte: back over continuation bytes of the same
        // document to the lead
        const bool c1 = cont(r1) && !S->ds[i - 1], c2 = cont(r2) && !S->ds[i - 2], c3 = cont(r3) && !S->ds[i - 3];
        const int k = !c1 ? 1 : !c2 ? 2 : !c3 ? 3 : 4;
        const uint32_t lead = k == 1 ? r1 : k == 2 ? r2 : r3;
        const bool bad_cont = S->ds[i] || k > 3 || p - k < 0 || cont(lead) || lead < 0xC2u || lead > 0xF4u ||
                              (int)seq_len(lead) <= k;
        // a lead: its continuation bytes, in the text and the document, and
        // the narrower second-byte ranges after E0, ED, F0 and F4
        const uint32_t len = seq_len(b0);
        const bool bad_lead = b0 < 0xC2u || b0 > 0xF4u || p + (int64_t)len > (int64_t)n ||
                              (len > 1 && (!cont(b1) || S->ds[i + 1])) || (len > 2 && (!cont(b2) || S->ds[i + 2])) ||
                              (len > 3 && (!cont(b3) || S->ds[i + 3])) || (b0 == 0xE0u && b1 < 0xA0u) ||
                              (b0 == 0xEDu && b1 > 0x9Fu) || (b0 == 0xF0u && b1 < 0x90u) || (b0 == 0xF4u && b1 > 0x8Fu);
        bad |= p < t1 && (cont(b0) ? bad_cont : b0 >= 0x80u && bad_lead);
      }
      if (bad) S->bad = 1;
    }
  }
  // at the end, after the last barrier (a barrier waits for every memory
  // operation in flight, and this one is contended): count this workgroup
  // among those that have read the call's number (the add waits for the
  // read: its operand depends on it; never more than 1), and the last one
  // counted starts the next call's number
  auto finish = [&]() {
    if (tid == 0) {
      const uint64_t counted = atomicAdd((unsigned long long*)&B.hand_tick[kHandCountWord], 1ull + (epoch >> 63));
      if (counted == tiles - 1) {
        __hip_atomic_store(&B.hand_tick[kHandCountWord], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&B.hand_tick[0], epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  __syncthreads();
  const uint64_t c0 = (uint64_t)tile * (kCaseTile / kChunk);
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  if (S->bad) {  // uniform: the call reports malformed input; the flags are zero
    if (tid == 0) {
      report(&B.ctr->err_utf8, B.gen);
      publish(B, tile, tag, (uint64_t)t1);  // a cursor all the same, so no successor waits
    }
    for (int c = tid; c < kCaseTile / kChunk; c += kCaseNT)
      if (c0 + c < n_chunks) B.flags[c0 + c] = 0;
    finish();
    return;
  }

  // cuts at the tile's code points (a wave's ballot is two words of the cut
  // bits), and the segments that start at them: the ballots of all rounds
  // first, then one slot reservation per wave
  {
    constexpr int kRounds = kCaseTile / kCaseNT;
    const uint32_t lane = lane_id();
    const uint64_t below = (1ull << lane) - 1;
    uint64_t m[kRounds];
    uint32_t total = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int64_t p = t0 + r * kCaseNT + tid;
      const int i = (int)(p - lo);
      const uint32_t v = S->q[i];
      // the code point before starts 1 to 4 bytes back in well-formed text (in
      // malformed text, which its own tile reports, any value will do)
      const uint32_t v1 = S->q[i - 1], v2 = S->q[i - 2], v3 = S->q[i - 3], v4 = S->q[i - 4];
      const uint32_t prev = v1 != kNotLead ? v1 : v2 != kNotLead ? v2 : v3 != kNotLead ? v3 : v4;
      const bool cut = p < t1 && v != kNotLead && (p == 0 || (v & kQDocStart) || sync_at(prev, v));
      m[r] = __ballot(cut);
      total += (uint32_t)__popcll(m[r]);
      if (lane == 0) {
        const uint32_t w0 = (uint32_t)(r * kCaseNT + (tid - lane)) / 32;
        S->cut[w0] = (uint32_t)m[r];
        S->cut[w0 + 1] = (uint32_t)(m[r] >> 32);
      }
    }
    uint32_t base = 0;
    if (lane == 0 && total) base = atomicAdd(&S->nseg, total);
    base = __shfl(base, 0, kWave);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      if ((m[r] >> lane) & 1u) S->job[base + __popcll(m[r] & below)] = (uint32_t)(t0 + r * kCaseNT + tid);
      base += (uint32_t)__popcll(m[r]);
    }
  }
  __syncthreads();
  auto is_cut = [&](uint64_t p) { return (S->cut[(p - t0) >> 5] >> ((p - t0) & 31)) & 1u; };
  // the tile's first code point, its first cut, and speculative starts
  // before its first cut
  if (tid == 0) {
    uint32_t fc = (uint32_t)t1;
    for (int w = 0; w < kCaseTile / 32; ++w)
      if (S->cut[w]) {
        fc = (uint32_t)(t0 + 32 * w + __builtin_ctz(S->cut[w]));
        break;
      }
    S->first_cut = fc;
    int64_t f = t0;
    while (f < t1 && S->q[f - lo] == kNotLead) ++f;
    S->first = (uint32_t)f;
    uint32_t nc = 0;
    for (int64_t j = f; j < (int64_t)S->first_cut && nc < (uint32_t)kCand; ++j) {
      if (S->q[j - lo] == kNotLead) continue;
      S->cstart[nc] = (uint32_t)j;
      S->cexit[nc] = (uint32_t)t1;
      S->cok[nc] = 1;
      ++nc;
    }
    S->ncand = nc;
  }
  // where each stretch of one kind ends: a boundary at every code point
  // whose kind differs from the one before it, where a document starts or
  // the text ends, and at the window's decoded end; each thread takes 5
  // consecutive bytes (and the 4 before them, for the code point before
  // each), and the first boundary after them comes from a suffix minimum
  // over the workgroup
  {
    constexpr int kPer = kCaseWin / kCaseNT;
    const int i0 = tid * kPer;
    uint32_t w[kPer + 4];  // info of bytes i0 - 4 .. i0 + kPer - 1
#pragma unroll
    for (int j = 0; j < kPer + 4; ++j) w[j] = S->q[max(i0 + j - 4, 0)];
    uint32_t bmask = 0, plen[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = i0 + j;
      const uint32_t v = w[j + 4];
      // the code point before i starts 1 to 4 bytes back in well-formed text
      const uint32_t back = w[j + 3] != kNotLead ? 1u : w[j + 2] != kNotLead ? 2u : w[j + 1] != kNotLead ? 3u : 4u;
      const uint32_t prev = back == 1u ? w[j + 3] : back == 2u ? w[j + 2] : back == 3u ? w[j + 1] : w[j];
      plen[j] = back;
      bool b;
      if (i >= kCaseValid) b = i == kCaseValid;
      else if (v == kNotLead) b = false;
      else b = i == 0 || (v & (kQDocStart | kQEnd)) || kind_of(prev) != kind_of(v);
      bmask |= (uint32_t)b << j;
    }
    const uint32_t mine = bmask ? (uint32_t)(i0 + __builtin_ctz(bmask)) : kNone32;
    uint32_t next = wg_excl_suffix<kCaseNT>(mine, kNone32, MinOp{}, S->red, nullptr);
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {
      const int i = i0 + j;
      const uint32_t ti = (uint32_t)(i - kCaseLeft);  // the tile byte, if in the tile
      const uint32_t cut = ti < (uint32_t)kCaseTile ? (S->cut[ti >> 5] >> (ti & 31)) & 1u : 0u;
      S->rend[i] = (uint16_t)(cut << 15 | min(next, (uint32_t)kCaseValid) << 2 | (plen[j] - 1u));
      if ((bmask >> j) & 1u) next = (uint32_t)i;
    }
  }
  __syncthreads();
  const WinAcc wacc{S->q, S->rend, lo, n, (uint64_t)(lo + kCaseValid), false};

  // every job, one per thread: a segment from its cut, or a speculative
  // start, matched until the next cut or the tile's end by the forward scan
  // (seg_rules.h), one step per iteration; a lane that finishes a job takes
  // its next one at once
  const uint32_t nseg = S->nseg, njobs = nseg + S->ncand;
  auto tile_bit = [&](uint32_t* words, uint32_t w) {  // w: a window index in the tile
    atomicOr(&words[(w - kCaseLeft) >> 5], 1u << ((w - kCaseLeft) & 31));
  };
  {
    const uint32_t tw1 = (uint32_t)(t1 - lo);                  // the tile's end as a window index
    // the kind past the decoded window: more text, or its end
    const uint32_t kpast = lo + kCaseValid < (int64_t)n ? (uint32_t)kKFar : (uint32_t)kKEnd;
    uint32_t jb = tid;
    uint32_t* mark = S->start;
    uint32_t js = 0;  // the job's first byte
    Scan<uint32_t> sc{0u, 0u, 0u, 0u, kStStart, 0u};
    auto open = [&]() {
      const bool cand = jb >= nseg;
      js = (uint32_t)((int64_t)(cand ? S->cstart[jb - nseg] : S->job[jb]) - lo);
      mark = cand ? S->cmask[jb - nseg] : S->start;
      sc = Scan<uint32_t>{js, js, 0u, 0u, kStStart, 0u};
    };
    if (jb < njobs) open();
    while (jb < njobs) {
      const uint32_t x = sc.x;
      const uint32_t xi = min(x, (uint32_t)kCaseValid - 1u);
      const uint32_t v = S->q[xi];
      const uint32_t rr = S->rend[xi];
      const bool gone = ((v & kQEnd) != 0) | ((x > sc.p) & ((v & kQDocStart) != 0));  // bitwise: no branches
      const uint32_t kin = gone ? (uint32_t)kKEnd : kind_of(v);
      const uint32_t k = x >= (uint32_t)kCaseValid ? kpast : kin;
      const uint32_t act = S->act[sc.st * kScanKinds + k];
      // at a piece's first code point: the job ends at the tile's end or at
      // another cut; else the piece starts here
      const bool at_start = sc.st == kStStart;
      const bool seg_end = at_start & ((x >= tw1) | (((rr >> 15) != 0) & (x != js)));
      if (at_start & !seg_end) tile_bit(mark, x);
      sc.sp = at_start ? (uint32_t)((v & kQSpace) != 0) : sc.sp;
      const uint32_t res = scan_apply(sc, act, v, k, (rr >> 2) & 0x1FFFu, x - 1u - (rr & 3u));
      if (!seg_end && res < kScanFar) {
        const bool piece = res == kScanPiece;
        const uint32_t e = sc.x > sc.p ? sc.x : sc.p + 1u;  // a piece always advances; the guard keeps the loop finite regardless
        sc.x = piece ? e : sc.x;
        sc.p = piece ? e : sc.p;
        sc.st = piece ? (uint32_t)kStStart : sc.st;
        continue;
      }
      const bool cand = jb >= nseg;
      if (seg_end) {
        if (cand) S->cexit[jb - nseg] = (uint32_t)(lo + x);
        else if (x >= tw1) S->exit = (uint32_t)(lo + x);
      } else {  // the matcher's (a mark) or the workgroup's (the text past the window), from this piece
        S->job[jb] = (uint32_t)(lo + sc.p);
        if (res == kScanHard) atomicOr(&S->hard[jb >> 5], 1u << (jb & 31));
        else if (cand) S->cok[jb - nseg] = 0;  // a speculative match that needs more is dropped
        else atomicOr(&S->far[jb >> 5], 1u << (jb & 31));
      }
      jb += kCaseNT;
      if (jb < njobs) open();
    }
  }
  __syncthreads();

  // jobs at a piece that starts with a mark: the matcher, one thread each
  for (uint32_t jb = tid; jb < njobs; jb += kCaseNT) {
    if (!((S->hard[jb >> 5] >> (jb & 31)) & 1u)) continue;
    const bool cand = jb >= nseg;
    const uint32_t c = jb - nseg;
    uint64_t p = S->job[jb];
    uint32_t* mark = cand ? S->cmask[c] : S->start;
    for (;;) {
      atomicOr(&mark[(p - t0) >> 5], 1u << ((p - t0) & 31));
      const Matcher<WinAcc> m{wacc, p};
      const uint64_t e = m.piece_end();
      if (m.a.far) {  // the workgroup finishes it
        if (cand) {
          S->cok[c] = 0;
        } else {
          S->job[jb] = (uint32_t)p;
          atomicOr(&S->far[jb >> 5], 1u << (jb & 31));
        }
        break;
      }
      p = e > p ? e : p + 1;  // a match always advances; the guard keeps the loop finite regardless
      if ((int64_t)p >= t1) {
        if (cand) S->cexit[c] = (uint32_t)p;
        else S->exit = (uint32_t)p;
        break;
      }
      if (is_cut(p)) {
        if (cand) S->cexit[c] = (uint32_t)p;
        break;
      }
    }
  }
  __syncthreads();

  // the segments whose matches need the text past the window, one at a time
  // by the whole workgroup, from where the thread stopped
  auto coop_walk = [&](uint64_t p) {
    const CoopAcc acc{S, lo, text, n, doc_limit(doc_off, n_docs, n, p)};
    for (;;) {
      if (tid == 0) atomicOr(&S->start[(p - t0) >> 5], 1u << ((p - t0) & 31));
      const Matcher<CoopAcc> m{acc, p};
      const uint64_t e = uni64(m.piece_end());
      p = e > p ? e : p + 1;
      if ((int64_t)p >= t1) return p;
      if (is_cut(p)) return p;
    }
  };
  for (uint32_t w = 0; w < (njobs + 31) / 32; ++w) {
    uint32_t bits = uni32(S->far[w]);
    while (bits) {
      const uint32_t jb = w * 32 + __builtin_ctz(bits);
      bits &= bits - 1;
      const uint64_t e = coop_walk(uni32(S->job[jb]));
      if ((int64_t)e >= t1 && tid == 0) S->exit = (uint32_t)e;
    }
  }
  __syncthreads();

  // a tile with a cut knows its cursor past its end: the last segment's
  const uint32_t first = uni32(S->first);
  const uint32_t first_cut = uni32(S->first_cut);
  if ((int64_t)first_cut < t1 && tid == 0) publish(B, tile, tag, S->exit);

  // the segment running into the tile, from the predecessor's cursor
  if (tile > 0 && (first < first_cut || (int64_t)first_cut == t1)) {
    // wave 0 reads the words of the 64 tiles before this one at once: the
    // nearest published one decides if it is the predecessor's, or if its
    // cursor already lies at or past this tile's start (then no tile in
    // between has a piece start, and the cursor passes through them)
    if (tid < kWave) {
      const uint32_t wtag = uni32(tag);
      const int64_t j = (int64_t)tile - 1 - tid;
      const uint64_t t_start = B.hand_wait ? (uint64_t)wall_clock64() : 0;
      uint32_t r = kNone32;
      for (;;) {
        const uint64_t v = j >= 0 ? __hip_atomic_load(&B.hand_state[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        const uint64_t pub = __ballot(j >= 0 && (uint32_t)(v >> 32) == wtag);
        if (pub) {
          const int l = __builtin_ctzll(pub);
          const uint32_t c = (uint32_t)__shfl((int)(uint32_t)v, l, kWave);
          if (l == 0 || (int64_t)c >= t0) {
            r = c;
            break;
          }
        }
        if (!B.hand_wait || (uint64_t)wall_clock64() - t_start > B.hand_wait) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (tid == 0) S->hand = r;
    }
    __syncthreads();
    uint64_t R = uni32(S->hand);
    if (R == kNone32) {
      // the wait ran out: walk back to the segment's cut (a document start
      // at the latest), then match forward to the tile
      if (tid == 0) {
        uint64_t dstart = 0;
        if (doc_off) {
          const uint32_t d = first_doc_at_or_after(doc_off, n_docs, (uint64_t)first + 1);
          dstart = d > 0 ? doc_off[d - 1] : 0;
        }
        auto info = [&](uint64_t p) {
          const int64_t w = (int64_t)p - lo;
          return w >= 0 && w < kCaseValid ? S->q[w] : text_q(text, n, p);
        };
        uint64_t j = first;
        uint32_t vj = info(j);
        while (j > dstart) {
          uint64_t k = j - 1;
          while (k > dstart && info(k) == kNotLead) --k;
          const uint32_t vk = info(k);
          if (sync_at(vk, vj)) break;
          j = k;
          vj = vk;
        }
        S->back = (uint32_t)j;
      }
      __syncthreads();
      uint64_t p = uni32(S->back);
      const CoopAcc acc{S, lo, text, n, doc_limit(doc_off, n_docs, n, p)};
      while ((int64_t)p < t0) {
        const Matcher<CoopAcc> m{acc, p};
        const uint64_t e = uni64(m.piece_end());
        p = e > p ? e : p + 1;
      }
      R = p;
    }
    uint64_t in_exit = R;
    if (R < first_cut) {
      uint64_t p = R;
      for (;;) {
        // a piece start of a speculative match: the rest of that match
        uint32_t hit = kNone32;
        for (uint32_t c = 0; c < S->ncand && hit == kNone32; ++c)
          if (S->cok[c] && ((S->cmask[c][(p - t0) >> 5] >> ((p - t0) & 31)) & 1u)) hit = c;
        hit = uni32(hit);
        if (hit != kNone32) {
          if (tid < kCaseTile / 32) {
            const uint32_t b = (uint32_t)(p - t0);
            const uint32_t keep = tid < (b >> 5) ? 0u : tid == (b >> 5) ? ~0u << (b & 31) : ~0u;
            atomicOr(&S->start[tid], S->cmask[hit][tid] & keep);
          }
          in_exit = uni32(S->cexit[hit]);
          break;
        }
        if (tid == 0) atomicOr(&S->start[(p - t0) >> 5], 1u << ((p - t0) & 31));
        const Matcher<WinAcc> m{wacc, p};
        uint64_t e = uni64(m.piece_end());
        if (uni32((uint32_t)m.a.far)) {
          const CoopAcc acc{S, lo, text, n, doc_limit(doc_off, n_docs, n, p)};
          const Matcher<CoopAcc> mc{acc, p};
          e = uni64(mc.piece_end());
        }
        p = e > p ? e : p + 1;
        if ((int64_t)p >= t1 || is_cut(p)) {
          in_exit = p;
          break;
        }
      }
    }
    if ((int64_t)first_cut == t1 && tid == 0) publish(B, tile, tag, in_exit);
  }

  if (unit_tab) {  // a unit of BPE also starts where no token can span the boundary
    for (int64_t p = max(t0, (int64_t)1) + tid; p < t1; p += kCaseNT) {
      const int i = (int)(p - lo);
      const uint32_t four = (uint32_t)S->raw[i - 2] | (uint32_t)S->raw[i - 1] << 8 | (uint32_t)S->raw[i] << 16 |
                            (uint32_t)S->raw[i + 1] << 24;  // bytes past either end of the text are 0
      if ((four & 0x808000u) && no_token_spans(unit_tab, four))
        atomicOr(&S->start[(p - t0) >> 5], 1u << ((p - t0) & 31));
    }
  }
  __syncthreads();
  // flag words of the tile's chunks
  for (int c = tid; c < kCaseTile / kChunk; c += kCaseNT)
    if (c0 + c < n_chunks) B.flags[c0 + c] = (uint16_t)(S->start[c >> 1] >> (16 * (c & 1)));
  finish();
}

}  // namespace

void launch_pretok_case(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                        const uint32_t* unit_tab, Bufs b, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t tiles = (uint32_t)((n + kCaseTile - 1) / kCaseTile);
  if (!tiles) return;
  launch_on(pretok_case_kernel, dim3(tiles), dim3(kCaseNT), s, e0, e1, text, n, doc_off, n_docs, unit_tab, b);
}

}  // namespace tok
