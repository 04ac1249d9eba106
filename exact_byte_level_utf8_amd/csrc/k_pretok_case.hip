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
// One workgroup per 1 KiB tile: the tile and 256 bytes on each side are
// loaded into LDS and decoded (code point, letter-case class, CR/LF, space,
// apostrophe, contraction letter, document start).  The tile's own bytes are
// checked as well-formed UTF-8 (Unicode Table 3-7; no sequence may cross a
// document boundary).  The segments that start in the tile are matched, plus
// the one running into the tile from the last cut before it; a segment that
// runs past the loaded window reads the text from global memory.  The
// result is the same flag words as the other families' pre-tokenization:
// bit i of word c set iff byte 16c + i starts a piece, or, ahead of the
// merge stage, a unit of BPE (no token spans the byte pair there).
#include "tok_internal.h"
#include "seg_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"
#include "uniclass_case.inc"

namespace tok {
namespace {

using namespace seg;

constexpr int kCaseNT = 256;
constexpr int kCaseTile = kPretokTile;                     // 1024 bytes
constexpr int kCaseHalo = 256;                             // context bytes on each side
constexpr int kCaseWin = kCaseTile + 2 * kCaseHalo;        // loaded bytes
constexpr uint32_t kNotLead = 0;                           // info of a continuation byte

__device__ inline uint32_t case_class(uint32_t cp) {
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

// Info word of the code point whose bytes are b[0 .. len) (taken as given;
// validation is separate).
__device__ inline uint32_t decode_q(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, uint32_t len) {
  uint32_t cp = b0;
  if (len == 2) cp = ((b0 & 0x1Fu) << 6) | (b1 & 0x3Fu);
  else if (len == 3) cp = ((b0 & 0x0Fu) << 12) | ((b1 & 0x3Fu) << 6) | (b2 & 0x3Fu);
  else if (len == 4) cp = ((b0 & 0x07u) << 18) | ((b1 & 0x3Fu) << 12) | ((b2 & 0x3Fu) << 6) | (b3 & 0x3Fu);
  return make_q(cp, case_class(cp), len, fold_code(cp, case_fold_extra(cp)));
}

// The text as the matcher reads it: decoded info from LDS inside the window,
// decoded from global memory outside it.
struct DevAcc {
  const uint32_t* q;      // info per window byte (LDS)
  int64_t lo;             // absolute position of window byte 0
  const uint8_t* text;
  uint64_t n;
  const uint64_t* doc_off;
  uint32_t n_docs;

  __device__ __forceinline__ uint32_t global_q(uint64_t p) const {
    const uint32_t b0 = text[p];
    if ((b0 & 0xC0u) == 0x80u) return kNotLead;
    const uint32_t len = seq_len(b0);
    const uint32_t b1 = len > 1 && p + 1 < n ? text[p + 1] : 0u;
    const uint32_t b2 = len > 2 && p + 2 < n ? text[p + 2] : 0u;
    const uint32_t b3 = len > 3 && p + 3 < n ? text[p + 3] : 0u;
    uint32_t v = decode_q(b0, b1, b2, b3, len);
    if (doc_off) {
      const uint32_t d = first_doc_at_or_after(doc_off, n_docs, p);
      if (d <= n_docs && doc_off[d] == p) v |= kQDocStart;
    } else if (p == 0) {
      v |= kQDocStart;
    }
    return v;
  }

  // info of the code point at byte p
  __device__ __forceinline__ uint32_t at(uint64_t p) const {
    if (p >= n) return kQEnd;
    const int64_t i = (int64_t)p - lo;
    if (i >= 0 && i < kCaseWin - 4) return q[i];
    return global_q(p);
  }
};

__global__ void __launch_bounds__(kCaseNT)
pretok_case_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off,
                   uint32_t n_docs, const uint32_t* __restrict__ joinable, Bufs B) {
  __shared__ uint8_t s_raw[kCaseWin + 4];
  __shared__ uint8_t s_ds[kCaseWin];        // a document starts at this byte
  __shared__ uint32_t s_q[kCaseWin];        // info per window byte
  __shared__ uint32_t s_cut[kCaseTile / 32];    // cut bit per tile byte
  __shared__ uint32_t s_start[kCaseTile / 32];  // piece-start bit per tile byte
  __shared__ uint32_t s_seg[kCaseTile + 1];     // segment starts (byte positions)
  __shared__ uint32_t s_nseg, s_doc0, s_bad;

  if (B.n_docs_dev) n_docs = *B.n_docs_dev;
  const uint32_t tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kCaseTile;
  const int64_t lo = t0 - kCaseHalo;
  const int64_t t1 = min((int64_t)n, t0 + kCaseTile);
  // per-call set-up for the later passes: clear the group sums of the tile
  // counts, and check the batch's document offsets
  if (tid == 0) {
    const uint32_t tiles = gridDim.x;
    if (blockIdx.x < ((tiles + 63u) >> kSum1Shift)) B.sum1[blockIdx.x] = 0;
    if (blockIdx.x < ((tiles + 4095u) >> kSum2Shift)) B.sum2[blockIdx.x] = 0;
    if (doc_off && blockIdx.x == 0 && (doc_off[0] != 0 || doc_off[n_docs] != n)) report(&B.ctr->err_docs, B.gen);
    s_nseg = 0;
    s_bad = 0;
    s_doc0 = doc_off ? first_doc_at_or_after(doc_off, n_docs, (uint64_t)max(lo, (int64_t)0)) : 0u;
  }
  if (doc_off) {
    bool bad_doc = false;
    for (uint32_t d = blockIdx.x * kCaseNT + tid; d < n_docs; d += gridDim.x * kCaseNT)
      bad_doc |= doc_off[d] > doc_off[d + 1];
    if (bad_doc) report(&B.ctr->err_docs, B.gen);
  }
  for (int i = tid; i < kCaseWin; i += kCaseNT) {
    const int64_t p = lo + i;
    s_raw[i] = p >= 0 && p < (int64_t)n ? text[p] : 0;
    s_ds[i] = 0;
  }
  if (tid < 4) s_raw[kCaseWin + tid] = 0;
  for (int i = tid; i < kCaseTile / 32; i += kCaseNT) {
    s_cut[i] = 0;
    s_start[i] = 0;
  }
  __syncthreads();
  // document starts inside the window
  if (doc_off) {
    for (uint32_t d = s_doc0 + tid; d <= n_docs; d += kCaseNT) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= lo + kCaseWin || p >= n) break;
      if ((int64_t)p >= lo) s_ds[p - lo] = 1;
    }
  } else if (lo <= 0 && tid == 0) {
    s_ds[-lo] = 1;
  }
  __syncthreads();
  // decode every window byte
  for (int i = tid; i < kCaseWin; i += kCaseNT) {
    const int64_t p = lo + i;
    uint32_t v = kQEnd;
    if (p >= 0 && p < (int64_t)n) {
      const uint32_t b0 = s_raw[i];
      if ((b0 & 0xC0u) == 0x80u) {
        v = kNotLead;
      } else {
        const uint32_t len = seq_len(b0);
        v = decode_q(b0, s_raw[i + 1], s_raw[i + 2], s_raw[i + 3], len);
        if (s_ds[i]) v |= kQDocStart;
      }
    }
    s_q[i] = v;
  }
  // well-formed UTF-8 over the tile's own bytes (Unicode Table 3-7): a lead
  // is ASCII or C2..F4 with the right continuation bytes, all in its
  // document; a continuation byte belongs to a lead at most 3 bytes before
  // it in the same document
  for (int64_t p = t0 + tid; p < t1; p += kCaseNT) {
    const int i = (int)(p - lo);
    const uint32_t b0 = s_raw[i];
    bool bad = false;
    if ((b0 & 0xC0u) == 0x80u) {
      if (s_ds[i]) {
        bad = true;
      } else {
        int k = 1;
        while (k <= 3 && (s_raw[i - k] & 0xC0u) == 0x80u && !s_ds[i - k]) ++k;
        const uint32_t lead = s_raw[i - k];
        bad = k > 3 || lo + i - k < 0 || (lead & 0xC0u) == 0x80u || lead < 0xC2u || lead > 0xF4u ||
              (int)seq_len(lead) <= k;
      }
    } else if (b0 >= 0x80u) {
      const uint32_t len = seq_len(b0);
      bad = b0 < 0xC2u || b0 > 0xF4u || p + (int64_t)len > (int64_t)n;
      for (uint32_t k = 1; k < len && !bad; ++k) bad = (s_raw[i + k] & 0xC0u) != 0x80u || s_ds[i + k];
      if (!bad && len > 2) {
        const uint32_t b1 = s_raw[i + 1];
        bad = (b0 == 0xE0u && b1 < 0xA0u) || (b0 == 0xEDu && b1 > 0x9Fu) || (b0 == 0xF0u && b1 < 0x90u) ||
              (b0 == 0xF4u && b1 > 0x8Fu);
      }
    }
    if (bad) s_bad = 1;
  }
  __syncthreads();
  const uint64_t c0 = (uint64_t)blockIdx.x * (kCaseTile / kChunk);
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  if (s_bad) {  // uniform: the call reports malformed input; the flags are zero
    if (tid == 0) report(&B.ctr->err_utf8, B.gen);
    for (int c = tid; c < kCaseTile / kChunk; c += kCaseNT)
      if (c0 + c < n_chunks) B.flags[c0 + c] = 0;
    return;
  }

  // cuts at the tile's code points, and the segments that start at them
  for (int64_t p = t0 + tid; p < t1; p += kCaseNT) {
    const int i = (int)(p - lo);
    const uint32_t v = s_q[i];
    if (v == kNotLead) continue;
    bool cut = p == 0 || (v & kQDocStart);
    if (!cut) {
      // the previous lead is at most 3 bytes back in well-formed text; the
      // bound keeps a malformed halo (reported by its own tile) in the window
      int k = 1;
      while (k < i && s_q[i - k] == kNotLead) ++k;
      cut = sync_at(s_q[i - k], v);
    }
    if (cut) {
      atomicOr(&s_cut[(p - t0) >> 5], 1u << ((p - t0) & 31));
      s_seg[atomicAdd(&s_nseg, 1u)] = (uint32_t)p;
    }
  }
  const DevAcc acc{s_q, lo, text, n, doc_off, n_docs};
  __syncthreads();
  // the segment running into the tile: from the last cut at or before the
  // tile's first code point (walking back, through global memory if the
  // cut lies before the window)
  if (tid == 0) {
    int64_t f = t0;
    while (f < t1 && s_q[f - lo] == kNotLead) ++f;
    if (f < t1 && !((s_cut[(f - t0) >> 5] >> ((f - t0) & 31)) & 1u)) {
      uint64_t j = (uint64_t)f;
      uint32_t vj = s_q[f - lo];
      for (;;) {
        if (j == 0 || (vj & kQDocStart)) break;
        uint64_t k = j - 1;
        while (k > 0 && ((int64_t)k - lo >= 0 && (int64_t)k - lo < kCaseWin ? s_q[k - lo] == kNotLead
                                                                           : (text[k] & 0xC0u) == 0x80u))
          --k;
        const uint32_t vk = acc.at(k);
        if (sync_at(vk, vj)) break;
        j = k;
        vj = vk;
      }
      s_seg[s_nseg] = (uint32_t)j;
      s_nseg = s_nseg + 1;
    }
  }
  __syncthreads();

  // every segment from its cut, one per thread: the pieces until the next
  // cut or the tile's end
  const uint32_t nseg = s_nseg;
  for (uint32_t k = tid; k < nseg; k += kCaseNT) {
    uint64_t p = s_seg[k];
    for (;;) {
      if ((int64_t)p >= t0) atomicOr(&s_start[(p - t0) >> 5], 1u << ((p - t0) & 31));
      const Matcher<DevAcc> m{acc, p};
      const uint64_t e = m.piece_end();
      p = e > p ? e : p + 1;  // a match always advances; the guard keeps the loop finite regardless
      if ((int64_t)p >= t1) break;
      if ((int64_t)p >= t0 && ((s_cut[(p - t0) >> 5] >> ((p - t0) & 31)) & 1u)) break;
    }
  }
  if (joinable) {  // a unit of BPE also starts where no token spans the byte pair
    for (int64_t p = max(t0, (int64_t)1) + tid; p < t1; p += kCaseNT) {
      const int i = (int)(p - lo);
      if (((s_raw[i - 1] | s_raw[i]) & 0x80u) && !pair_joinable(joinable, s_raw[i - 1], s_raw[i]))
        atomicOr(&s_start[(p - t0) >> 5], 1u << ((p - t0) & 31));
    }
  }
  __syncthreads();
  // flag words of the tile's chunks
  for (int c = tid; c < kCaseTile / kChunk; c += kCaseNT)
    if (c0 + c < n_chunks) B.flags[c0 + c] = (uint16_t)(s_start[c >> 1] >> (16 * (c & 1)));
}

}  // namespace

void launch_pretok_case(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                        const uint32_t* joinable, Bufs b, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t tiles = (uint32_t)((n + kCaseTile - 1) / kCaseTile);
  if (!tiles) return;
  launch_on(pretok_case_kernel, dim3(tiles), dim3(kCaseNT), s, e0, e1, text, n, doc_off, n_docs, joinable, b);
}

}  // namespace tok
