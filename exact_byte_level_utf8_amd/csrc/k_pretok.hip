// Pre-tokenization kernel: UTF-8 decode and validation, character classes,
// run aggregates and the piece-start predicate, one 1 KiB tile per workgroup.
//
// Each workgroup loads its tile plus 64 bytes of context on each side into LDS
// with coalesced byte loads, decodes every code point once into an info word
// (class and the few character flags the rules test), and evaluates the
// run-local rules of pretok_rules.h at every code point of the tile (TokTier,
// "Exact GPU Tokenization"; GraphTok, section 4 "Parallel tokenizer
// frontends").  Positions are dealt to lanes interleaved (position j * 256 +
// thread), so a wave touches 64 consecutive LDS entries at every step and a
// wave ballot yields four flag words at once: bit i of word c is set iff byte
// 16c + i starts a piece.
//
// The Llama-3 style needs three run aggregates whose runs may cross the tile
// edge.  They are (reset, value) scan elements: four workgroup scans in
// position order combine the tile's elements, and the carry into the tile is
// found by walking the LDS halo; a run longer than the halo (a long digit or
// whitespace run) falls back to reducing 4 KiB blocks from global memory until
// the run ends, which costs time only on such input and keeps the result
// exact.
#include "tok_internal.h"
#include "pretok_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"

namespace tok {
namespace {

constexpr int kPT = kPretokTile;          // tile bytes
constexpr int kWin = kPT + 2 * kHalo;     // LDS window bytes
constexpr int kRounds = kPT / kThreads;   // tile positions per thread
constexpr int kWinRounds = (kWin + kThreads - 1) / kThreads;
// per-byte flags in LDS
constexpr uint8_t kBDoc = 1, kBOut = 2;

__device__ inline uint32_t dev_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
  if (cp < 0x10000) return (kClsBmp[cp >> 2] >> (2 * (cp & 3u))) & 3u;
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
#pragma unroll
  for (int i = 0; i < 20; ++i) {
    const int64_t p = x + i;
    b[i] = (p >= 0 && p < (int64_t)n) ? text[p] : 0u;
    if (p >= (int64_t)n) edge |= 1u << i;
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

// previous code point's lead index in the window, same document, or -1
__device__ inline int prev_lead(const uint32_t* info, const uint8_t* fl, int k) {
  if (k < 0 || (fl[k] & kBDoc)) return -1;
  int j = k - 1;
  for (int t = 0; t < 4 && j >= 0; ++t, --j) {
    if (fl[j] & kBOut) return -1;
    if (info[j] & kILead) return j;
  }
  return -1;
}

__device__ inline uint32_t info_at(const uint32_t* info, int k) { return k < 0 ? kNone : info[k]; }

template <int PATTERN>
__global__ void __launch_bounds__(kThreads)
pretok_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off,
              uint32_t n_docs, Bufs B) {
  __shared__ uint8_t s_raw[kWin + 4];
  __shared__ uint8_t s_fl[kWin + 4];
  __shared__ uint32_t s_info[kWin];
  __shared__ uint32_t s_scan[kThreads / kWave];
  __shared__ uint32_t s_misc[4];

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
    for (uint32_t d = blockIdx.x * kThreads + tid; d < n_docs; d += gridDim.x * kThreads)
      bad_doc |= doc_off[d] > doc_off[d + 1];
    if (bad_doc) report(&B.ctr->err_docs, B.gen);
  }
  const int64_t lo = base - kHalo;
  const int64_t sn = (int64_t)n;

  for (int k = tid; k < kWin + 4; k += kThreads) {
    const int64_t p = lo + k;
    const bool in = p >= 0 && p < sn;
    s_raw[k] = in ? text[p] : 0;
    s_fl[k] = in ? 0 : kBOut;
  }
  if (doc_off && tid == 0) s_misc[0] = first_doc_at_or_after(doc_off, n_docs, lo < 0 ? 0 : (uint64_t)lo);
  __syncthreads();
  if (doc_off) {
    for (uint32_t d = s_misc[0] + tid; d <= n_docs; d += kThreads) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= lo + kWin) break;
      if ((int64_t)p >= lo && (int64_t)p < sn) s_fl[p - lo] |= kBDoc;  // equal offsets write equal bytes
    }
  } else if (tid == 0 && lo <= 0 && sn > 0) {
    s_fl[-lo] |= kBDoc;
  }
  __syncthreads();

  // decode every lead byte of the window; all class lookups of a thread are
  // issued before any is used
  {
    uint32_t cps[kWinRounds], lens[kWinRounds], pre[kWinRounds];
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) {
      const int k = tid + j * kThreads;
      cps[j] = 0;
      lens[j] = 0;
      pre[j] = 0;
      if (k < kWin) {
        const uint8_t fl = s_fl[k];
        const uint32_t b = s_raw[k];
        if (!(fl & kBOut) && (b & 0xC0) != 0x80) {
          const uint32_t len = utf8_len(b);
          lens[j] = len;
          pre[j] = kILead | ((fl & kBDoc) ? kIDocStart : 0u);
          if (k + (int)len >= kWin) {
            pre[j] |= kIUndecoded;
          } else {
            cps[j] = utf8_cp(b, s_raw[k + 1], s_raw[k + 2], s_raw[k + 3], len);
            if (s_fl[k + len] & (kBDoc | kBOut)) pre[j] |= kILastInDoc;
          }
        }
      }
    }
    uint32_t cls[kWinRounds];
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) cls[j] = dev_class(cps[j]);
#pragma unroll
    for (int j = 0; j < kWinRounds; ++j) {
      const int k = tid + j * kThreads;
      if (k >= kWin) continue;
      uint32_t in = 0;
      if (pre[j] & kIUndecoded) in = kO | (lens[j] << kILenShift) | pre[j];
      else if (pre[j]) in = make_info(cps[j], cls[j], lens[j], dev_fold_extra(cps[j])) | pre[j];
      s_info[k] = in;
    }
  }

  // UTF-8 validation of the tile's own bytes (Unicode Table 3-7, well-formed
  // byte sequences); a sequence may not cross a document boundary
  bool bad = false;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int k = kHalo + tid + j * kThreads;
    if (s_fl[k] & kBOut) continue;
    const uint32_t b = s_raw[k];
    if (b < 0x80) continue;
    if ((b & 0xC0) == 0x80) {
      if (s_fl[k] & kBDoc) { bad = true; continue; }
      bool ok = false;
      for (int steps = 1; steps <= 3; ++steps) {
        const int jj = k - steps;
        if (s_fl[jj] & kBOut) break;
        const uint32_t rb = s_raw[jj];
        if ((rb & 0xC0) != 0x80) {
          ok = rb >= 0xC0 && utf8_len(rb) > (uint32_t)steps;
          break;
        }
        if (s_fl[jj] & kBDoc) break;
      }
      bad |= !ok;
    } else {
      if (b < 0xC2 || b > 0xF4) { bad = true; continue; }
      const uint32_t len = utf8_len(b);
      for (uint32_t t = 1; t < len; ++t) {
        const int jj = k + t;
        if ((s_fl[jj] & (kBOut | kBDoc)) || (s_raw[jj] & 0xC0) != 0x80) bad = true;
      }
      const uint32_t c1 = s_raw[k + 1];
      if ((b == 0xE0 && c1 < 0xA0) || (b == 0xED && c1 > 0x9F) || (b == 0xF0 && c1 < 0x90) ||
          (b == 0xF4 && c1 > 0x8F))
        bad = true;
    }
  }
  if (bad) report(&B.ctr->err_utf8, B.gen);
  __syncthreads();

  // Llama-3 style: run-aggregate states before (forward) and after (backward)
  // every tile position
  uint32_t fst[kRounds], hst[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) fst[j] = hst[j] = 0;
  if (PATTERN == 1) {
    if (tid == 0) {  // walk left through the halo until both forward aggregates reset
      uint32_t acc = kFwdId, done = 0;
      for (int k = kHalo - 1; k >= 0; --k) {
        if (s_fl[k] & kBOut) { done = 1; break; }
        const uint32_t in = s_info[k];
        if (in & kILead) {
          acc = fwd_comp(fwd_elem(in), acc);
          if (fwd_resolved(acc)) { done = 1; break; }
        }
      }
      s_misc[1] = fwd_apply(acc, 0);
      s_misc[2] = done;
    }
    if (tid == kWave) {  // walk right until the backward aggregate resets
      uint32_t acc = kBwdId, done = 0;
      for (int k = kHalo + kPT; k < kWin; ++k) {
        if (s_fl[k] & kBOut) { done = 1; break; }
        const uint32_t in = s_info[k];
        if (in & kILead) {
          if (in & kIUndecoded) break;
          acc = bwd_comp(acc, bwd_elem(in));
          if (acc & 1u) { done = 1; break; }
        }
      }
      s_misc[3] = bwd_apply(acc, 0) | (done << 1);
    }
    __syncthreads();
    uint32_t carry_f = __builtin_amdgcn_readfirstlane(s_misc[1]);
    const bool fdone = __builtin_amdgcn_readfirstlane(s_misc[2]) != 0;
    const uint32_t m3 = __builtin_amdgcn_readfirstlane(s_misc[3]);
    uint32_t carry_h = m3 & 1u;
    const bool bdone = (m3 >> 1) & 1u;
    __syncthreads();
    if (!fdone) {  // a run longer than the halo ends before the tile: reduce 4 KiB blocks
      uint32_t acc = kFwdId;
      for (int64_t end = base;; end -= kThreads * kChunk) {
        const int64_t start = end - kThreads * kChunk;
        uint32_t fe, be;
        chunk_elems_global(text, n, doc_off, n_docs, start + (int64_t)tid * kChunk, &fe, &be);
        uint32_t tot;
        wg_excl_scan<kThreads>(fe, kFwdId, FwdOp(), s_scan, &tot);
        acc = __builtin_amdgcn_readfirstlane(fwd_comp(tot, acc));  // uniform loop exit
        if (fwd_resolved(acc) || start <= 0) break;
      }
      carry_f = fwd_apply(acc, 0);
    }
    if (!bdone) {
      uint32_t acc = kBwdId;
      for (int64_t start = base + kPT;; start += kThreads * kChunk) {
        uint32_t fe, be;
        chunk_elems_global(text, n, doc_off, n_docs, start + (int64_t)tid * kChunk, &fe, &be);
        uint32_t tot;
        wg_excl_suffix<kThreads>(be, kBwdId, BwdOp(), s_scan, &tot);
        acc = __builtin_amdgcn_readfirstlane(bwd_comp(acc, tot));  // uniform loop exit
        if ((acc & 1u) || start + kThreads * kChunk >= sn) break;
      }
      carry_h = bwd_apply(acc, 0);
    }
    // forward: rounds in position order; backward: rounds in reverse order
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const uint32_t in = s_info[kHalo + tid + j * kThreads];
      uint32_t tot;
      const uint32_t pre = wg_excl_scan<kThreads>((in & kILead) ? fwd_elem(in) : kFwdId, kFwdId, FwdOp(),
                                                  s_scan, &tot);
      fst[j] = fwd_apply(pre, carry_f);
      carry_f = fwd_apply(tot, carry_f);
    }
#pragma unroll
    for (int j = kRounds - 1; j >= 0; --j) {
      const uint32_t in = s_info[kHalo + tid + j * kThreads];
      uint32_t tot;
      const uint32_t suf = wg_excl_suffix<kThreads>((in & kILead) ? bwd_elem(in) : kBwdId, kBwdId, BwdOp(),
                                                    s_scan, &tot);
      hst[j] = bwd_apply(suf, carry_h);
      carry_h = bwd_apply(tot, carry_h);
    }
  }

#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int k = kHalo + tid + j * kThreads;
    const uint32_t c = s_info[k];
    bool st = false;
    if (c & kILead) {
      const int j1 = prev_lead(s_info, s_fl, k);
      const int j2 = prev_lead(s_info, s_fl, j1);
      const int j3 = prev_lead(s_info, s_fl, j2);
      const int j4 = prev_lead(s_info, s_fl, j3);
      const uint32_t p1 = info_at(s_info, j1), p2 = info_at(s_info, j2);
      const uint32_t p3 = info_at(s_info, j3), p4 = info_at(s_info, j4);
      const uint32_t len = (c >> kILenShift) & 7u;
      const uint32_t n1 = (c & kILastInDoc) ? kNone : s_info[k + len];
      st = PATTERN == 0 ? piece_start_gpt2(c, p1, p2, p3, p4, n1)
                        : piece_start_llama3(c, p1, p2, p3, p4, n1, fst[j] & 3u, (fst[j] >> 2) & 1u,
                                             hst[j] & 1u);
    }
    // this wave holds 64 consecutive positions: four flag words
    const uint64_t m = __ballot(st);
    const uint64_t p0 = (uint64_t)base + (uint64_t)j * kThreads + wv * kWave;
    if (lane < 4) {
      const uint64_t cw = p0 / kChunk + lane;
      if (cw * kChunk < n) flags[cw] = (uint16_t)(m >> (16 * lane));
    }
  }
}

}  // namespace

void launch_pretok(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                   int pattern, Bufs b, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kPretokTile - 1) / kPretokTile);
  if (!tiles) return;
  if (pattern == 0)
    pretok_kernel<0><<<tiles, kThreads, 0, s>>>(text, n, doc_off, n_docs, b);
  else
    pretok_kernel<1><<<tiles, kThreads, 0, s>>>(text, n, doc_off, n_docs, b);
}

}  // namespace tok
