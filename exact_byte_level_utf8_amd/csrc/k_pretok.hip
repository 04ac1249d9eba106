// Pre-tokenization kernel: UTF-8 decode and validation, character classes,
// run aggregates and the piece-start predicate, one 4 KiB tile per workgroup.
//
// Each workgroup loads its tile plus 64 bytes of context on each side into LDS
// with coalesced byte loads, decodes every code point once into an info word
// (class and the few character flags the rules test), and then evaluates the
// run-local rules of pretok_rules.h at every code point of the tile (TokTier,
// "Exact GPU Tokenization"; GraphTok, section 4 "Parallel tokenizer
// frontends").  The output is one 16-bit flag word per 16-byte chunk: bit i
// set iff byte 16c + i starts a piece.
//
// The Llama-3 style needs three run aggregates whose runs may cross the tile
// edge.  They are (reset, value) scan elements: a workgroup scan combines the
// per-thread chunks, and the carry into the tile is found by walking the LDS
// halo; a run longer than the halo (a long digit or whitespace run) falls back
// to reducing whole 4 KiB blocks from global memory until the run ends, which
// costs time only on such input and keeps the result exact.
#include "tok_internal.h"
#include "pretok_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"

namespace tok {
namespace {

constexpr int kWin = kTile + 2 * kHalo;
// per-byte flags in LDS
constexpr uint8_t kBDoc = 1, kBOut = 2;

// Padded LDS indexing.  Each thread walks 16 consecutive positions, so lanes
// touch positions 16 apart; one pad word per 16 info words and four pad bytes
// per 16 bytes spread those lanes over distinct banks.
__device__ inline int IX(int k) { return k + (k >> 4); }
__device__ inline int BX(int k) { return k + ((k >> 4) << 2); }
constexpr int kWinI = kWin + kWin / 16 + 1;
constexpr int kWinB = kWin + 4 * (kWin / 16) + 4;

__device__ inline uint32_t dev_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
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

// Code point of the sequence at b[0..len); continuation bits are taken as
// they are (validation is separate).
__device__ inline uint32_t utf8_cp(const uint8_t* b, uint32_t len) {
  uint32_t cp = len == 1 ? b[0] : len == 2 ? (b[0] & 0x1Fu) : len == 3 ? (b[0] & 0x0Fu) : (b[0] & 0x07u);
  for (uint32_t k = 1; k < len; ++k) cp = (cp << 6) | (b[k] & 0x3Fu);
  return cp;
}

// First index d in [0, n_docs] with doc_off[d] >= x (n_docs + 1 if none).
__device__ inline uint32_t first_doc_at_or_after(const uint64_t* doc_off, uint32_t n_docs, uint64_t x) {
  uint32_t lo = 0, hi = n_docs + 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (doc_off[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Scan elements of the code points whose lead byte lies in [x, x + 16), read
// from global memory (slow path for runs longer than the halo).
__device__ void chunk_elems_global(const uint8_t* text, uint64_t n, const uint64_t* doc_off,
                                   uint32_t n_docs, int64_t x, uint32_t* fe, uint32_t* be) {
  uint8_t b[20];
  uint32_t edge = 0;  // bit i: a document starts at x + i, or x + i >= n
  for (int i = 0; i < 20; ++i) {
    const int64_t p = x + i;
    b[i] = (p >= 0 && p < (int64_t)n) ? text[p] : 0;
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
  for (int i = 0; i < kChunk; ++i) {
    const int64_t p = x + i;
    if (p < 0 || p >= (int64_t)n || (b[i] & 0xC0) == 0x80) continue;
    const uint32_t len = utf8_len(b[i]);
    const uint32_t cp = utf8_cp(b + i, len);
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
  if (k < 0 || (fl[BX(k)] & kBDoc)) return -1;
  int j = k - 1;
  for (int t = 0; t < 4 && j >= 0; ++t, --j) {
    if (fl[BX(j)] & kBOut) return -1;
    if (info[IX(j)] & kILead) return j;
  }
  return -1;
}

__device__ inline uint32_t info_at(const uint32_t* info, int k) { return k < 0 ? kNone : info[IX(k)]; }

template <int PATTERN>
__global__ void __launch_bounds__(kThreads)
pretok_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off,
              uint32_t n_docs, uint16_t* __restrict__ flags, Counters* __restrict__ ctr) {
  __shared__ uint8_t s_raw[kWinB];
  __shared__ uint8_t s_fl[kWinB];
  __shared__ uint32_t s_info[kWinI];
  __shared__ uint32_t s_scan[kThreads / kWave];
  __shared__ uint32_t s_misc[4];

  const uint32_t tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kTile;
  const int64_t lo = base - kHalo;
  const int64_t sn = (int64_t)n;

  for (int k = tid; k < kWin; k += kThreads) {
    const int64_t p = lo + k;
    const bool in = p >= 0 && p < sn;
    s_raw[BX(k)] = in ? text[p] : 0;
    s_fl[BX(k)] = in ? 0 : kBOut;
  }
  if (doc_off && tid == 0) s_misc[0] = first_doc_at_or_after(doc_off, n_docs, lo < 0 ? 0 : (uint64_t)lo);
  __syncthreads();
  if (doc_off) {
    for (uint32_t d = s_misc[0] + tid; d <= n_docs; d += kThreads) {
      const uint64_t p = doc_off[d];
      if ((int64_t)p >= lo + kWin) break;
      if ((int64_t)p >= lo && (int64_t)p < sn) s_fl[BX(p - lo)] |= kBDoc;  // equal offsets write equal bytes
    }
  } else if (tid == 0 && lo <= 0 && sn > 0) {
    s_fl[BX(-lo)] |= kBDoc;
  }
  __syncthreads();

  // decode every lead byte of the window into an info word
  for (int k = tid; k < kWin; k += kThreads) {
    const uint8_t fl = s_fl[BX(k)];
    uint32_t in = 0;
    const uint32_t b = s_raw[BX(k)];
    if (!(fl & kBOut) && (b & 0xC0) != 0x80) {
      const uint32_t len = utf8_len(b);
      if (k + (int)len >= kWin) {
        in = kO | kILead | kIUndecoded | (len << kILenShift);
      } else {
        uint8_t sb[4];
        for (uint32_t t = 0; t < 4; ++t) sb[t] = t < len ? s_raw[BX(k + (int)t)] : 0;
        const uint32_t cp = utf8_cp(sb, len);
        in = make_info(cp, dev_class(cp), len, dev_fold_extra(cp));
        if (s_fl[BX(k + len)] & (kBDoc | kBOut)) in |= kILastInDoc;
      }
      if (fl & kBDoc) in |= kIDocStart;
    }
    s_info[IX(k)] = in;
  }

  // UTF-8 validation of the tile's own bytes (Unicode Table 3-7, well-formed
  // byte sequences); a sequence may not cross a document boundary
  bool bad = false;
  for (int i = 0; i < kChunk; ++i) {
    const int k = kHalo + tid * kChunk + i;
    if (s_fl[BX(k)] & kBOut) break;
    const uint32_t b = s_raw[BX(k)];
    if (b < 0x80) continue;
    if ((b & 0xC0) == 0x80) {
      if (s_fl[BX(k)] & kBDoc) { bad = true; continue; }
      bool ok = false;
      for (int steps = 1; steps <= 3; ++steps) {
        const int j = k - steps;
        if (s_fl[BX(j)] & kBOut) break;
        const uint32_t rb = s_raw[BX(j)];
        if ((rb & 0xC0) != 0x80) {
          ok = rb >= 0xC0 && utf8_len(rb) > (uint32_t)steps;
          break;
        }
        if (s_fl[BX(j)] & kBDoc) break;
      }
      bad |= !ok;
    } else {
      if (b < 0xC2 || b > 0xF4) { bad = true; continue; }
      const uint32_t len = utf8_len(b);
      for (uint32_t t = 1; t < len; ++t) {
        const int j = k + t;
        if ((s_fl[BX(j)] & (kBOut | kBDoc)) || (s_raw[BX(j)] & 0xC0) != 0x80) bad = true;
      }
      const uint32_t c1 = s_raw[BX(k + 1)];
      if ((b == 0xE0 && c1 < 0xA0) || (b == 0xED && c1 > 0x9F) || (b == 0xF0 && c1 < 0x90) ||
          (b == 0xF4 && c1 > 0x8F))
        bad = true;
    }
  }
  if (bad) atomicOr(&ctr->status, kStUtf8);
  __syncthreads();

  // Llama-3 style: carries of the run aggregates into and out of the tile
  uint32_t carry_f = 0, carry_h = 0;
  if (PATTERN == 1) {
    if (tid == 0) {  // walk left through the halo until both forward aggregates reset
      uint32_t acc = kFwdId, done = 0;
      for (int k = kHalo - 1; k >= 0; --k) {
        if (s_fl[BX(k)] & kBOut) { done = 1; break; }
        const uint32_t in = s_info[IX(k)];
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
      for (int k = kHalo + kTile; k < kWin; ++k) {
        if (s_fl[BX(k)] & kBOut) { done = 1; break; }
        const uint32_t in = s_info[IX(k)];
        if (in & kILead) {
          if (in & kIUndecoded) break;
          acc = bwd_comp(acc, bwd_elem(in));
          if (acc & 1u) { done = 1; break; }
        }
      }
      s_misc[3] = bwd_apply(acc, 0) | (done << 1);
    }
    __syncthreads();
    carry_f = __builtin_amdgcn_readfirstlane(s_misc[1]);
    const bool fdone = __builtin_amdgcn_readfirstlane(s_misc[2]) != 0;
    const uint32_t m3 = __builtin_amdgcn_readfirstlane(s_misc[3]);
    carry_h = m3 & 1u;
    const bool bdone = (m3 >> 1) & 1u;
    __syncthreads();
    if (!fdone) {  // a run longer than the halo ends before the tile: reduce 4 KiB blocks
      uint32_t acc = kFwdId;
      for (int64_t end = base;; end -= kTile) {
        const int64_t start = end - kTile;
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
      for (int64_t start = base + kTile;; start += kTile) {
        uint32_t fe, be;
        chunk_elems_global(text, n, doc_off, n_docs, start + (int64_t)tid * kChunk, &fe, &be);
        uint32_t tot;
        wg_excl_suffix<kThreads>(be, kBwdId, BwdOp(), s_scan, &tot);
        acc = __builtin_amdgcn_readfirstlane(bwd_comp(acc, tot));  // uniform loop exit
        if ((acc & 1u) || start + kTile >= sn) break;
      }
      carry_h = bwd_apply(acc, 0);
    }
  }

  // this thread's chunk
  const int k0 = kHalo + tid * kChunk;
  uint32_t fstate = 0, hmask = 0;
  if (PATTERN == 1) {
    uint32_t fe = kFwdId, be = kBwdId;
    for (int i = 0; i < kChunk; ++i) {
      const uint32_t in = s_info[IX(k0 + i)];
      if (in & kILead) {
        fe = fwd_comp(fe, fwd_elem(in));
        be = bwd_comp(be, bwd_elem(in));
      }
    }
    const uint32_t fpre = wg_excl_scan<kThreads>(fe, kFwdId, FwdOp(), s_scan, nullptr);
    const uint32_t bsuf = wg_excl_suffix<kThreads>(be, kBwdId, BwdOp(), s_scan, nullptr);
    fstate = fwd_apply(fpre, carry_f);
    uint32_t h = bwd_apply(bsuf, carry_h);
    for (int i = kChunk - 1; i >= 0; --i) {  // h to the right of each lead
      const uint32_t in = s_info[IX(k0 + i)];
      if (in & kILead) {
        hmask |= h << i;
        h = bwd_apply(bwd_elem(in), h);
      }
    }
  }

  uint32_t word = 0;
  for (int i = 0; i < kChunk; ++i) {
    const int k = k0 + i;
    const uint32_t c = s_info[IX(k)];
    if (!(c & kILead)) continue;
    const int j1 = prev_lead(s_info, s_fl, k);
    const int j2 = prev_lead(s_info, s_fl, j1);
    const int j3 = prev_lead(s_info, s_fl, j2);
    const int j4 = prev_lead(s_info, s_fl, j3);
    const uint32_t p1 = info_at(s_info, j1), p2 = info_at(s_info, j2);
    const uint32_t p3 = info_at(s_info, j3), p4 = info_at(s_info, j4);
    const uint32_t len = (c >> kILenShift) & 7u;
    const uint32_t n1 = (c & kILastInDoc) ? kNone : s_info[IX(k + len)];
    bool st;
    if (PATTERN == 0) {
      st = piece_start_gpt2(c, p1, p2, p3, p4, n1);
    } else {
      st = piece_start_llama3(c, p1, p2, p3, p4, n1, fstate & 3u, (fstate >> 2) & 1u, (hmask >> i) & 1u);
      fstate = fwd_apply(fwd_elem(c), fstate);
    }
    word |= (uint32_t)st << i;
  }
  const uint64_t c = (uint64_t)blockIdx.x * kThreads + tid;
  if (c * kChunk < n) flags[c] = (uint16_t)word;
}

}  // namespace

void launch_pretok(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                   int pattern, Bufs b, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kTile - 1) / kTile);
  if (!tiles) return;
  if (pattern == 0)
    pretok_kernel<0><<<tiles, kThreads, 0, s>>>(text, n, doc_off, n_docs, b.flags, b.ctr);
  else
    pretok_kernel<1><<<tiles, kThreads, 0, s>>>(text, n, doc_off, n_docs, b.flags, b.ctr);
}

}  // namespace tok
