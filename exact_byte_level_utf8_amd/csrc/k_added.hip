// Added-token literals: a leftmost-longest literal pass ahead of the pattern
// (TokTier, section 4 "Single-request path": added and special tokens are
// literal strings reserved as single IDs, extracted by a leftmost-longest pass
// before the tokenizer family handles the remaining segments; GraphTok,
// section 4 "Design": a device lookup first finds the literals, emits their
// IDs directly and passes only the unmatched regions to the family predicate).
//
//   lit_match_kernel   one 1 KiB tile per workgroup, its bytes staged in LDS: at
//                      every byte, the longest literal that starts there (a
//                      256-bit first-byte mask in LDS rejects most bytes at
//                      once; candidates of two or more bytes are grouped by
//                      their first two bytes, longest first, and compared a
//                      word at a time); each tile writes its matches in
//                      position order.
//   lit_select_kernel  one workgroup: the matches of all tiles in order; when
//                      no match overlaps the next one every match is taken,
//                      else one lane keeps, in order, each match that starts at
//                      or after the end of the last one kept (the cursor scan
//                      of the definition, over the matches only).  The taken
//                      literals cut the text into 2k + 1 parts: segment,
//                      literal, segment, ..., segment.
// The parts then run through the usual pipeline as documents (their count
// read on the device, so the host enqueues everything without waiting),
// which are hard boundaries for code points, pieces and merges, exactly as
// the segments between literals must be.  Then:
//   lit_insert_kernel  one workgroup: output offsets of the parts, where a
//                      literal part counts one ID; writes the literal IDs.
//   lit_scatter_kernel every ID of a segment part to its final place; the IDs
//                      the pipeline made from a literal's own bytes are dropped.
// With span export the pipeline also gives each segment token's first byte
// (counted from the start of the text, as the parts are), the literal's first
// byte goes with its ID, and the scatter moves both.
#include "ext_internal.h"
#include "wg_scan.h"

namespace tok {
namespace {

constexpr uint32_t kMatchThreads = 256;  // 4 consecutive positions per thread
constexpr uint32_t kSelThreads = 1024;
constexpr uint32_t kScatterThreads = 256;
constexpr uint32_t kInsPer = 4;  // parts per thread in one pass of the insertion

__device__ inline uint32_t lit_len(const Literals& L, uint32_t li) { return L.off[li + 1] - L.off[li]; }

// Bytes b .. b + 3 of a byte array held as words (little endian), from two
// aligned word reads.
__device__ inline uint32_t bytes_at(const uint32_t* w, uint32_t b) {
  return __builtin_amdgcn_alignbyte(w[(b >> 2) + 1], w[b >> 2], b & 3u);
}

// The longest literal that starts at byte p of text[0, n) and ends by the end
// of p's document, or -1.  b0: the byte at p; q: p's byte in the tile's LDS
// copy s_text (the tile plus the longest literal's reach).  The literal's
// bytes are compared a word at a time, every load issued at once.
__device__ inline int32_t literal_at(const uint32_t* s_text, uint32_t q, uint32_t b0, uint64_t n, uint64_t p,
                                     const Literals& L, const uint64_t* __restrict__ doc_off, uint32_t n_docs) {
  uint64_t lim = n;  // a literal never reaches into the next document
  if (doc_off) {
    const uint32_t d = first_doc_at_or_after(doc_off, n_docs, p + 1);
    if (d <= n_docs) lim = min(lim, doc_off[d]);
  }
  if (p + 1 < lim) {
    const uint32_t b1 = (bytes_at(s_text, q) >> 8) & 0xFFu;
    const uint32_t e = L.key2[b0 | (b1 << 8)];
    const uint32_t start = e >> 16, cnt = e & 0xFFFFu;
    const uint32_t* blob = reinterpret_cast<const uint32_t*>(L.bytes);  // word-aligned, padded past its end
    for (uint32_t c = 0; c < cnt; ++c) {  // longest first: the first full match is the longest
      const uint32_t li = L.order[start + c];
      const uint32_t a = L.off[li], len = L.off[li + 1] - a;
      if (p + len > lim) continue;
      const uint32_t w0 = a >> 2, sh = a & 3u;
      bool eq = true;
#pragma unroll
      for (uint32_t j = 0; j < (uint32_t)kLitMax / 4; ++j) {
        if (4 * j < len) {
          const uint32_t lw = __builtin_amdgcn_alignbyte(blob[w0 + j + 1], blob[w0 + j], sh);
          const uint32_t rem = len - 4 * j;
          const uint32_t mask = rem >= 4 ? 0xFFFFFFFFu : (1u << (8 * rem)) - 1u;
          eq &= ((lw ^ bytes_at(s_text, q + 4 * j)) & mask) == 0;
        }
      }
      if (eq) return (int32_t)li;
    }
  }
  return L.key1[b0];
}

__global__ void __launch_bounds__(kMatchThreads)
lit_match_kernel(const uint8_t* __restrict__ text, uint64_t n, const uint64_t* __restrict__ doc_off, uint32_t n_docs,
                 Literals L, LitBufs lb) {
  // the tile's bytes, the longest literal's reach past it, and a guard word
  constexpr uint32_t kWords = (kLitTile + kLitMax + 8) / 4;
  __shared__ uint32_t s_text[kWords];
  __shared__ uint32_t s_first[8];
  __shared__ uint32_t s_scan[kMatchThreads / kWave];
  const uint32_t tile = blockIdx.x, tid = threadIdx.x;
  const uint64_t base = (uint64_t)tile * kLitTile;
  {
    const bool aligned = (reinterpret_cast<uintptr_t>(text) & 3u) == 0;
    for (uint32_t w = tid; w < kWords; w += kMatchThreads) {
      const uint64_t p = base + 4u * w;
      uint32_t v = 0;
      if (aligned && p + 4 <= n) {
        v = *reinterpret_cast<const uint32_t*>(text + p);
      } else {
        for (uint32_t i = 0; i < 4; ++i)
          if (p + i < n) v |= (uint32_t)text[p + i] << (8 * i);
      }
      s_text[w] = v;
    }
    if (tid < 8) s_first[tid] = L.first[tid];
  }
  __syncthreads();
  const uint64_t p0 = base + 4u * tid;
  const uint32_t cur = s_text[tid];
  int32_t m[4];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b0 = (cur >> (8 * j)) & 0xFFu;
    const bool cand = p0 + j < n && ((s_first[b0 >> 5] >> (b0 & 31u)) & 1u);
    m[j] = cand ? literal_at(s_text, 4u * tid + j, b0, n, p0 + j, L, doc_off, n_docs) : -1;
    c += m[j] >= 0 ? 1u : 0u;
  }
  uint32_t tot = 0;
  uint32_t at = wg_excl_scan<kMatchThreads>(c, 0u, AddOp(), s_scan, &tot);
  uint64_t* out = lb.cand + (uint64_t)tile * kLitTile;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (m[j] >= 0) out[at++] = ((p0 + j) << 32) | (uint32_t)m[j];
  if (tid == 0) lb.tile_cnt[tile] = tot;
}

__global__ void __launch_bounds__(kSelThreads)
lit_select_kernel(uint64_t n, uint32_t tiles, const uint64_t* __restrict__ doc_off, uint32_t n_docs, Literals L,
                  LitBufs lb, Counters* ctr, uint64_t gen) {
  __shared__ uint32_t s_scan[kSelThreads / kWave];
  __shared__ uint32_t s_over, s_kept, s_bad;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    s_over = 0;
    s_bad = 0;
  }
  // the caller's documents (one document [0, n) without offsets): the
  // pipeline sees only the parts, so their offsets are checked here
  const uint32_t nd = doc_off ? n_docs : 1u;
  auto D = [&](uint32_t d) -> uint64_t { return doc_off ? doc_off[d] : (d == 0 ? 0ull : n); };
  bool bad = false;
  for (uint32_t d = tid; d < nd; d += kSelThreads) bad |= D(d) > D(d + 1);
  if (tid == 0) bad |= D(0) != 0 || D(nd) != n;
  // matches before each tile, and each tile's matches copied after them in
  // the same pass (uniform trip count: the scan holds barriers)
  uint32_t carry = 0;
  for (uint32_t t0 = 0; t0 < tiles; t0 += kSelThreads) {
    const uint32_t t = t0 + tid;
    const uint32_t v = t < tiles ? lb.tile_cnt[t] : 0u;
    uint32_t tot = 0;
    const uint32_t b = carry + wg_excl_scan<kSelThreads>(v, 0u, AddOp(), s_scan, &tot);
    for (uint32_t j = 0; j < v; ++j) lb.sel[b + j] = lb.cand[(uint64_t)t * kLitTile + j];
    carry += tot;
  }
  if (bad) s_bad = 1u;
  const uint32_t K = carry;
  __syncthreads();
  bool over = false;
  for (uint32_t i = tid; i + 1 < K; i += kSelThreads) {
    const uint64_t a = lb.sel[i], b = lb.sel[i + 1];
    over |= (a >> 32) + lit_len(L, (uint32_t)a) > (b >> 32);
  }
  if (over) s_over = 1u;
  __syncthreads();
  // malformed offsets: report, and fall back to one part with no literal
  // (the call fails; everything below stays in bounds)
  const bool bad_docs = s_bad != 0;
  uint32_t k = bad_docs ? 0u : K;
  if (!bad_docs && s_over) {  // uniform: LDS words read after a barrier
    if (tid == 0) {
      uint64_t end = 0;
      uint32_t w = 0;
      for (uint32_t i = 0; i < K; ++i) {
        const uint64_t a = lb.sel[i];
        if ((a >> 32) >= end) {
          lb.sel[w++] = a;
          end = (a >> 32) + lit_len(L, (uint32_t)a);
        }
      }
      s_kept = w;
    }
    __syncthreads();
    k = s_kept;
  }
  // cut points: the document boundaries merged with each literal's start and
  // end.  A boundary comes before a literal starting on it and after a
  // literal ending on it; literals never straddle a boundary.
  //   index of start j = 2j + #{d : D(d) <= S_j}
  //   index of end j   = 2j + 1 + #{d : D(d) < E_j}
  //   index of D(d)    = d + 2 #{j : S_j < D(d)}
  const uint32_t nb = bad_docs ? 1u : nd;  // boundaries 0..nb
  auto Db = [&](uint32_t d) -> uint64_t { return bad_docs ? (d == 0 ? 0ull : n) : D(d); };
  const uint32_t parts = nb + 2 * k;
  for (uint32_t i = tid; i < parts; i += kSelThreads) lb.part_lit[i] = -1;
  __syncthreads();
  for (uint32_t j = tid; j < k; j += kSelThreads) {
    const uint64_t a = lb.sel[j];
    const uint64_t S = a >> 32, E = S + lit_len(L, (uint32_t)a);
    uint32_t lo = 0, hi = nb + 1;  // #{d : D(d) <= S}
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (Db(mid) <= S) lo = mid + 1;
      else hi = mid;
    }
    const uint32_t is = 2 * j + lo;
    lo = 0;
    hi = nb + 1;  // #{d : D(d) < E}
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (Db(mid) < E) lo = mid + 1;
      else hi = mid;
    }
    const uint32_t ie = 2 * j + 1 + lo;
    lb.cut[is] = S;
    lb.cut[ie] = E;
    lb.part_lit[is] = (int32_t)j;
  }
  for (uint32_t d = tid; d <= nb; d += kSelThreads) {
    const uint64_t x = Db(d);
    // #{j : S_j < x}: none before the text, all at its end (so one request
    // needs no search), else a binary search over the taken literals
    uint32_t lo = x == 0 ? 0u : x >= n ? k : 0u, hi = x == 0 || x >= n ? lo : k;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if ((lb.sel[mid] >> 32) < x) lo = mid + 1;
      else hi = mid;
    }
    const uint32_t id = d + 2 * lo;
    lb.cut[id] = x;
    lb.doc_part[d] = id;
  }
  if (tid == 0) {
    lb.misc[1] = k;
    lb.misc[2] = parts;  // read by the pipeline as its document count
    lb.misc[3] = nb;
    ctr->lits = k;
    if (bad_docs) report(&ctr->err_docs, gen);
    __threadfence_system();
    report(&ctr->lit_done, gen);
  }
}

__global__ void __launch_bounds__(kSelThreads)
lit_insert_kernel(Literals L, LitBufs lb, int32_t* __restrict__ out, uint32_t* __restrict__ spans, uint64_t cap,
                  uint64_t* __restrict__ out_off, Counters* ctr, uint64_t gen) {
  __shared__ uint32_t s_scan[kSelThreads / kWave];
  const uint32_t tid = threadIdx.x, parts = lb.misc[2], nb = lb.misc[3];
  // kInsPer consecutive parts per thread, so that a pass covers 4,096 parts
  // with all their loads in flight before the one scan
  uint32_t carry = 0;
  for (uint32_t i0 = 0; i0 < parts; i0 += kSelThreads * kInsPer) {
    const uint32_t ib = i0 + tid * kInsPer;
    int32_t lj[kInsPer];
    uint32_t v[kInsPer], sum = 0;
#pragma unroll
    for (uint32_t j = 0; j < kInsPer; ++j) {
      const uint32_t i = ib + j;
      lj[j] = i < parts ? lb.part_lit[i] : -1;
      v[j] = i >= parts ? 0u : lj[j] >= 0 ? 1u : (uint32_t)(lb.out_off[i + 1] - lb.out_off[i]);
      sum += v[j];
    }
    uint32_t tot = 0;
    uint32_t at = carry + wg_excl_scan<kSelThreads>(sum, 0u, AddOp(), s_scan, &tot);
#pragma unroll
    for (uint32_t j = 0; j < kInsPer; ++j) {
      const uint32_t i = ib + j;
      if (i < parts) {
        lb.fin[i] = at;
        if (lj[j] >= 0 && at < cap) {
          out[at] = L.ids[(uint32_t)lb.sel[lj[j]]];
          if (spans) spans[at] = (uint32_t)lb.cut[i];  // the literal starts its part
        }
      }
      at += v[j];
    }
    carry += tot;
  }
  if (tid == 0) lb.fin[parts] = carry;
  // for the scatter: the part holding pipeline token 256 b, for every b (the
  // parts tile the tokens, so each b is written once); the candidate buffer is
  // free by now and holds it
  if (parts > 1) {
    uint32_t* blk = reinterpret_cast<uint32_t*>(lb.cand);
    for (uint32_t i = tid; i < parts; i += kSelThreads) {
      const uint32_t o0 = (uint32_t)lb.out_off[i], o1 = (uint32_t)lb.out_off[i + 1];
      for (uint32_t b = (o0 + kScatterThreads - 1) / kScatterThreads; b * kScatterThreads < o1; ++b) blk[b] = i;
    }
  }
  __syncthreads();
  // each document's output offset: that of its first part
  if (out_off)
    for (uint32_t d = tid; d <= nb; d += kSelThreads) out_off[d] = lb.fin[lb.doc_part[d]];
  if (tid == 0) {
    lb.misc[0] = (uint32_t)lb.out_off[parts];
    ctr->total = carry;
    __threadfence_system();
    report(&ctr->ins_done, gen);
  }
}

__global__ void __launch_bounds__(kScatterThreads)
lit_scatter_kernel(LitBufs lb, int32_t* __restrict__ out, uint32_t* __restrict__ spans, uint64_t cap) {
  const uint32_t parts = lb.misc[2];
  const uint32_t T = lb.misc[0];
  const uint32_t* blk = reinterpret_cast<const uint32_t*>(lb.cand);
  for (uint32_t t = blockIdx.x * kScatterThreads + threadIdx.x; t < T; t += gridDim.x * kScatterThreads) {
    // the part holding pipeline token t: the last i with out_off[i] <= t,
    // from the part of token 256 floor(t / 256) forward
    uint32_t lo = parts > 1 ? blk[t / kScatterThreads] : 0u;
    while (lo + 1 < parts && lb.out_off[lo + 1] <= t) ++lo;
    if (lb.part_lit[lo] >= 0) continue;  // made from a literal's own bytes: replaced by its ID
    const uint64_t at = (uint64_t)lb.fin[lo] + (t - (uint32_t)lb.out_off[lo]);
    if (at < cap) {
      out[at] = lb.ids[t];
      if (spans) spans[at] = lb.spans[t];
    }
  }
}

}  // namespace

void launch_literal_pass(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, Literals L,
                         LitBufs lb, Counters* ctr, uint64_t gen, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kLitTile - 1) / kLitTile);
  lit_match_kernel<<<tiles, kMatchThreads, 0, s>>>(text, n, doc_off, n_docs, L, lb);
  lit_select_kernel<<<1, kSelThreads, 0, s>>>(n, tiles, doc_off, n_docs, L, lb, ctr, gen);
}

void launch_literal_insert(uint64_t n, Literals L, LitBufs lb, int32_t* out, uint32_t* spans, uint64_t cap,
                           uint64_t* out_off, Counters* ctr, uint64_t gen, hipStream_t s) {
  lit_insert_kernel<<<1, kSelThreads, 0, s>>>(L, lb, out, spans, cap, out_off, ctr, gen);
  const uint32_t blocks = (uint32_t)std::min<uint64_t>((n + kScatterThreads - 1) / kScatterThreads, 8192);
  lit_scatter_kernel<<<blocks, kScatterThreads, 0, s>>>(lb, out, spans, cap);
}

}  // namespace tok
