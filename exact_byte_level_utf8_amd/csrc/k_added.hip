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
//                      word at a time).  The cursor scan of the definition
//                      keeps each match that starts at or after the end of
//                      the last one kept; each tile resolves that for its own
//                      matches (clusters of overlapping matches, one thread
//                      each, decided exactly from the matches of the 256
//                      bytes before the tile) and writes the kept ones in
//                      position order.
//   lit_select_kernel  the kept matches of all tiles in order: workgroups
//                      copy shares of the tiles and place the cut points;
//                      the last one to finish checks the offsets and, if a
//                      tile whose first cluster began too far back listed
//                      all its matches, runs the cursor scan over the whole
//                      list.  The taken literals cut the text into 2k + 1
//                      parts: segment, literal, segment, ..., segment.
// The parts then run through the usual pipeline as documents (their count
// read on the device, so the host enqueues everything without waiting),
// which are hard boundaries for code points, pieces and merges, exactly as
// the segments between literals must be.  Without span export the literal
// IDs are folded into that pipeline: the match kernel clears its tile's
// literal marks, the pre-tokenization kernel marks the taken literals on
// its way in (1 on the first byte, 2 on the others, and the ID at the first
// byte), and the piece pass takes each marked literal as one piece whose
// token is its ID, so the pipeline's output is the result; only a batch's
// document offsets are mapped afterwards (lit_doc_offsets_kernel).  With
// span export the literals' own bytes go through the pipeline too, and:
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
constexpr uint32_t kInsPer = 6;  // parts per thread in one pass of the insertion (48 KiB of LDS)
constexpr uint32_t kLitBack = 256;        // bytes before its tile whose matches the match kernel also finds
constexpr uint32_t kTileRaw = 1u << 31;   // tile count flag: every match of the tile listed, unresolved
constexpr uint8_t kMarkHead = 1, kMarkKept = 2;
// marks of the selection in the literal half of a match word
constexpr uint64_t kSelKeep = 1ull << 31, kSelHead = 1ull << 30;
constexpr uint32_t kSelIndex = kLitMaxCount - 1;  // the literal index bits
static_assert((kLitMaxCount & (kLitMaxCount - 1)) == 0 && kLitMaxCount <= (1u << 30), "index bits below the marks");

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
  // the window: kLitBack bytes before the tile, the tile, the longest
  // literal's reach past it, and a guard word; at most one match per position
  constexpr uint32_t kWords = (kLitBack + kLitTile + kLitMax + 8) / 4;
  constexpr uint32_t kList = kLitBack + kLitTile;
  constexpr uint32_t kPer = (kList + kMatchThreads - 1) / kMatchThreads;
  static_assert(kLitBack == kMatchThreads && kLitTile == 4 * kMatchThreads, "one window-front and four tile positions per thread");
  static_assert(kLitBack >= 2 * kLitMax, "the front of the window decides the cluster heads of the tile's matches");
  __shared__ uint32_t s_text[kWords];
  __shared__ uint32_t s_first[8];
  __shared__ uint32_t s_scan[kMatchThreads / kWave];
  __shared__ uint32_t s_pos[kList];  // each match's start and end, counted from the window's first byte
  __shared__ uint32_t s_end[kList];
  __shared__ uint16_t s_lit[kList];
  __shared__ uint8_t s_mark[kList];  // kMarkHead, kMarkKept
  __shared__ uint32_t s_first_exact, s_raw;
  const uint32_t tile = blockIdx.x, tid = threadIdx.x;
  const uint64_t base = (uint64_t)tile * kLitTile;
  const int64_t w0 = (int64_t)base - (int64_t)kLitBack;  // the window's first byte (before the text for tile 0)
  if (tile == 0 && tid == 0) lb.misc[4] = 0;  // the selection's count of finished workgroups
  {
    const bool aligned = (reinterpret_cast<uintptr_t>(text) & 3u) == 0;
    for (uint32_t w = tid; w < kWords; w += kMatchThreads) {
      const int64_t p = w0 + 4 * (int64_t)w;
      uint32_t v = 0;
      if (aligned && p >= 0 && p + 4 <= (int64_t)n) {
        v = *reinterpret_cast<const uint32_t*>(text + p);
      } else {
        for (uint32_t i = 0; i < 4; ++i)
          if (p + i >= 0 && p + i < (int64_t)n) v |= (uint32_t)text[p + i] << (8 * i);
      }
      s_text[w] = v;
    }
    if (tid < 8) s_first[tid] = L.first[tid];
    if (lb.fold)  // this tile's literal marks start clear (the selection writes them)
      for (uint32_t w = tid; w < kLitTile / 4; w += kMatchThreads)
        reinterpret_cast<uint32_t*>(lb.lmark + base)[w] = 0;
  }
  __syncthreads();
  // the longest literal at window-front position tid and at tile positions
  // 4 tid .. 4 tid + 3
  auto match = [&](uint32_t q) -> int32_t {  // q: window byte
    const int64_t p = w0 + (int64_t)q;
    if (p < 0 || p >= (int64_t)n) return -1;
    const uint32_t b0 = (s_text[q >> 2] >> (8 * (q & 3u))) & 0xFFu;
    if (!((s_first[b0 >> 5] >> (b0 & 31u)) & 1u)) return -1;
    return literal_at(s_text, q, b0, n, (uint64_t)p, L, doc_off, n_docs);
  };
  const int32_t mf = match(tid);
  int32_t m[4];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = match(kLitBack + 4u * tid + j);
    c += m[j] >= 0 ? 1u : 0u;
  }
  uint32_t nf = 0, nt = 0;
  const uint32_t af = wg_excl_scan<kMatchThreads>(mf >= 0 ? 1u : 0u, 0u, AddOp(), s_scan, &nf);
  const uint32_t at0 = nf + wg_excl_scan<kMatchThreads>(c, 0u, AddOp(), s_scan, &nt);
  auto put = [&](uint32_t i, uint32_t q, int32_t li) {
    s_pos[i] = q;
    s_end[i] = q + lit_len(L, (uint32_t)li);
    s_lit[i] = (uint16_t)li;
    s_mark[i] = 0;
  };
  if (mf >= 0) put(af, tid, mf);
  {
    uint32_t i = at0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (m[j] >= 0) put(i++, kLitBack + 4u * tid + j, m[j]);
  }
  __syncthreads();
  // Cluster heads: a match that no earlier match reaches (the cursor keeps it
  // whatever came before; the selection kernel describes the clusters).  A
  // match before the window reaches at most kLitMax - 1 bytes into it, so a
  // head decided at a window byte from kLitMax on is exact.
  const uint32_t nl = nf + nt;
  const uint32_t i0 = min(nl, tid * kPer), i1 = min(nl, i0 + kPer);
  uint32_t mx = 0;
  for (uint32_t i = i0; i < i1; ++i) mx = max(mx, s_end[i]);
  uint32_t reach = wg_excl_scan<kMatchThreads>(mx, 0u, MaxOp(), s_scan, nullptr);
  for (uint32_t i = i0; i < i1; ++i) {
    if (reach <= s_pos[i]) s_mark[i] = kMarkHead;
    reach = max(reach, s_end[i]);
  }
  if (tid == 0) {
    s_raw = 0;
    s_first_exact = nl;
  }
  __syncthreads();
  // the head that governs the tile's first match: resolved when it is exact
  if (tid == 0 && nt > 0) {
    uint32_t g = nf;
    while (g > 0 && !(s_mark[g] & kMarkHead)) --g;
    const bool exact = (s_mark[g] & kMarkHead) && s_pos[g] >= kLitMax;
    s_raw = exact ? 0u : 1u;
    s_first_exact = g;
  }
  __syncthreads();
  // every cluster from the governing head on, one thread per head, in order
  const uint32_t g = s_first_exact;
  for (uint32_t h = max(i0, g); h < i1; ++h) {
    if (!(s_mark[h] & kMarkHead)) continue;
    uint32_t end = 0, j = h;
    do {
      if (s_pos[j] >= end) {
        s_mark[j] |= kMarkKept;
        end = s_end[j];
      }
      ++j;
    } while (j < nl && !(s_mark[j] & kMarkHead));
  }
  __syncthreads();
  // the tile's matches in order: only the kept ones once resolved, else all
  // of them (the selection kernel then resolves them with the rest)
  const bool raw = s_raw != 0;
  uint32_t keep[4], k = 0;
  {
    uint32_t i = at0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      keep[j] = 0;
      if (m[j] >= 0) {
        keep[j] = raw || (s_mark[i] & kMarkKept) ? 1u : 0u;
        ++i;
      }
      k += keep[j];
    }
  }
  uint32_t tot = 0;
  uint32_t at = wg_excl_scan<kMatchThreads>(k, 0u, AddOp(), s_scan, &tot);
  uint64_t* out = lb.cand + (uint64_t)tile * kLitTile;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (keep[j]) out[at++] = ((base + 4u * tid + j) << 32) | (uint32_t)m[j];
  if (tid == 0) lb.tile_cnt[tile] = tot | (raw ? kTileRaw : 0u);
}

constexpr uint32_t kSelBatch = 16;  // global loads one selection thread keeps in flight
constexpr uint32_t kSelWaves = kSelThreads / kWave;
constexpr uint32_t kCopyTiles = 4;     // tiles whose matches one selection wave loads at once
constexpr uint32_t kSelDocs = 2048;    // document boundaries a selection workgroup holds in LDS
constexpr uint32_t kSelTilesPerWg = 32;  // selection workgroups: about one per this many tiles,
constexpr uint32_t kSelMaxWgs = 64;      // at most this many

__global__ void __launch_bounds__(kSelThreads)
lit_select_kernel(uint64_t n, uint32_t tiles, const uint64_t* __restrict__ doc_off, uint32_t n_docs, Literals L,
                  LitBufs lb, Counters* ctr, uint64_t gen) {
  __shared__ uint32_t s_scan[kSelWaves];
  __shared__ uint32_t s_over, s_bad, s_last;
  __shared__ uint32_t s_tb[kSelThreads], s_tv[kSelThreads];  // a chunk's tiles: first output index, match count
  __shared__ uint8_t s_len[kLitMaxCount];                      // the literals' lengths
  __shared__ uint64_t s_doc[kSelDocs];                         // the document boundaries, where they fit
  const uint32_t tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  if (tid == 0) {
    s_over = 0;
    s_bad = 0;
    s_last = 0;
  }
  for (uint32_t i = tid; i < L.n; i += kSelThreads) s_len[i] = (uint8_t)lit_len(L, i);
  // the caller's documents (one document [0, n) without offsets): the
  // pipeline sees only the parts, so their offsets are checked here
  const uint32_t nd = doc_off ? n_docs : 1u;
  const bool doc_lds = nd < kSelDocs;
  auto D = [&](uint32_t d) -> uint64_t { return doc_off ? doc_off[d] : (d == 0 ? 0ull : n); };
  if (doc_lds)
    for (uint32_t d = tid; d <= nd; d += kSelThreads) s_doc[d] = D(d);
  __syncthreads();
  auto Dc = [&](uint32_t d) -> uint64_t { return doc_lds ? s_doc[d] : D(d); };
  // cut points: the document boundaries merged with each literal's start and
  // end.  A boundary comes before a literal starting on it and after a
  // literal ending on it; literals never straddle a boundary.
  //   index of start j = 2j + #{d : D(d) <= S_j}
  //   index of end j   = 2j + 1 + #{d : D(d) < E_j}
  //   index of D(d)    = d + 2 #{j : S_j < D(d)}
  // With one boundary pair, 0 and n, literal j's start and end are cut
  // points 2j + 1 and 2j + 2.
  auto place = [&](uint32_t j, uint64_t a) {
    const uint32_t li = (uint32_t)a & kSelIndex;
    const uint64_t S = a >> 32, E = S + s_len[li];
    if (nd == 1) {
      lb.cut[2 * j + 1] = S;
      lb.cut[2 * j + 2] = E;
      if (!lb.fold) {
        lb.part_lit[2 * j] = -1;  // the stretch before the literal
        lb.part_lit[2 * j + 1] = L.ids[li];
      }
      return;
    }
    uint32_t lo = 0, hi = nd + 1;  // #{d : D(d) <= S}
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (Dc(mid) <= S) lo = mid + 1;
      else hi = mid;
    }
    const uint32_t is = 2 * j + lo;
    lo = 0;
    hi = nd + 1;  // #{d : D(d) < E}
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (Dc(mid) < E) lo = mid + 1;
      else hi = mid;
    }
    lb.cut[is] = S;
    lb.cut[2 * j + 1 + lo] = E;
  };
  // Matches before each tile (a scan of the tile counts, a chunk of tiles at
  // a time; uniform trip count: the scan holds barriers).  Every workgroup
  // scans all counts and copies its share of each chunk's tiles into the
  // list, placing each match's cut points as it goes: a wave per tile, its
  // lanes on consecutive matches so that loads and stores coalesce,
  // kCopyTiles tiles in flight.
  uint32_t carry = 0;
  bool raw = false;  // a tile listed all its matches, unresolved
  for (uint32_t t0 = 0; t0 < tiles; t0 += kSelThreads) {
    const uint32_t t = t0 + tid;
    const uint32_t w = t < tiles ? lb.tile_cnt[t] : 0u, v = w & ~kTileRaw;
    raw |= (w & kTileRaw) != 0;
    uint32_t tot = 0;
    s_tb[tid] = carry + wg_excl_scan<kSelThreads>(v, 0u, AddOp(), s_scan, &tot);
    s_tv[tid] = v;
    __syncthreads();
    const uint32_t nt = min(tiles - t0, kSelThreads);
    const uint32_t qa = (uint32_t)((uint64_t)nt * g / G), qb = (uint32_t)((uint64_t)nt * (g + 1) / G);
    for (uint32_t q0 = qa + wave; q0 < qb; q0 += kCopyTiles * kSelWaves) {
      uint32_t vmax = 0;  // the most matches of the wave's tiles (the same on every lane)
#pragma unroll
      for (uint32_t u = 0; u < kCopyTiles; ++u) {
        const uint32_t q = q0 + u * kSelWaves;
        vmax = max(vmax, q < qb ? s_tv[q] : 0u);
      }
      for (uint32_t e0 = 0; e0 < vmax; e0 += kWave) {
        const uint32_t e = e0 + lane;
        uint64_t x[kCopyTiles];
#pragma unroll
        for (uint32_t u = 0; u < kCopyTiles; ++u) {
          const uint32_t q = q0 + u * kSelWaves;
          x[u] = q < qb && e < s_tv[q] ? lb.cand[(uint64_t)(t0 + q) * kLitTile + e] : 0ull;
        }
#pragma unroll
        for (uint32_t u = 0; u < kCopyTiles; ++u) {
          const uint32_t q = q0 + u * kSelWaves;
          if (q < qb && e < s_tv[q]) {
            const uint32_t j = s_tb[q] + e;
            lb.sel[j] = x[u];
            place(j, x[u]);
          }
        }
      }
    }
    carry += tot;
    __syncthreads();  // the next chunk rewrites s_tb and s_tv
  }
  if (raw) s_over = 1u;  // (a possible overlap: checked below)
  const uint32_t K = carry;
  // The last workgroup to finish its share completes the selection (the
  // match kernel zeroed the count word); the others are done.
  if (G > 1) {
    __syncthreads();
    if (tid == 0) {
      __threadfence();  // this workgroup's list entries and cut points, before its count
      if (atomicAdd(&lb.misc[4], 1u) == G - 1) {
        __threadfence();  // every other workgroup's writes, before the reads below
        s_last = 1u;
      }
    }
    __syncthreads();
    if (!s_last) return;
  }
  bool bad = false;
  for (uint32_t d = tid; d < nd; d += kSelThreads) bad |= Dc(d) > Dc(d + 1);
  if (tid == 0) bad |= Dc(0) != 0 || Dc(nd) != n;
  if (bad) s_bad = 1u;
  __syncthreads();
  // Tiles resolve their own clusters (lit_match_kernel), so the list holds
  // only taken matches, which never overlap, unless a tile was left
  // unresolved: then the cursor scan runs here over the whole list.
  if (s_over) {  // uniform: some tile was left unresolved; do its matches overlap?
    __syncthreads();
    if (tid == 0) s_over = 0;
    __syncthreads();
    bool over = false;
    for (uint32_t i = tid; i + 1 < K; i += kSelThreads) {
      const uint64_t a = lb.sel[i], b = lb.sel[i + 1];
      over |= (a >> 32) + s_len[(uint32_t)a & kSelIndex] > (b >> 32);
    }
    if (over) s_over = 1u;
    __syncthreads();
  }
  // malformed offsets: report, and fall back to one part with no literal
  // (the call fails; everything below stays in bounds)
  const bool bad_docs = s_bad != 0;
  uint32_t k = bad_docs ? 0u : K;
  const bool resolve = !bad_docs && s_over;  // uniform: LDS words read after a barrier
  if (resolve) {
    // The cursor keeps a match iff it starts at or after the end of the last
    // match kept.  Where no earlier match reaches the next one's start (the
    // running maximum of the ends, a scan), the last kept match has ended
    // too, so that match is kept whatever came before: the matches split
    // there into clusters that are resolved independently, one thread
    // walking each in order.  Marks go into the literal half of the words
    // (indexes stay below kLitMaxCount); then the kept matches move down in
    // order.  Positions fit 32 bits (inputs are under 2^32 bytes).
    uint32_t reach = 0;  // the largest end before this chunk
    for (uint32_t c0 = 0; c0 < K; c0 += kSelThreads) {  // uniform trip count: the scan holds barriers
      const uint32_t i = c0 + tid;
      const uint64_t a = i < K ? lb.sel[i] : 0ull;
      const uint32_t S = (uint32_t)(a >> 32), E = S + s_len[(uint32_t)a & kSelIndex];
      uint32_t tot = 0;
      const uint32_t before = max(reach, wg_excl_scan<kSelThreads>(i < K ? E : 0u, 0u, MaxOp(), s_scan, &tot));
      if (i < K && (i == 0 || before <= S)) lb.sel[i] = a | kSelHead;
      reach = max(reach, tot);
    }
    __syncthreads();  // every cluster head marked
    for (uint32_t h = tid; h < K; h += kSelThreads) {
      if (!(lb.sel[h] & kSelHead)) continue;
      uint32_t end = 0, j = h;
      do {
        const uint64_t a = lb.sel[j];
        const uint32_t S = (uint32_t)(a >> 32);
        if (S >= end) {
          lb.sel[j] = a | kSelKeep;
          end = S + s_len[(uint32_t)a & kSelIndex];
        }
        ++j;
      } while (j < K && !(lb.sel[j] & kSelHead));
    }
    __syncthreads();  // every kept match marked
    uint32_t kept = 0;
    for (uint32_t c0 = 0; c0 < K; c0 += kSelThreads) {
      const uint32_t i = c0 + tid;
      const uint64_t a = i < K ? lb.sel[i] : 0ull;
      const uint32_t keep = (a & kSelKeep) ? 1u : 0u;
      uint32_t tot = 0;
      // the scan's barriers put every read of this chunk before any write; a
      // match only moves down, and later chunks are read after
      const uint32_t at = kept + wg_excl_scan<kSelThreads>(keep, 0u, AddOp(), s_scan, &tot);
      if (keep) lb.sel[at] = a & ~(kSelHead | kSelKeep);
      kept += tot;
    }
    __syncthreads();
    k = kept;
  }
  const uint32_t nb = bad_docs ? 1u : nd;  // boundaries 0..nb
  auto Db = [&](uint32_t d) -> uint64_t { return bad_docs ? (d == 0 ? 0ull : n) : Dc(d); };
  const uint32_t parts = nb + 2 * k;
  // The cut points and literal IDs placed with the copy stand, unless the
  // list was resolved here, the offsets were malformed (one part, no
  // literal), or literal IDs go to parts among several documents: those are
  // placed here, after every part is marked as no literal.  (The parts'
  // literal IDs serve the insertion; they are unused when the IDs are folded
  // into the piece pass.)
  if (!lb.fold && !(bad_docs || resolve || nb > 1) && tid == 0)
    lb.part_lit[2 * k] = -1;  // the stretch after the last literal
  if (bad_docs || resolve || (!lb.fold && nb > 1)) {  // uniform
    if (!lb.fold)
      for (uint32_t i = tid; i < parts; i += kSelThreads) lb.part_lit[i] = -1;
    __syncthreads();
    if (nb == 1) {
      // one boundary pair, 0 and n (one document, or the fallback): literal j's
      // start and end are cut points 2j + 1 and 2j + 2
      for (uint32_t j0 = tid; j0 < k; j0 += kSelBatch * kSelThreads) {
        uint64_t aa[kSelBatch];
#pragma unroll
        for (uint32_t u = 0; u < kSelBatch; ++u) aa[u] = j0 + u * kSelThreads < k ? lb.sel[j0 + u * kSelThreads] : 0ull;
#pragma unroll
        for (uint32_t u = 0; u < kSelBatch; ++u) {
          const uint32_t j = j0 + u * kSelThreads, li = (uint32_t)aa[u] & kSelIndex;
          if (j < k) {
            const uint64_t S = aa[u] >> 32;
            lb.cut[2 * j + 1] = S;
            lb.cut[2 * j + 2] = S + s_len[li];
            if (!lb.fold) lb.part_lit[2 * j + 1] = L.ids[li];
          }
        }
      }
    } else {
      for (uint32_t j0 = tid; j0 < k; j0 += kSelBatch * kSelThreads) {
        uint64_t aa[kSelBatch];  // kSelBatch literals per pass, their loads in flight together
        uint32_t len[kSelBatch];
        int32_t id[kSelBatch];
#pragma unroll
        for (uint32_t u = 0; u < kSelBatch; ++u) aa[u] = j0 + u * kSelThreads < k ? lb.sel[j0 + u * kSelThreads] : 0ull;
#pragma unroll
        for (uint32_t u = 0; u < kSelBatch; ++u) {
          const bool in = j0 + u * kSelThreads < k;
          len[u] = in ? s_len[(uint32_t)aa[u] & kSelIndex] : 0u;
          id[u] = in && !lb.fold ? L.ids[(uint32_t)aa[u]] : -1;
        }
#pragma unroll
        for (uint32_t u = 0; u < kSelBatch; ++u) {
          const uint32_t j = j0 + u * kSelThreads;
          if (j >= k) break;
          const uint64_t S = aa[u] >> 32, E = S + len[u];
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
          if (!lb.fold) lb.part_lit[is] = id[u];  // the literal's ID (IDs are never negative)
        }
      }
    }
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
  __shared__ int32_t s_plit[kSelThreads * kInsPer];     // a pass's part words: the literal ID, or -1
  __shared__ uint32_t s_poff[kSelThreads * kInsPer + 1];  // and the pipeline's output offsets
  const uint32_t tid = threadIdx.x, parts = lb.misc[2], nb = lb.misc[3];
  // kInsPer consecutive parts per thread, so that a pass covers 6,144 parts
  // with one scan.  The pass's part words are read coalesced into LDS first
  // and each thread then takes its own run of them.  The same pass writes,
  // for the scatter, the part that holds pipeline token 256 b for every b
  // (the parts tile the pipeline's tokens, so each b is written once; the
  // candidate buffer is free by now and holds it).
  uint32_t* blk = reinterpret_cast<uint32_t*>(lb.cand);
  uint32_t carry = 0;
  for (uint32_t i0 = 0; i0 < parts; i0 += kSelThreads * kInsPer) {
    for (uint32_t r = tid; r <= kSelThreads * kInsPer; r += kSelThreads) {
      const uint32_t i = i0 + r;
      if (r < kSelThreads * kInsPer) s_plit[r] = i < parts ? lb.part_lit[i] : -1;
      s_poff[r] = i <= parts ? (uint32_t)lb.out_off[i] : 0u;
    }
    __syncthreads();
    const uint32_t rb = tid * kInsPer, ib = i0 + rb;
    uint32_t v[kInsPer], sum = 0;
#pragma unroll
    for (uint32_t j = 0; j < kInsPer; ++j) {
      const uint32_t i = ib + j;
      v[j] = i >= parts ? 0u : s_plit[rb + j] >= 0 ? 1u : s_poff[rb + j + 1] - s_poff[rb + j];
      sum += v[j];
    }
    uint32_t tot = 0;
    uint32_t at = carry + wg_excl_scan<kSelThreads>(sum, 0u, AddOp(), s_scan, &tot);
#pragma unroll
    for (uint32_t j = 0; j < kInsPer; ++j) {
      const uint32_t i = ib + j;
      if (i < parts) {
        lb.fin[i] = at;
        const int32_t id = s_plit[rb + j];
        if (id >= 0 && at < cap) {
          out[at] = id;
          if (spans) spans[at] = (uint32_t)lb.cut[i];  // the literal starts its part
        }
        const uint32_t o0 = s_poff[rb + j], o1 = s_poff[rb + j + 1];
        if (parts > 1)
          for (uint32_t bk = (o0 + kScatterThreads - 1) / kScatterThreads; bk * kScatterThreads < o1; ++bk) blk[bk] = i;
      }
      at += v[j];
    }
    carry += tot;
    __syncthreads();  // the LDS words are reloaded by the next pass
  }
  if (tid == 0) lb.fin[parts] = carry;
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

// The caller's document offsets when the literal IDs are folded into the
// piece pass: the pipeline's offset of each document's first part.
__global__ void __launch_bounds__(kScatterThreads)
lit_doc_offsets_kernel(LitBufs lb, uint64_t* __restrict__ out_off) {
  const uint32_t nb = lb.misc[3];
  for (uint32_t d = blockIdx.x * kScatterThreads + threadIdx.x; d <= nb; d += gridDim.x * kScatterThreads)
    out_off[d] = lb.out_off[lb.doc_part[d]];
}

}  // namespace

void launch_literal_doc_offsets(LitBufs lb, uint64_t* out_off, uint32_t n_docs, hipStream_t s) {
  const uint32_t blocks = (uint32_t)std::min<uint64_t>(((uint64_t)n_docs + kScatterThreads) / kScatterThreads, 1024);
  lit_doc_offsets_kernel<<<blocks, kScatterThreads, 0, s>>>(lb, out_off);
}

void launch_literal_pass(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, Literals L,
                         LitBufs lb, Counters* ctr, uint64_t gen, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kLitTile - 1) / kLitTile);
  lit_match_kernel<<<tiles, kMatchThreads, 0, s>>>(text, n, doc_off, n_docs, L, lb);
  const uint32_t wgs = std::max(1u, std::min(tiles / kSelTilesPerWg, kSelMaxWgs));
  lit_select_kernel<<<wgs, kSelThreads, 0, s>>>(n, tiles, doc_off, n_docs, L, lb, ctr, gen);
}

void launch_literal_insert(uint64_t n, Literals L, LitBufs lb, int32_t* out, uint32_t* spans, uint64_t cap,
                           uint64_t* out_off, Counters* ctr, uint64_t gen, hipStream_t s) {
  lit_insert_kernel<<<1, kSelThreads, 0, s>>>(L, lb, out, spans, cap, out_off, ctr, gen);
  const uint32_t blocks = (uint32_t)std::min<uint64_t>((n + kScatterThreads - 1) / kScatterThreads, 8192);
  lit_scatter_kernel<<<blocks, kScatterThreads, 0, s>>>(lb, out, spans, cap);
}

}  // namespace tok
