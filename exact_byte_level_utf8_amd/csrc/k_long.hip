// Long pieces: BPE of every piece longer than 64 bytes by a whole workgroup.
//
// The piece pass defers such a piece: it appends the piece's first byte to a
// device work queue and leaves one marker entry for it in its tile's run of
// IDs.  This kernel runs next: its workgroups take pieces from the queue
// (an atomic counter; every workgroup leaves when the queue is empty) and
// merge each with all 512 threads, its symbols held in LDS up to 4,096 (in
// the byte-indexed workspace in global memory above that).  The tokens go to
// ws_sym[s ..], each token's first byte relative to s to ws_rk[s ..], and the
// token count to the queue entry and into the tile counts, so the assembly
// can expand the marker (TokTier, section 4 "GPU BPE": longer pieces fall to a
// block-per-piece kernel; GraphTok, section 4 "Design": long pieces get their
// own path).
//
// A round merges, at once, every pair of the piece's lowest rank and every
// sheltered pair, then compacts the piece.  A pair (x, y) of rank r is
// sheltered when walking left from x, across pairs ranked above r, reaches a
// token that no merge ranked below r takes as its right operand (x itself
// counts) or the piece start, and likewise walking right from y with left
// operands.  Then no merge ranked below r can ever change x or y: any merge
// touching the walked stretch first has the rank of a pair on it or of a
// barrier token's operand, both above r.  So textbook BPE merges (x, y)
// before anything changes them, and merging it now cannot change the result
// (GraphTok, section 4 "Warp-cooperative BPE": lowest rank wins, leftmost on
// equal rank; TokTier, "Exact GPU Tokenization": all leftmost non-overlapping
// occurrences of the minimum-rank pair merge in one round).  The merge rows of
// the piece pass walk at most two pairs; here a walk goes up to 64, which
// bounds the rounds of a long piece by its merge depth rather than by the
// number of distinct ranks in it.  Adjacent chosen pairs share one rank, and
// a run of them keeps every other pair from its first (the leftmost
// non-overlapping occurrences).
#include "tok_internal.h"
#include "wg_scan.h"

namespace tok {
namespace {

constexpr int kLongNT = 512;                        // threads per workgroup
constexpr int kLongE = 8;                           // symbols per thread per chunk
constexpr uint32_t kLongCap = kLongNT * kLongE;     // symbols per chunk, and the LDS capacity
constexpr uint32_t kWalkMax = 64;                   // pairs a shelter walk may cross
constexpr uint32_t kChosen = 0x40000000u;           // marks a chosen pair's rank within a round

__device__ inline uint32_t rank_of(uint32_t v) { return v == kNoRank ? kNoRank : (v & ~kChosen); }
__device__ inline bool chosen_bit(uint32_t v) { return (v >> 30) == 1u; }

struct MinOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct MaxOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

// Rank of the merge (a, b), or kNoRank: open addressing over buckets of
// kBucket slots (left << 44 | right << 24 | rank).
__device__ inline uint32_t long_merge_rank(const Tables& T, uint32_t a, uint32_t b) {
  const uint32_t khi = (a << 12) | (b >> 8), klo = b & 0xFFu;
  uint32_t h = merge_hash(a, b) & T.merge_buckets;
  for (uint32_t probe = 0; probe <= T.merge_buckets; ++probe) {
    const ulonglong2* bk = reinterpret_cast<const ulonglong2*>(T.merge_slots + (size_t)h * kBucket);
    const ulonglong2 s01 = bk[0], s23 = bk[1];
    const uint64_t v[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (uint32_t)v[j], hi = (uint32_t)(v[j] >> 32);
      if (hi == khi && (lo >> 24) == klo) return lo & 0xFFFFFFu;
    }
    if (s23.y == kEmptySlot) return kNoRank;  // slots fill in order within a bucket
    h = (h + 1) & T.merge_buckets;
  }
  return kNoRank;
}

// Shelter walks of the pair k (symbols k, k + 1) of rank r among n symbols.
__device__ inline bool sheltered(const uint32_t* rk, const uint2* mm, uint32_t n, uint32_t k, uint32_t r) {
  bool left = false;
  uint32_t i = k;
  for (uint32_t s = 0; s <= kWalkMax; ++s) {
    if (mm[i].x > r || i == 0) {
      left = true;
      break;
    }
    if (rank_of(rk[i - 1]) <= r) break;
    --i;
  }
  if (!left) return false;
  i = k + 1;
  for (uint32_t s = 0; s <= kWalkMax; ++s) {
    if (mm[i].y > r || i == n - 1) return true;
    if (rank_of(rk[i]) <= r) return false;
    ++i;
  }
  return false;
}

// BPE of the n-symbol piece held in sym / rk / mm (LDS or global memory), in
// rounds; returns the final symbol count.  Called by every thread with
// uniform arguments.  sym[i]: token i; rk[i]: rank of the pair (i, i + 1)
// (kNoRank for the last); mm[i]: the token's lowest ranks as right operand
// (x) and as left operand (y).
__device__ __forceinline__ uint32_t merge_piece(const Tables& T, uint32_t* sym, uint32_t* rk, uint2* mm,
                                                uint32_t n, uint32_t low, uint32_t* s_scan) {
  const uint32_t tid = threadIdx.x;
  while (low != kNoRank) {  // uniform
    // pass A: which pairs merge; mark the chosen ones in rk
    uint32_t rs_carry = 0;  // 1 + the last pair before this chunk that does not merge (0: none)
    const uint32_t pairs = n - 1;
    for (uint32_t c0 = 0; c0 < pairs; c0 += kLongCap) {
      const uint32_t k0 = c0 + tid * kLongE;
      bool take[kLongE];
      uint32_t last_stop = 0;  // 1 + last non-merging pair among this thread's
#pragma unroll
      for (int e = 0; e < kLongE; ++e) {
        const uint32_t k = k0 + e;
        take[e] = false;
        if (k < pairs) {
          const uint32_t r = rank_of(rk[k]);
          take[e] = r != kNoRank && (r == low || sheltered(rk, mm, n, k, r));
          if (!take[e]) last_stop = k + 1;
        }
      }
      uint32_t total = 0;
      const uint32_t before = MaxOp()(rs_carry, wg_excl_scan<kLongNT>(last_stop, 0u, MaxOp(), s_scan, &total));
      uint32_t rs = before;  // run start of this thread's first pair
#pragma unroll
      for (int e = 0; e < kLongE; ++e) {
        const uint32_t k = k0 + e;
        if (k < pairs) {
          if (take[e] && ((k - rs) & 1u) == 0u) rk[k] |= kChosen;
          if (!take[e]) rs = k + 1;
        }
      }
      rs_carry = __builtin_amdgcn_readfirstlane(MaxOp()(rs_carry, total));
      __syncthreads();  // marks visible before the next chunk's walks
    }
    // pass B: compaction, chunk by chunk in place (a symbol only moves down);
    // pairs next to a merge are probed again
    uint32_t removed = 0;        // symbols removed before this chunk
    bool prev_chosen = false;    // the last pair before this chunk merged
    uint32_t new_low = kNoRank;
    for (uint32_t c0 = 0; c0 < n; c0 += kLongCap) {
      const uint32_t i0 = c0 + tid * kLongE;
      uint32_t ns[kLongE], nr[kLongE];
      uint2 nm[kLongE];
      bool alive[kLongE], chose[kLongE];
      uint32_t mine = 0;  // chosen pairs among this thread's positions
      bool pc = i0 == c0 ? prev_chosen : (i0 < n && chosen_bit(rk[i0 - 1]));
#pragma unroll
      for (int e = 0; e < kLongE; ++e) {
        const uint32_t i = i0 + e;
        alive[e] = false;
        chose[e] = false;
        if (i < n) {
          const uint32_t v = rk[i];
          const bool ch = chosen_bit(v);
          chose[e] = ch;
          alive[e] = !pc;
          if (alive[e]) {
            ns[e] = ch ? 256u + rank_of(v) : sym[i];
            nm[e] = ch ? T.tok_min[ns[e]] : mm[i];
            const uint32_t kn = ch ? i + 2 : i + 1;
            nr[e] = kNoRank;
            if (kn < n) {
              const uint32_t vn = rk[kn];
              const bool chn = chosen_bit(vn);
              if (ch || chn) nr[e] = long_merge_rank(T, ns[e], chn ? 256u + rank_of(vn) : sym[kn]);
              else nr[e] = rank_of(v);
            }
          }
          mine += ch ? 1u : 0u;
          pc = ch;
        }
      }
      uint32_t chunk_chosen = 0;
      const uint32_t before = wg_excl_scan<kLongNT>(mine, 0u, AddOp(), s_scan, &chunk_chosen);
      // the last pair of this chunk, for the next chunk's first symbol (read
      // before any write of this chunk: the scan above holds barriers)
      const uint32_t last = min(c0 + kLongCap, n) - 1;
      const bool last_chosen = last + 1 < n && chosen_bit(rk[last]);
      __syncthreads();
      // symbol i moves to i less the chosen pairs before it; a symbol absorbed
      // by the pair before it is not written (its index is its partner's)
      uint32_t q = i0 - removed - before;
#pragma unroll
      for (int e = 0; e < kLongE; ++e) {
        const uint32_t i = i0 + e;
        if (i < n && alive[e]) {
          sym[q] = ns[e];
          rk[q] = nr[e];
          mm[q] = nm[e];
          new_low = min(new_low, nr[e]);
        }
        q += chose[e] ? 0u : 1u;
      }
      removed = __builtin_amdgcn_readfirstlane(removed + chunk_chosen);
      prev_chosen = __builtin_amdgcn_readfirstlane((uint32_t)last_chosen) != 0u;
      __syncthreads();
    }
    n -= removed;
    uint32_t all = 0;
    (void)wg_excl_scan<kLongNT>(new_low, kNoRank, MinOp(), s_scan, &all);
    low = __builtin_amdgcn_readfirstlane(all);
  }
  return n;
}

// Byte offset of the first piece start after s, or n (one wave).
__device__ inline uint64_t next_start_wave(const uint16_t* flags, uint64_t n, uint64_t s) {
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t c = s / kChunk;
  const uint32_t own = flags[c] & ~((2u << (s % kChunk)) - 1u);
  if (own) return c * kChunk + __builtin_ctz(own);
  for (uint64_t cb = c + 1; cb < n_chunks; cb += 64) {
    const uint64_t ci = cb + lane;
    const uint32_t wv = ci < n_chunks ? flags[ci] : 0u;
    const uint64_t mask = __ballot(wv != 0);
    if (mask) {
      const uint32_t l = __builtin_ctzll(mask);
      const uint32_t wl = __builtin_amdgcn_readfirstlane(__shfl(wv, l, 64));
      return (cb + l) * kChunk + __builtin_ctz(wl);
    }
  }
  return n;
}

// One piece of len bytes at text[s]: load its bytes as symbols into sym / rk
// / mm (the LDS arrays or the piece's own stretch of the workspace), merge,
// then write its tokens to ws_sym[s ..] and their first bytes relative to s
// to ws_rk[s ..].  Returns the token count.  LDS selects the instance whose
// arrays are in LDS, so the compiler keeps LDS accesses as such.
template <bool LDS>
__device__ __forceinline__ uint32_t long_piece(const uint8_t* __restrict__ text, uint64_t s, uint32_t len,
                                               const Tables& T, const Bufs& B, uint32_t* sym, uint32_t* rk,
                                               uint2* mm, uint32_t* s_scan) {
  const uint32_t tid = threadIdx.x;
  uint32_t low = kNoRank;
  for (uint32_t i = tid; i < len; i += kLongNT) {
    const uint32_t a = text[s + i];
    sym[i] = a;
    const uint32_t r = i + 1 < len ? T.pair_rank[(a << 8) | text[s + i + 1]] : kNoRank;
    rk[i] = r;
    mm[i] = T.tok_min[a];
    low = min(low, r);
  }
  uint32_t all = 0;
  (void)wg_excl_scan<kLongNT>(low, kNoRank, MinOp(), s_scan, &all);  // its barriers order the stores above
  const uint32_t cnt =
      __builtin_amdgcn_readfirstlane(merge_piece(T, sym, rk, mm, len, __builtin_amdgcn_readfirstlane(all), s_scan));
  uint32_t at = 0;
  for (uint32_t i0 = 0; i0 < cnt; i0 += kLongNT) {
    const uint32_t i = i0 + tid;
    const uint32_t t = i < cnt ? sym[i] : 0u;
    const uint32_t l = i < cnt ? T.tok_len[t] : 0u;
    uint32_t chunk = 0;
    const uint32_t before = wg_excl_scan<kLongNT>(l, 0u, AddOp(), s_scan, &chunk);  // reads before any write
    if (i < cnt) {
      B.ws_sym[s + i] = t;
      B.ws_rk[s + i] = at + before;
    }
    at = __builtin_amdgcn_readfirstlane(at + chunk);
  }
  return cnt;
}

__global__ void __launch_bounds__(kLongNT, 1)
long_piece_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B) {
  __shared__ uint32_t s_sym[kLongCap], s_rk[kLongCap];
  __shared__ uint2 s_mm[kLongCap];
  __shared__ uint32_t s_scan[kLongNT / kWave];
  __shared__ uint32_t s_item, s_end_lo, s_end_hi;
  const uint32_t tid = threadIdx.x;
  const uint32_t queued = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&B.lq_ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  for (;;) {
    if (tid == 0) s_item = atomicAdd(&B.lq_ctr[1], 1u);
    __syncthreads();
    const uint32_t j = __builtin_amdgcn_readfirstlane(s_item);
    if (j >= queued) break;  // uniform: every workgroup leaves once the queue is empty
    const uint64_t s = B.lq_start[j];
    if (tid < kWave) {
      const uint64_t e = next_start_wave(B.flags, n, s);
      if (tid == 0) {
        s_end_lo = (uint32_t)e;
        s_end_hi = (uint32_t)(e >> 32);
      }
    }
    __syncthreads();
    const uint64_t e = ((uint64_t)s_end_hi << 32) | s_end_lo;
    const uint32_t len = __builtin_amdgcn_readfirstlane((uint32_t)(e - s));
    const uint32_t cnt = len <= kLongCap
                             ? long_piece<true>(text, s, len, T, B, s_sym, s_rk, s_mm, s_scan)
                             : long_piece<false>(text, s, len, T, B, B.ws_sym + s, B.ws_rk + s,
                                                 reinterpret_cast<uint2*>(B.ws_sel + s), s_scan);
    if (tid == 0) {
      B.lq_len[j] = len;
      B.lq_cnt[j] = cnt;
      const uint32_t tile = (uint32_t)(s / kPieceTile), extra = cnt - 1;  // the marker counted one
      if (extra) {
        atomicAdd(&B.tile_cnt[tile], extra);
        atomicAdd(&B.sum1[tile >> kSum1Shift], extra);
        atomicAdd(&B.sum2[tile >> kSum2Shift], extra);
      }
    }
    __syncthreads();  // the LDS arrays and s_item are reused by the next piece
  }
}

}  // namespace

void launch_long(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t tiles = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
  if (!tiles) return;
  // a work queue: any grid drains it; one workgroup per CU slot of the device
  // (64 KiB of LDS each), fewer for small inputs
  const uint32_t grid = std::min<uint32_t>(std::max<uint32_t>(tiles / 2, 1u), 512u);
  launch_on(long_piece_kernel, dim3(grid), dim3(kLongNT), s, e0, e1, text, n, t, b);
}

}  // namespace tok
