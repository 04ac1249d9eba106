// Merge rounds of one long piece (over 64 bytes) by a whole workgroup.
//
// A round merges, at once, every pair of the piece's lowest rank and every
// sheltered pair, then compacts the piece.  A pair (x, y) of rank r is
// sheltered when walking left from x, across pairs ranked above r, reaches a
// token that no merge ranked below r takes as its right operand (x itself
// counts) or the piece start, and likewise walking right from y with left
// operands.  Then no merge ranked below r can ever change x or y: any merge
// touching the walked stretch first has the rank of a pair on it or of a
// barrier token's operand, both above r.  A walk also ends sheltered once the
// stretch it has crossed, x included, is longer than the longest token: no
// pair on it ranks below r, so a change could only enter at its far end and
// reach x as one token spanning the whole stretch (each merge on the way
// joins the changed token with the next symbol), and no token is that long.  So textbook BPE merges (x, y)
// before anything changes them, and merging it now cannot change the result
// (GraphTok, section 4 "Warp-cooperative BPE": lowest rank wins, leftmost on
// equal rank; TokTier, "Exact GPU Tokenization": all leftmost non-overlapping
// occurrences of the minimum-rank pair merge in one round).  The piece pass's
// merge rows walk at most two pairs; a long piece walks up to 64, which
// bounds its rounds by its merge depth rather than by the number of distinct
// ranks in it (TokTier, section 4 "GPU BPE": longer pieces fall to a
// block-per-piece path).  Adjacent chosen pairs share one rank, and a run of
// them keeps every other pair from its first (the leftmost non-overlapping
// occurrences).
//
// The piece's symbols live in sym / rk / mm, in LDS or in global memory; the
// round processes them in chunks of G::kSize * E symbols, E consecutive
// symbols per thread, with carries from chunk to chunk.  G is the group of
// threads that merges the piece: the whole workgroup (WgGroup), or one wave
// (WaveGroup), so that the waves of a workgroup merge several pieces at
// once with wave scans and no workgroup barrier.
#pragma once

#include "tok_internal.h"
#include "merge_table.h"
#include "wg_scan.h"

namespace tok {
namespace longp {

constexpr uint32_t kWalkMax = 64;          // pairs a shelter walk may cross
constexpr uint32_t kChosen = 0x40000000u;  // marks a chosen pair's rank within a round

__device__ inline uint32_t rank_of(uint32_t v) { return v == kNoRank ? kNoRank : (v & ~kChosen); }
__device__ inline bool chosen_bit(uint32_t v) { return (v >> 30) == 1u; }


// The whole workgroup of NT threads: workgroup scans and barriers.
template <int NT>
struct WgGroup {
  static constexpr uint32_t kSize = NT;
  static constexpr bool kScanSyncs = true;  // a scan holds barriers
  __device__ static uint32_t rank() { return threadIdx.x; }
  __device__ static void sync() { __syncthreads(); }
  template <typename Op>
  __device__ static uint32_t excl_scan(uint32_t v, uint32_t id, Op op, uint32_t* scratch, uint32_t* total) {
    return wg_excl_scan<NT>(v, id, op, scratch, total);
  }
};

// One wave: DPP scans; a wave's LDS accesses take effect in issue order, so
// a wavefront fence (which keeps the compiler from moving memory accesses
// across it) stands in for the barrier.
struct WaveGroup {
  static constexpr uint32_t kSize = kWave;
  static constexpr bool kScanSyncs = false;
  __device__ static uint32_t rank() { return lane_id(); }
  __device__ static void sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  template <typename Op>
  __device__ static uint32_t excl_scan(uint32_t v, uint32_t id, Op op, uint32_t*, uint32_t* total) {
    const uint32_t incl = wave_incl_scan(v, op, id);
    // lane i - 1 across the whole wave (wave_shr:1); lane 0 takes the identity
    const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)incl, 0x138, 0xF, 0xF, false);
    if (total) *total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    return lane_id() == 0 ? id : prev;
  }
};

// A symbol's entry in mm: its token's lowest ranks as right and as left
// operand, packed as in Tables::tok_min, and its first byte's offset in the
// piece.
__device__ inline uint32_t low_right(uint2 v, uint32_t shift) { return (v.x >> 16) << shift; }
__device__ inline uint32_t low_left(uint2 v, uint32_t shift) { return (v.x & 0xFFFFu) << shift; }

// Shelter walks of the pair k (symbols k, k + 1) of rank r among n symbols;
// maxlen: bytes of the longest token.
__device__ inline bool sheltered(const uint32_t* rk, const uint2* mm, uint32_t n, uint32_t k, uint32_t r,
                                 uint32_t shift, uint32_t maxlen) {
  bool left = false;
  uint32_t i = k;
  const uint32_t end_x = mm[k + 1].y;  // the byte after x
  for (uint32_t s = 0; s <= kWalkMax; ++s) {
    const uint2 v = mm[i];
    if (low_right(v, shift) > r || i == 0 || end_x - v.y > maxlen) {  // symbols i .. k span more than a token
      left = true;
      break;
    }
    if (rank_of(rk[i - 1]) <= r) break;
    --i;
  }
  if (!left) return false;
  i = k + 1;
  const uint32_t start_y = mm[k + 1].y;
  for (uint32_t s = 0; s <= kWalkMax; ++s) {
    const uint2 v = mm[i];
    if (low_left(v, shift) > r || i == n - 1 || v.y - start_y > maxlen) return true;  // k + 1 .. i - 1 do
    if (rank_of(rk[i]) <= r) return false;
    ++i;
  }
  return false;
}

// BPE of the n-symbol piece held in sym / rk / mm (LDS or global memory), in
// rounds; returns the final symbol count.  Called by every thread with
// uniform arguments.  sym[i]: token i; rk[i]: rank of the pair (i, i + 1)
// (kNoRank for the last); mm[i]: the token's lowest ranks as right and left
// operand (packed) and its first byte's offset in the piece.
template <typename G, int E>
__device__ __forceinline__ uint32_t merge_piece(const Tables& T, uint32_t* sym, uint32_t* rk, uint2* mm,
                                                uint32_t n, uint32_t low, uint32_t* s_scan) {
  constexpr uint32_t kCap = G::kSize * E;  // symbols per chunk
  const uint32_t tid = G::rank();
  while (low != kNoRank) {  // uniform
    // pass A: which pairs merge; mark the chosen ones in rk
    uint32_t rs_carry = 0;  // 1 + the last pair before this chunk that does not merge (0: none)
    const uint32_t pairs = n - 1;
    for (uint32_t c0 = 0; c0 < pairs; c0 += kCap) {
      const uint32_t k0 = c0 + tid * E;
      bool take[E];
      uint32_t last_stop = 0;  // 1 + last non-merging pair among this thread's
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t k = k0 + e;
        take[e] = false;
        if (k < pairs) {
          const uint32_t r = rank_of(rk[k]);
          take[e] = r != kNoRank && (r == low || sheltered(rk, mm, n, k, r, T.min_shift, T.max_tok_len));
          if (!take[e]) last_stop = k + 1;
        }
      }
      uint32_t total = 0;
      const uint32_t before = MaxOp()(rs_carry, G::excl_scan(last_stop, 0u, MaxOp(), s_scan, &total));
      uint32_t rs = before;  // run start of this thread's first pair
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t k = k0 + e;
        if (k < pairs) {
          if (take[e] && ((k - rs) & 1u) == 0u) rk[k] |= kChosen;
          if (!take[e]) rs = k + 1;
        }
      }
      rs_carry = __builtin_amdgcn_readfirstlane(MaxOp()(rs_carry, total));
      G::sync();  // marks visible before the next chunk's walks
    }
    // pass B: compaction, chunk by chunk in place (a symbol only moves down);
    // pairs next to a merge are probed again
    uint32_t removed = 0;        // symbols removed before this chunk
    bool prev_chosen = false;    // the last pair before this chunk merged
    uint32_t new_low = kNoRank;
    for (uint32_t c0 = 0; c0 < n; c0 += kCap) {
      const uint32_t i0 = c0 + tid * E;
      uint32_t ns[E], nr[E];
      uint2 nm[E];
      bool alive[E], chose[E];
      uint32_t mine = 0;  // chosen pairs among this thread's positions
      bool pc = i0 == c0 ? prev_chosen : (i0 < n && chosen_bit(rk[i0 - 1]));
#pragma unroll
      for (int e = 0; e < E; ++e) {
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
            nm[e] = ch ? make_uint2(T.tok_min[ns[e]], mm[i].y) : mm[i];  // a merged token starts where its left part did
            const uint32_t kn = ch ? i + 2 : i + 1;
            nr[e] = kNoRank;
            if (kn < n) {
              const uint32_t vn = rk[kn];
              const bool chn = chosen_bit(vn);
              if (ch || chn) nr[e] = merge_rank(T, ns[e], chn ? 256u + rank_of(vn) : sym[kn]);
              else nr[e] = rank_of(v);
            }
          }
          mine += ch ? 1u : 0u;
          pc = ch;
        }
      }
      uint32_t chunk_chosen = 0;
      const uint32_t before = G::excl_scan(mine, 0u, AddOp(), s_scan, &chunk_chosen);
      // the last pair of this chunk, for the next chunk's first symbol (read
      // before any write of this chunk: the scan above holds barriers)
      const uint32_t last = min(c0 + kCap, n) - 1;
      const bool last_chosen = last + 1 < n && chosen_bit(rk[last]);
      G::sync();
      // symbol i moves to i less the chosen pairs before it; a symbol absorbed
      // by the pair before it is not written (its index is its partner's)
      uint32_t q = i0 - removed - before;
#pragma unroll
      for (int e = 0; e < E; ++e) {
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
      G::sync();
    }
    n -= removed;
    uint32_t all = 0;
    (void)G::excl_scan(new_low, kNoRank, MinOp(), s_scan, &all);
    low = __builtin_amdgcn_readfirstlane(all);
  }
  return n;
}


// BPE of the long piece text[s .. s + len) by the group G: its bytes become
// the symbols in sym / rk / mm, the rounds run, and its tokens are left in
// out[0 ..] (the global workspace at the piece's bytes; when the arrays are
// that workspace already, nothing moves).  Returns the token count.  Called
// by every thread of the group with uniform arguments.
template <typename G, int E>
__device__ __forceinline__ uint32_t long_piece(const uint8_t* __restrict__ text, uint64_t s, uint32_t len,
                                               const Tables& T, uint32_t* sym, uint32_t* rk, uint2* mm,
                                               uint32_t* out, uint32_t* s_scan) {
  constexpr uint32_t NT = G::kSize;
  const uint32_t tid = G::rank();
  uint32_t low = kNoRank;
  for (uint32_t i = tid; i < len; i += NT) {
    const uint32_t a = text[s + i];
    sym[i] = a;
    const uint32_t r = i + 1 < len ? T.pair_rank[(a << 8) | text[s + i + 1]] : kNoRank;
    rk[i] = r;
    mm[i] = make_uint2(T.tok_min[a], i);
    low = min(low, r);
  }
  uint32_t all = 0;
  if (!G::kScanSyncs) G::sync();  // the stores above before any read of them
  (void)G::excl_scan(low, kNoRank, MinOp(), s_scan, &all);
  const uint32_t cnt = __builtin_amdgcn_readfirstlane(
      merge_piece<G, E>(T, sym, rk, mm, len, __builtin_amdgcn_readfirstlane(all), s_scan));
  if (sym != out)
    for (uint32_t i = tid; i < cnt; i += NT) out[i] = sym[i];
  return cnt;
}

}  // namespace longp
}  // namespace tok
