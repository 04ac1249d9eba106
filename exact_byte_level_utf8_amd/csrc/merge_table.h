// Lookup of a merge's rank in the device merge table, shared by the piece
// pass's rows and its long-piece rounds.
#pragma once

#include "tok_internal.h"

namespace tok {

// Rank held by one merge-table slot, or kNoRank.  A slot is left << 44 |
// right << 24 | rank, so its high dword is left << 12 | right >> 8 (khi) and
// the top byte of its low dword is right & 0xFF (klo); an empty slot (all
// ones) never matches, since token IDs stay below 2^20 - 1 (TOK_MAX_MERGES)
// and khi is then never all ones.
__device__ inline uint32_t slot_rank(ulonglong2 two, int which, uint32_t khi, uint32_t klo) {
  const uint64_t v = which ? two.y : two.x;
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  return hi == khi && (lo >> 24) == klo ? (lo & 0xFFFFFFu) : kNoRank;
}

__device__ inline uint32_t bucket_rank(ulonglong2 s01, ulonglong2 s23, uint32_t khi, uint32_t klo) {
  return min(min(slot_rank(s01, 0, khi, klo), slot_rank(s01, 1, khi, klo)),
             min(slot_rank(s23, 0, khi, klo), slot_rank(s23, 1, khi, klo)));
}

// The rest of a lookup whose first bucket h was full without the key (rare:
// the table is at most half full): the following buckets in turn, until the
// key or a bucket with a free slot.
__device__ inline uint32_t merge_rank_rest(const Tables& T, uint32_t khi, uint32_t klo, uint32_t h) {
  for (uint32_t probe = 1; probe < T.merge_buckets; ++probe) {
    h = next_bucket(h, T.merge_buckets);
    const ulonglong2* bk = reinterpret_cast<const ulonglong2*>(T.merge_slots + (size_t)h * kBucket);
    const ulonglong2 t01 = bk[0], t23 = bk[1];
    const uint32_t r = bucket_rank(t01, t23, khi, klo);
    if (r != kNoRank || t23.y == kEmptySlot) return r;
  }
  return kNoRank;
}

// Rank of the merge (a, b), or kNoRank (callers use it for a pair next to a
// merge, where a or b is a merged token and the byte-pair table never
// applies).  Open addressing over buckets of kBucket slots, each read with
// two 16-byte loads; the first bucket is compared without branches, and only
// a full first bucket without the key goes on to the next ones.
__device__ inline uint32_t merge_rank(const Tables& T, uint32_t a, uint32_t b) {
  const uint32_t khi = (a << 12) | (b >> 8), klo = b & 0xFFu;
  const uint32_t h = merge_bucket(a, b, T.merge_buckets);
  const ulonglong2* bk = reinterpret_cast<const ulonglong2*>(T.merge_slots + (size_t)h * kBucket);
  const ulonglong2 s01 = bk[0], s23 = bk[1];
  const uint32_t r = bucket_rank(s01, s23, khi, klo);
  // slots fill in order within a bucket
  return r == kNoRank && s23.y != kEmptySlot ? merge_rank_rest(T, khi, klo, h) : r;
}

}  // namespace tok
