// Pure helpers of the merge kernels (no memory access), shared with the CPU
// build used by the tests.
#pragma once

#include <stdint.h>

#ifndef TOK_HD
#define TOK_HD __host__ __device__
#endif

namespace tok {

// Leftmost non-overlapping choice among 64 consecutive pair positions.
//
// m: bit j set iff the pair at position j has the round's minimum rank.
// carry: 1 iff the pair just before bit 0 was chosen (it consumed the left
// symbol of pair 0).  Occurrences of one pair value overlap only inside runs
// of one repeated symbol ("aaaa" under the merge (a, a)); sequential BPE takes
// them from left to right, i.e. every other position of each run starting with
// its first (GraphTok, section 4 "Warp-cooperative BPE": a round takes every
// other pair of a chain; TokTier, "Exact GPU Tokenization": merging all
// leftmost non-overlapping occurrences of the minimum-rank pair equals
// iterated single merges).
//
// Closed form: a run that starts at an even bit keeps its even bits, a run
// that starts at an odd bit keeps its odd bits.  Adding the odd run starts to
// m clears exactly the bits of the runs that begin there (the carry stops at
// the zero after each run), which separates the two kinds of runs.  A run
// through bit 0 after a chosen pair behaves as if it had started at bit -1.
TOK_HD inline uint64_t select_leftmost(uint64_t m, uint32_t carry) {
  const uint64_t even = 0x5555555555555555ull;
  uint64_t starts = m & ~(m << 1);
  uint64_t odd_starts = starts & ~even;
  if (carry && (m & 1ull)) odd_starts |= 1ull;
  const uint64_t odd_runs = m & ~(m + odd_starts);
  return (odd_runs & ~even) | (m & ~odd_runs & even);
}

}  // namespace tok
