// Decoupled look-back over tiles taken in dispatch order (each workgroup
// takes a ticket), for the exclusive prefix of per-tile token counts.
#pragma once

#include "tok_internal.h"

namespace tok {

// state word: bits 62-63 flag, bits 0-31 value
constexpr unsigned long long kLbAgg = 1ull << 62, kLbPre = 2ull << 62;
constexpr uint32_t kLbSpinLimit = 1u << 22;

// Called by one whole wave.  Publishes this tile's aggregate, sums the
// predecessors' states 64 at a time until one holds an inclusive prefix, then
// publishes this tile's inclusive prefix.  Every value that steers the loops
// is wave-uniform (ballots, counters) and no lane-specific branch sits inside
// them, so the wave stays together.  Each state word carries its flag and
// value together and nothing else is published through it, so relaxed
// device-scope atomics suffice: acquire and release would add an L2 write-back
// or invalidate per access on a multi-die part.  A predecessor that never publishes ends
// the wait after a bounded number of polls with kStSpin set.
__device__ inline uint32_t look_back(unsigned long long* state, uint32_t tile, uint32_t total, Counters* ctr) {
  const uint32_t lane = threadIdx.x & 63u;
  if (tile == 0) {
    if (lane == 0) __hip_atomic_store(&state[0], kLbPre | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0) __hip_atomic_store(&state[tile], kLbAgg | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t base = 0, spins = 0;
  bool stuck = false;
  int64_t top = (int64_t)tile - 1;
  while (top >= 0) {
    const int64_t i = top - lane;
    unsigned long long v = kLbPre;  // past tile 0: an empty prefix
    if (i >= 0) v = __hip_atomic_load(&state[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (__ballot((v >> 62) == 0)) {
      if (++spins > kLbSpinLimit) {
        stuck = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if ((v >> 62) == 0) v = __hip_atomic_load(&state[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (stuck) break;
    const uint64_t pre = __ballot((v & kLbPre) != 0);
    const uint32_t upto = pre ? (uint32_t)__builtin_ctzll(pre) : 63u;  // lanes 0..upto count
    uint32_t add = lane <= upto ? (uint32_t)v : 0u;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) add += __shfl_xor(add, d, 64);
    base += __builtin_amdgcn_readfirstlane(add);
    if (pre) break;
    top -= 64;
  }
  if (stuck) {
    if (lane == 0) atomicOr(&ctr->status, kStSpin);
    return base;
  }
  if (lane == 0)
    __hip_atomic_store(&state[tile], kLbPre | (uint32_t)(base + total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return base;
}

}  // namespace tok
