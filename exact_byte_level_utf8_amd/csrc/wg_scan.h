// Wave64 / workgroup scans and reductions over small monoid elements packed in
// 32 bits.  Order matters (the monoids are not commutative): element i is
// combined with element i+1 as op(e_i, e_{i+1}).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tok {

constexpr int kWave = 64;

__device__ inline uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// inclusive prefix over the lanes of one wave
template <typename Op>
__device__ inline uint32_t wave_incl_scan(uint32_t v, Op op) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, kWave);
    if (lane >= (uint32_t)d) v = op(o, v);
  }
  return v;
}

// inclusive suffix over the lanes of one wave: op(e_i, op(e_{i+1}, ...))
template <typename Op>
__device__ inline uint32_t wave_incl_suffix(uint32_t v, Op op) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_down(v, d, kWave);
    if (lane + d < (uint32_t)kWave) v = op(v, o);
  }
  return v;
}

// Exclusive prefix over the workgroup (blockDim.x = NT, a multiple of 64),
// and the total.  scratch: NT / 64 words of LDS.  Contains barriers: call
// from all threads.
template <int NT, typename Op>
__device__ inline uint32_t wg_excl_scan(uint32_t v, uint32_t id, Op op, uint32_t* scratch,
                                        uint32_t* total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, op);
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  uint32_t before = id;
  for (uint32_t i = 0; i < w; ++i) before = op(before, scratch[i]);
  uint32_t all = id;
#pragma unroll
  for (int i = 0; i < NW; ++i) all = op(all, scratch[i]);
  uint32_t excl = __shfl_up(incl, 1, kWave);
  excl = lane == 0 ? before : op(before, excl);
  __syncthreads();  // scratch may be reused right after
  if (total) *total = all;
  return excl;
}

// Exclusive suffix over the workgroup: op(e_{i+1}, op(e_{i+2}, ...)), and
// the total op(e_0, ...).
template <int NT, typename Op>
__device__ inline uint32_t wg_excl_suffix(uint32_t v, uint32_t id, Op op, uint32_t* scratch,
                                          uint32_t* total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_suffix(v, op);
  if (lane == 0) scratch[w] = incl;
  __syncthreads();
  uint32_t after = id;
  for (int i = NW - 1; i > (int)w; --i) after = op(scratch[i], after);
  uint32_t all = id;
#pragma unroll
  for (int i = NW - 1; i >= 0; --i) all = op(scratch[i], all);
  uint32_t excl = __shfl_down(incl, 1, kWave);
  excl = lane == kWave - 1 ? after : op(excl, after);
  __syncthreads();
  if (total) *total = all;
  return excl;
}

struct AddOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};

}  // namespace tok
