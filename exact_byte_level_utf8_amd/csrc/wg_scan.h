// Wave64 / workgroup scans and reductions over small monoid elements packed in
// 32 bits.  Order matters (the monoids are not commutative): element i is
// combined with element i+1 as op(e_i, e_{i+1}).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tok {

constexpr int kWave = 64;

__device__ inline uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// Value of lane i - D (prefix direction) or i + D (suffix direction) of the
// same 16-lane row, by DPP row_shr / row_shl; lanes whose source lies outside
// the row get `id`.
template <int D>
__device__ inline uint32_t row_from_below(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x110 + D, 0xF, 0xF, false);  // row_shr:D
}
template <int D>
__device__ inline uint32_t row_from_above(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x100 + D, 0xF, 0xF, false);  // row_shl:D
}

// inclusive prefix over the lanes of one wave: in-row steps by DPP, then the
// totals of the lower rows (read as scalars) in front.  id: the identity.
template <typename Op>
__device__ inline uint32_t wave_incl_scan(uint32_t v, Op op, uint32_t id) {
  v = op(row_from_below<1>(v, id), v);
  v = op(row_from_below<2>(v, id), v);
  v = op(row_from_below<4>(v, id), v);
  v = op(row_from_below<8>(v, id), v);
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 15), r1 = __builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 47);
  const uint32_t row = lane_id() >> 4;
  const uint32_t b1 = r0, b2 = op(r0, r1), b3 = op(b2, r2);
  const uint32_t before = row == 0 ? id : row == 1 ? b1 : row == 2 ? b2 : b3;
  return op(before, v);
}

// inclusive suffix over the lanes of one wave: op(e_i, op(e_{i+1}, ...))
template <typename Op>
__device__ inline uint32_t wave_incl_suffix(uint32_t v, Op op, uint32_t id) {
  v = op(v, row_from_above<1>(v, id));
  v = op(v, row_from_above<2>(v, id));
  v = op(v, row_from_above<4>(v, id));
  v = op(v, row_from_above<8>(v, id));
  const uint32_t r1 = __builtin_amdgcn_readlane((int)v, 16), r2 = __builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = __builtin_amdgcn_readlane((int)v, 48);
  const uint32_t row = lane_id() >> 4;
  const uint32_t a2 = r3, a1 = op(r2, r3), a0 = op(r1, a1);
  const uint32_t after = row == 3 ? id : row == 2 ? a2 : row == 1 ? a1 : a0;
  return op(v, after);
}

// Exclusive prefix over the workgroup (blockDim.x = NT, a multiple of 64),
// and the total.  scratch: NT / 64 words of LDS.  Contains barriers: call
// from all threads.
template <int NT, typename Op>
__device__ inline uint32_t wg_excl_scan(uint32_t v, uint32_t id, Op op, uint32_t* scratch,
                                        uint32_t* total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, op, id);
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  uint32_t before = id;
  for (uint32_t i = 0; i < w; ++i) before = op(before, scratch[i]);
  uint32_t all = id;
#pragma unroll
  for (int i = 0; i < NW; ++i) all = op(all, scratch[i]);
  // lane i - 1 across the whole wave (wave_shr:1); lane 0 takes the identity
  const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)incl, 0x138, 0xF, 0xF, false);
  const uint32_t excl = lane == 0 ? before : op(before, prev);
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
  const uint32_t incl = wave_incl_suffix(v, op, id);
  if (lane == 0) scratch[w] = incl;
  __syncthreads();
  uint32_t after = id;
  for (int i = NW - 1; i > (int)w; --i) after = op(scratch[i], after);
  uint32_t all = id;
#pragma unroll
  for (int i = NW - 1; i >= 0; --i) all = op(scratch[i], all);
  // lane i + 1 across the whole wave (wave_shl:1); lane 63 takes the identity
  const uint32_t next = (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)incl, 0x130, 0xF, 0xF, false);
  const uint32_t excl = lane == kWave - 1 ? after : op(next, after);
  __syncthreads();
  if (total) *total = all;
  return excl;
}

struct AddOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MinOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct MaxOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

}  // namespace tok
