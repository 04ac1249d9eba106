// Per-call reset and output assembly.
//
// reset_kernel clears the device counters and the look-back state of the
// token-count scan with stores from a kernel (never a memset node, so the
// sequence stays correct when a caller captures it in a graph), checks batch
// offsets, and answers the degenerate empty batch.
//
// assemble_kernel places each tile's run of IDs in the output: one workgroup
// per tile, taken in dispatch order, finds the tile's output offset by a
// decoupled look-back over the tile counts and copies the run with coalesced
// loads and stores (GraphTok, section 4: the fused assembly scans output
// lengths, restores document order and writes the result).  It also turns
// the in-run offsets of the documents that start in the tile into output
// offsets.
#include "tok_internal.h"
#include "lookback.h"
#include "wg_scan.h"

namespace tok {
namespace {

__global__ void reset_kernel(Bufs B, uint32_t n_tiles, const uint64_t* doc_off, uint32_t n_docs, uint64_t n,
                             uint64_t* out_off) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t stride = gridDim.x * blockDim.x;
  if (i == 0) {
    B.ctr->ticket = 0;
    B.ctr->total = 0;
    uint32_t st = 0;
    if (doc_off && (doc_off[0] != 0 || doc_off[n_docs] != n)) st |= kStDocOff;
    B.ctr->status = st;
  }
  for (uint32_t t = i; t < n_tiles; t += stride) B.scan_state[t] = 0;
  if (doc_off) {
    for (uint32_t d = i; d < n_docs; d += stride)
      if (doc_off[d] > doc_off[d + 1]) atomicOr(&B.ctr->status, kStDocOff);
    if (n == 0 && out_off)  // no tile runs: every document is empty
      for (uint32_t d = i; d <= n_docs; d += stride) out_off[d] = 0;
  }
}

__global__ void __launch_bounds__(kThreads)
assemble_kernel(uint64_t n, Bufs B, int32_t* __restrict__ out, uint64_t cap, const uint64_t* __restrict__ doc_off,
                uint32_t n_docs, uint64_t* __restrict__ out_off) {
  __shared__ uint32_t s_tile, s_base, s_doc0;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) s_tile = atomicAdd(&B.ctr->ticket, 1u);  // tiles in dispatch order
  __syncthreads();
  const uint32_t tile = __builtin_amdgcn_readfirstlane(s_tile);
  const bool last = tile == gridDim.x - 1;
  const uint32_t cnt = __builtin_amdgcn_readfirstlane(B.tile_cnt[tile]);
  if (tid < (uint32_t)kWave) {
    const uint32_t base = look_back(B.scan_state, tile, cnt, B.ctr);
    if (tid == 0) {
      s_base = base;
      if (last) B.ctr->total = base + cnt;
    }
  }
  if (doc_off && tid == kWave) s_doc0 = first_doc_at_or_after(doc_off, n_docs, (uint64_t)tile * kPieceTile);
  __syncthreads();
  const uint64_t base = __builtin_amdgcn_readfirstlane(s_base);
  const int32_t* run = B.staging + B.tile_first[tile];
  for (uint32_t i = tid; i < cnt; i += kThreads)
    if (base + i < cap) out[base + i] = run[i];
  if (doc_off) {
    const uint64_t t0 = (uint64_t)tile * kPieceTile;
    for (uint32_t d = s_doc0 + tid; d <= n_docs; d += kThreads) {
      const uint64_t p = doc_off[d];
      if (p >= n) {
        if (!last) break;
        out_off[d] = base + cnt;  // documents that start at the end of the text
        continue;
      }
      if (p >= t0 + kPieceTile) break;
      out_off[d] += base;  // the piece pass stored the offset within the tile's run
    }
  }
}

}  // namespace

void launch_reset(Bufs b, uint32_t n_tiles, const uint64_t* doc_off, uint32_t n_docs, uint64_t n,
                  uint64_t* out_off, hipStream_t s) {
  uint32_t work = n_tiles > n_docs + 1 ? n_tiles : n_docs + 1;
  uint32_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  reset_kernel<<<blocks, 256, 0, s>>>(b, n_tiles, doc_off, n_docs, n, out_off);
}

}  // namespace tok

namespace tok {

void launch_assemble(uint64_t n, Bufs b, int32_t* out, uint64_t cap, const uint64_t* doc_off,
                     uint32_t n_docs, uint64_t* out_off, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
  if (tiles) assemble_kernel<<<tiles, kThreads, 0, s>>>(n, b, out, cap, doc_off, n_docs, out_off);
}

}  // namespace tok
