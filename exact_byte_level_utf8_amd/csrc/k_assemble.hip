// Output assembly: one workgroup per 1 KiB tile places the tile's run of IDs.
//
// The tile's output offset is the sum of the token counts of all earlier
// tiles.  The piece pass left three levels of counts (per tile, per aligned
// group of 64 tiles, per group of 4096), so a workgroup reads at most 63 tile
// counts, 63 group counts and G / 4096 large-group counts and reduces them:
// no workgroup waits for another, and the cost per tile stays bounded for
// any input up to the size limit.  The run is then copied with coalesced
// loads and stores (GraphTok, section 4: the assembly scans output lengths,
// restores document order and writes the result), and the documents that
// start in the tile get their output offsets.  The last tile publishes the
// total.
//
// With span export on, each ID also gets the byte where its token starts
// (TokTier, section 7 "Session-state construction" and Appendix E, "Route C:
// GPU full tokenization with span export": gather each token's byte length,
// a cumulative sum gives the offsets).  A tile's run covers the text
// contiguously from its first piece start, so the offsets are that byte plus
// a workgroup scan of the lengths along the run: no scan crosses tiles.
#include "tok_internal.h"
#include "wg_scan.h"

namespace tok {
namespace {

constexpr uint32_t kAsmThreads = 256;

template <bool SPANS>
__global__ void __launch_bounds__(kAsmThreads)
assemble_kernel(uint64_t n, Bufs B, int32_t* __restrict__ out, uint32_t* __restrict__ spans,
                const uint32_t* __restrict__ tok_len, uint64_t cap, const uint64_t* __restrict__ doc_off,
                uint32_t n_docs, uint64_t* __restrict__ out_off) {
  __shared__ uint32_t s_part[kAsmThreads / kWave];
  __shared__ uint32_t s_scan[kAsmThreads / kWave];
  __shared__ uint32_t s_doc0;
  if (B.n_docs_dev) n_docs = *B.n_docs_dev;
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t tile = blockIdx.x;
  const bool last = tile == gridDim.x - 1;
  if (doc_off && tid == 0) s_doc0 = first_doc_at_or_after(doc_off, n_docs, (uint64_t)tile * kPieceTile);

  // counts before this tile: large groups, then groups of the current large
  // group, then tiles of the current group
  const uint32_t g2 = tile >> kSum2Shift, g1 = tile >> kSum1Shift;
  const uint32_t g1_lo = g2 << (kSum2Shift - kSum1Shift), t_lo = g1 << kSum1Shift;
  uint32_t part = 0;
  for (uint32_t i = tid; i < g2; i += kAsmThreads) part += B.sum2[i];
  if (tid < 64u) {
    if (g1_lo + tid < g1) part += B.sum1[g1_lo + tid];
  } else if (tid < 128u) {
    if (t_lo + (tid - 64u) < tile) part += B.tile_cnt[t_lo + (tid - 64u)];
  }
  part = wave_incl_scan(part, AddOp(), 0u);
  if (lane == 63u) s_part[tid >> 6] = part;
  __syncthreads();
  const uint32_t base = __builtin_amdgcn_readfirstlane(s_part[0] + s_part[1] + s_part[2] + s_part[3]);
  const uint32_t cnt = __builtin_amdgcn_readfirstlane(B.tile_cnt[tile]);
  const uint32_t first = __builtin_amdgcn_readfirstlane(B.tile_first[tile]);
  const int32_t* run = B.staging + first;
  if constexpr (SPANS) {
    // uniform trip count: the scan inside holds barriers
    uint32_t at = first;
    for (uint32_t i0 = 0; i0 < cnt; i0 += kAsmThreads) {
      const uint32_t i = i0 + tid;
      const int32_t id = i < cnt ? run[i] : 0;
      const uint32_t len = i < cnt ? tok_len[id] : 0u;
      uint32_t chunk = 0;
      const uint32_t before = wg_excl_scan<kAsmThreads>(len, 0u, AddOp(), s_scan, &chunk);
      if (i < cnt && (uint64_t)base + i < cap) {
        out[base + i] = id;
        spans[base + i] = at + before;
      }
      at += chunk;
    }
  } else {
    for (uint32_t i = tid; i < cnt; i += kAsmThreads)
      if ((uint64_t)base + i < cap) out[base + i] = run[i];
  }
  if (last && tid == 0) {
    B.ctr->total = base + cnt;
    __threadfence_system();
    report(&B.ctr->done, B.gen);
  }
  if (doc_off) {
    const uint64_t t0 = (uint64_t)tile * kPieceTile;
    for (uint32_t d = s_doc0 + tid; d <= n_docs; d += kAsmThreads) {
      const uint64_t p = doc_off[d];
      if (p >= n) {
        if (!last) break;
        out_off[d] = base + cnt;  // documents that start at the end of the text
        continue;
      }
      if (p >= t0 + kPieceTile) break;
      if (p < t0) continue;  // only with unordered offsets, which the call rejects
      out_off[d] += base;    // the piece pass stored the offset within the tile's run
    }
  }
}

// A batch whose documents are all empty: every offset must be 0, and every
// output offset is 0.
__global__ void empty_batch_kernel(Bufs B, const uint64_t* __restrict__ doc_off, uint32_t n_docs,
                                   uint64_t* __restrict__ out_off) {
  bool bad = false;
  for (uint32_t d = blockIdx.x * blockDim.x + threadIdx.x; d <= n_docs; d += gridDim.x * blockDim.x) {
    bad |= doc_off[d] != 0;
    out_off[d] = 0;
  }
  if (bad) report(&B.ctr->err_docs, B.gen);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    B.ctr->total = 0;
    __threadfence_system();
    report(&B.ctr->done, B.gen);
  }
}

}  // namespace

void launch_assemble(uint64_t n, Bufs b, int32_t* out, uint32_t* spans, const uint32_t* tok_len, uint64_t cap,
                     const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off, hipStream_t s, hipEvent_t e0,
                     hipEvent_t e1) {
  const uint32_t tiles = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
  if (!tiles) return;
  if (spans)
    launch_on(assemble_kernel<true>, dim3(tiles), dim3(kAsmThreads), s, e0, e1, n, b, out, spans, tok_len, cap,
              doc_off, n_docs, out_off);
  else
    launch_on(assemble_kernel<false>, dim3(tiles), dim3(kAsmThreads), s, e0, e1, n, b, out, spans, tok_len, cap,
              doc_off, n_docs, out_off);
}

void launch_empty_batch(Bufs b, const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off, hipStream_t s) {
  const uint32_t blocks = (uint32_t)std::min<uint64_t>(((uint64_t)n_docs + 256u) / 256u, 1024u);
  empty_batch_kernel<<<blocks, 256, 0, s>>>(b, doc_off, n_docs, out_off);
}

}  // namespace tok
