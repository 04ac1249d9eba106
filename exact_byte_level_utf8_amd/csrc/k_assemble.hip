// Assembly kernels: counter reset, token-count scan + scatter into the compact
// output, and per-document output offsets (GraphTok, section 4: the fused
// assembly scans output lengths, restores document order and writes the
// result; TokTier, "Exact GPU Tokenization": counts and output length stay in
// device memory).
#include "tok_internal.h"
#include "wg_scan.h"

namespace tok {
namespace {

// Clears the device counters and the look-back state of the count scan with
// stores from a kernel (never a memset node, so the sequence stays correct
// when a caller captures it in a graph), and checks batch offsets.
__global__ void reset_kernel(Bufs B, uint32_t n_tiles, const uint64_t* doc_off, uint32_t n_docs,
                             uint64_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    B.ctr->n_long = 0;
    B.ctr->k3_ticket = 0;
    B.ctr->total = 0;
    uint32_t st = 0;
    if (doc_off && (doc_off[0] != 0 || doc_off[n_docs] != n)) st |= kStDocOff;
    B.ctr->status = st;
  }
  for (uint32_t t = i; t < n_tiles; t += gridDim.x * blockDim.x) B.scan_state[t] = 0;
  if (doc_off) {
    for (uint32_t d = i; d < n_docs; d += gridDim.x * blockDim.x)
      if (doc_off[d] > doc_off[d + 1]) atomicOr(&B.ctr->status, kStDocOff);
  }
}

// decoupled look-back state: bits 62-63 flag, bits 0-31 value
constexpr unsigned long long kAgg = 1ull << 62, kPre = 2ull << 62;
constexpr uint32_t kSpinLimit = 1u << 22;

__global__ void __launch_bounds__(kThreads)
assemble_kernel(uint64_t n, int32_t* __restrict__ out, uint64_t cap, Bufs B) {
  __shared__ uint32_t s_scan[kThreads / kWave];
  __shared__ uint32_t s_tile, s_base;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) s_tile = atomicAdd(&B.ctr->k3_ticket, 1u);
  __syncthreads();
  const uint32_t tile = s_tile;
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  const uint64_t c = (uint64_t)tile * kThreads + tid;
  const uint32_t cnt = c < n_chunks ? B.chunk_cnt[c] : 0u;
  uint32_t total;
  const uint32_t excl_local = wg_excl_scan<kThreads>(cnt, 0u, AddOp(), s_scan, &total);
  if (tid == 0) {
    uint32_t base = 0;
    if (tile == 0) {
      __hip_atomic_store(&B.scan_state[0], kPre | total, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(&B.scan_state[tile], kAgg | total, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      int64_t i = (int64_t)tile - 1;
      uint32_t spins = 0;
      while (i >= 0) {
        const unsigned long long v =
            __hip_atomic_load(&B.scan_state[i], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long f = v & (3ull << 62);
        if (f == 0) {
          if (++spins > kSpinLimit) {
            atomicOr(&B.ctr->status, kStSpin);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        base += (uint32_t)v;
        if (f == kPre) break;
        --i;
      }
      __hip_atomic_store(&B.scan_state[tile], kPre | (uint32_t)(base + total), __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    s_base = base;
    if (tile == gridDim.x - 1) B.ctr->total = base + total;
  }
  __syncthreads();
  const uint64_t excl = (uint64_t)s_base + excl_local;
  if (c < n_chunks) {
    B.chunk_excl[c] = (uint32_t)excl;
    if (cnt) {
      const uint64_t first = c * kChunk + __builtin_ctz((uint32_t)B.flags[c]);
      const int32_t* src = B.staging + first;
      for (uint32_t k = 0; k < cnt; ++k)
        if (excl + k < cap) out[excl + k] = src[k];
    }
  }
}

// out_off[d] = number of tokens of the pieces that start before doc_off[d]:
// the chunk's exclusive offset plus the tokens of the chunk's pieces before
// the document start, counted by their byte lengths.
__global__ void doc_offsets_kernel(uint64_t n, const uint64_t* __restrict__ doc_off, uint32_t n_docs,
                                   uint64_t* __restrict__ out_off, Tables T, Bufs B) {
  const uint32_t d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d > n_docs) return;
  const uint64_t p = doc_off[d];
  if (p >= n) {
    out_off[d] = B.ctr->total;
    return;
  }
  const uint64_t c = p / kChunk;
  const uint32_t w = B.flags[c];
  const uint32_t before = w & ((1u << (p % kChunk)) - 1u);
  uint64_t k = 0;
  if (before) {
    const uint64_t first = c * kChunk + __builtin_ctz(w);
    const uint64_t need = p - first;
    const uint32_t cnt = B.chunk_cnt[c];
    uint64_t got = 0;
    while (got < need && k < cnt) got += T.tok_len[B.staging[first + k++]];
  }
  out_off[d] = B.chunk_excl[c] + k;
}

}  // namespace

void launch_reset(Bufs b, uint32_t n_tiles, const uint64_t* doc_off, uint32_t n_docs, uint64_t n,
                  hipStream_t s) {
  uint32_t work = n_tiles > n_docs ? n_tiles : n_docs;
  uint32_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  reset_kernel<<<blocks, 256, 0, s>>>(b, n_tiles, doc_off, n_docs, n);
}

void launch_assemble(uint64_t n, int32_t* out, uint64_t cap, Bufs b, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kTile - 1) / kTile);
  if (tiles) assemble_kernel<<<tiles, kThreads, 0, s>>>(n, out, cap, b);
}

void launch_doc_offsets(uint64_t n, const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off,
                        Tables t, Bufs b, hipStream_t s) {
  const uint32_t blocks = (n_docs + 1 + 255) / 256;
  doc_offsets_kernel<<<blocks, 256, 0, s>>>(n, doc_off, n_docs, out_off, t, b);
}

}  // namespace tok
