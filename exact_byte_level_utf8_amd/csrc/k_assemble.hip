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
    B.ctr->n_list[0] = 0;
    B.ctr->n_list[1] = 0;
    B.ctr->n_list[2] = 0;
    B.ctr->work = 0;
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

// Wave 0 of the workgroup finds the exclusive prefix of this tile from its
// predecessors' published states, 64 at a time (decoupled look-back).
__device__ uint32_t look_back(unsigned long long* state, uint32_t tile, uint32_t total, Counters* ctr) {
  const uint32_t lane = threadIdx.x & 63u;
  if (tile == 0) {
    if (lane == 0) __hip_atomic_store(&state[0], kPre | total, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0) __hip_atomic_store(&state[tile], kAgg | total, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  // Every value that steers these loops is wave-uniform (ballots, counters),
  // and no lane-specific branch sits inside them, so the wave stays together.
  uint32_t base = 0, spins = 0;
  bool stuck = false;
  int64_t top = (int64_t)tile - 1;
  while (top >= 0) {
    const int64_t i = top - lane;
    unsigned long long v = kPre;  // past tile 0: an empty prefix
    if (i >= 0) v = __hip_atomic_load(&state[i], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    while (__ballot((v >> 62) == 0)) {
      if (++spins > kSpinLimit) {
        stuck = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if ((v >> 62) == 0) v = __hip_atomic_load(&state[i], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (stuck) break;
    const uint64_t pre = __ballot((v & kPre) != 0);
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
    __hip_atomic_store(&state[tile], kPre | (uint32_t)(base + total), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return base;
}

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
  if (tid < kWave) {
    const uint32_t base = look_back(B.scan_state, tile, total, B.ctr);
    if (tid == 0) {
      s_base = base;
      if (tile == gridDim.x - 1) B.ctr->total = base + total;
    }
  }
  __syncthreads();
  const uint64_t excl = (uint64_t)s_base + excl_local;
  if (c < n_chunks) {
    B.chunk_excl[c] = (uint32_t)excl;
    uint32_t w = B.flags[c];
    uint32_t done = 0;
    while (w && done < cnt) {
      const uint32_t b = __builtin_ctz(w);
      w &= w - 1;
      const uint64_t s = c * kChunk + b;
      const uint32_t k = w ? B.cnt8[s] : cnt - done;  // the chunk's last piece takes the rest
      const int32_t* src = B.staging + s;
      for (uint32_t j = 0; j < k; ++j)
        if (excl + done + j < cap) out[excl + done + j] = src[j];
      done += k;
    }
  }
}

// out_off[d] = tokens of the pieces that start before doc_off[d]: the chunk's
// exclusive offset plus the counts of the chunk's pieces before that byte.
__global__ void doc_offsets_kernel(uint64_t n, const uint64_t* __restrict__ doc_off, uint32_t n_docs,
                                   uint64_t* __restrict__ out_off, Bufs B) {
  const uint32_t d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d > n_docs) return;
  const uint64_t p = doc_off[d];
  if (p >= n) {
    out_off[d] = B.ctr->total;
    return;
  }
  const uint64_t c = p / kChunk;
  uint32_t before = B.flags[c] & ((1u << (p % kChunk)) - 1u);
  uint64_t k = B.chunk_excl[c];
  while (before) {
    k += B.cnt8[c * kChunk + __builtin_ctz(before)];
    before &= before - 1;
  }
  out_off[d] = k;
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
  (void)t;
  const uint32_t blocks = (n_docs + 1 + 255) / 256;
  doc_offsets_kernel<<<blocks, 256, 0, s>>>(n, doc_off, n_docs, out_off, b);
}

}  // namespace tok
