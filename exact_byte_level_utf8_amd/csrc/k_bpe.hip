// Merge kernels: byte-level BPE of every piece by lowest merge rank.
//
// BPE never crosses a piece boundary, so pieces are independent; inside a
// piece the merges are ordered (GraphTok, section 4 "Warp-cooperative BPE").
// textbook order: while some adjacent pair has a rank, replace the leftmost
// occurrence of the lowest-rank pair by ID 256 + rank.
//
// bpe_kernel: one thread per 16-byte chunk of a 4 KiB tile takes the pieces
// that start in its chunk, in order:
//   - a 1-byte piece is its byte's ID;
//   - a 2..13-byte piece that is a whole vocabulary string whose own BPE is
//     that single token is emitted with one probe of the whole-piece table
//     (TokTier, "Exact GPU Tokenization": whole-piece vocabulary hits; only
//     strings checked at load to encode to themselves are in the table);
//   - any other piece of at most 32 bytes is merged in the thread's registers:
//     symbols and the ranks of adjacent pairs live in fully unrolled arrays,
//     each step takes the minimum rank (leftmost on ties), merges, and probes
//     only the two pairs next to the merge (TokTier: only pairs adjacent to a
//     completed merge are re-probed);
//   - a longer piece is the chunk's last piece; it goes to a device list for
//     bpe_long_kernel.
// The chunk's tokens are written contiguously from its first piece start.
//
// bpe_long_kernel: one wave per long piece, any length, in rounds: a round
// finds the minimum rank r, takes every leftmost non-overlapping occurrence of
// that (unique) pair value at once, compacts the symbol array and re-probes
// the pairs next to each merge (TokTier: merging all leftmost non-overlapping
// occurrences of the minimum-rank pair equals iterated single merges; GraphTok,
// section 4: round merges for long pieces of repeated characters).
#include "tok_internal.h"
#include "bpe_util.h"

namespace tok {
namespace {

__device__ inline uint32_t merge_rank(const Tables& T, uint32_t a, uint32_t b) {
  if ((a | b) < 256u) return T.pair_rank[(a << 8) | b];
  const uint64_t key = ((uint64_t)a << 20) | b;
  uint32_t h = merge_hash(a, b) & T.merge_mask;
  for (uint32_t probe = 0; probe <= T.merge_mask; ++probe) {
    const uint64_t s = T.merge_slots[h];
    if (s == kEmptySlot) return kNoRank;
    if ((s >> 24) == key) return (uint32_t)(s & 0xFFFFFFu);
    h = (h + 1) & T.merge_mask;
  }
  return kNoRank;
}

// Whole-piece probe: token ID of the piece bytes p[0..len), 2 <= len <= 13,
// or kNoRank.
__device__ inline uint32_t word_lookup(const Tables& T, const uint8_t* p, uint32_t len) {
  uint64_t a = 0, b = 0;
#pragma unroll
  for (uint32_t i = 0; i < 8; ++i)
    if (i < len) a |= (uint64_t)p[i] << (8 * i);
#pragma unroll
  for (uint32_t i = 8; i < (uint32_t)kWordMax; ++i)
    if (i < len) b |= (uint64_t)p[i] << (8 * (i - 8));
  b |= (uint64_t)len << 40;
  const ulonglong2* slots = reinterpret_cast<const ulonglong2*>(T.word_slots);
  uint32_t h = word_hash(a, b) & T.word_mask;
  for (uint32_t probe = 0; probe <= T.word_mask; ++probe) {
    const ulonglong2 s = slots[h];
    if (s.y == 0) return kNoRank;
    if (s.x == a && (s.y & ((1ull << 44) - 1)) == b) return (uint32_t)(s.y >> 44);
    h = (h + 1) & T.word_mask;
  }
  return kNoRank;
}

// Textbook BPE of p[0..n), 2 <= n <= CAP, in registers; writes the tokens to
// out and returns their count.
template <int CAP>
__device__ inline uint32_t bpe_regs(const Tables& T, const uint8_t* p, uint32_t n, int32_t* out) {
  uint32_t sym[CAP], rk[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) sym[i] = (uint32_t)i < n ? p[i] : 0u;
#pragma unroll
  for (int i = 0; i < CAP; ++i) rk[i] = (uint32_t)i + 1 < n ? T.pair_rank[(sym[i] << 8) | sym[i + 1 < CAP ? i + 1 : i]] : kNoRank;
  for (;;) {
    uint32_t best = rk[0], bi = 0;
#pragma unroll
    for (int i = 1; i < CAP - 1; ++i) {
      if (rk[i] < best) { best = rk[i]; bi = i; }
    }
    if (best == kNoRank) break;
    const uint32_t nid = 256u + best;
    uint32_t left = 0, right = 0;
#pragma unroll
    for (int i = 0; i < CAP; ++i) {
      if ((uint32_t)i + 1 == bi) left = sym[i];
      if ((uint32_t)i == bi + 2) right = sym[i];
    }
    const uint32_t rl = bi > 0 ? merge_rank(T, left, nid) : kNoRank;
    const uint32_t rr = bi + 2 < n ? merge_rank(T, nid, right) : kNoRank;
#pragma unroll
    for (int i = 0; i < CAP; ++i) {
      const uint32_t nxt_s = i + 1 < CAP ? sym[i + 1] : 0u;
      const uint32_t nxt_r = i + 1 < CAP ? rk[i + 1] : kNoRank;
      const uint32_t ui = (uint32_t)i;
      sym[i] = ui < bi ? sym[i] : (ui == bi ? nid : nxt_s);
      rk[i] = ui + 1 < bi ? rk[i] : (ui + 1 == bi ? rl : (ui == bi ? rr : nxt_r));
    }
    --n;
  }
#pragma unroll
  for (int i = 0; i < CAP; ++i)
    if ((uint32_t)i < n) out[i] = (int32_t)sym[i];
  return n;
}

__global__ void __launch_bounds__(kThreads)
bpe_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B) {
  constexpr int kTextLds = kTile + 2 * kShortMax + 16;
  constexpr int kFlagLds = kThreads + 4;
  __shared__ uint8_t s_text[kTextLds];
  __shared__ uint16_t s_flags[kFlagLds];

  const uint32_t tid = threadIdx.x;
  const uint64_t base = (uint64_t)blockIdx.x * kTile;
  const uint64_t c0 = (uint64_t)blockIdx.x * kThreads;
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  for (int k = tid; k < kTextLds; k += kThreads) {
    const uint64_t p = base + k;
    s_text[k] = p < n ? text[p] : 0;
  }
  for (int k = tid; k < kFlagLds; k += kThreads) {
    const uint64_t c = c0 + k;
    s_flags[k] = c < n_chunks ? B.flags[c] : 0;
  }
  __syncthreads();

  const uint64_t c = c0 + tid;
  if (c >= n_chunks) return;
  uint32_t w = s_flags[tid];
  if (!w) {
    B.chunk_cnt[c] = 0;
    return;
  }
  const uint64_t first = c * kChunk + __builtin_ctz(w);
  int32_t* out = B.staging + first;
  uint32_t cnt = 0;
  const bool words = T.word_slots != nullptr;
  while (w) {
    const uint32_t bit = __builtin_ctz(w);
    w &= w - 1;
    const uint64_t s = c * kChunk + bit;
    uint64_t e;
    if (w) {
      e = c * kChunk + __builtin_ctz(w);
    } else {
      const uint32_t w1 = s_flags[tid + 1], w2 = s_flags[tid + 2], w3 = s_flags[tid + 3];
      e = w1 ? (c + 1) * kChunk + __builtin_ctz(w1)
             : w2 ? (c + 2) * kChunk + __builtin_ctz(w2)
                  : w3 ? (c + 3) * kChunk + __builtin_ctz(w3) : ~0ull;
    }
    if (e > n) e = n;
    if (e - s > (uint64_t)kShortMax) {
      const uint32_t slot = atomicAdd(&B.ctr->n_long, 1u);
      B.longs[slot] = make_uint4((uint32_t)s, (uint32_t)c, (uint32_t)(first + cnt), 0u);
      break;
    }
    const uint32_t len = (uint32_t)(e - s);
    const uint8_t* p = s_text + (s - base);
    if (len == 1) {
      out[cnt++] = p[0];
      continue;
    }
    if (words && len <= (uint32_t)kWordMax) {
      const uint32_t id = word_lookup(T, p, len);
      if (id != kNoRank) {
        out[cnt++] = (int32_t)id;
        continue;
      }
    }
    cnt += bpe_regs<kShortMax>(T, p, len, out + cnt);
  }
  B.chunk_cnt[c] = cnt;
}

__device__ inline uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d, 64));
  return v;
}

// Byte offset of the first piece start after s, or n.
__device__ inline uint64_t next_start(const uint16_t* flags, uint64_t n, uint64_t s) {
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t c = s / kChunk;
  const uint32_t own = flags[c] & ~((2u << (s % kChunk)) - 1u);
  if (own) return c * kChunk + __builtin_ctz(own);
  for (uint64_t cb = c + 1; cb < n_chunks; cb += 64) {
    const uint64_t ci = cb + lane;
    const uint32_t wv = ci < n_chunks ? flags[ci] : 0u;
    const uint64_t mask = __ballot(wv != 0);
    if (mask) {
      const uint32_t l = __builtin_ctzll(mask);
      const uint32_t wl = __shfl(wv, l, 64);
      return (cb + l) * kChunk + __builtin_ctz(wl);
    }
  }
  return n;
}

__global__ void __launch_bounds__(kThreads)
bpe_long_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t n_waves = (gridDim.x * kThreads) >> 6;
  const uint32_t n_long = B.ctr->n_long;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (uint32_t item = wave; item < n_long; item += n_waves) {
    const uint4 L = B.longs[item];
    const uint64_t s = L.x, c = L.y, dest = L.z;
    const uint64_t e = next_start(B.flags, n, s);
    uint32_t* sym = B.ws_sym + s;
    uint32_t* rk = B.ws_rk + s;
    uint64_t* sel = B.ws_sel + s;
    uint32_t cur = (uint32_t)(e - s);
    for (uint32_t k = lane; k < cur; k += 64) {
      const uint32_t a = text[s + k];
      sym[k] = a;
      rk[k] = k + 1 < cur ? T.pair_rank[(a << 8) | text[s + k + 1]] : kNoRank;
    }
    for (;;) {
      uint32_t m = kNoRank;
      for (uint32_t k = lane; k + 1 < cur; k += 64) m = min(m, rk[k]);
      m = wave_min(m);
      if (m == kNoRank) break;
      // choose the leftmost non-overlapping occurrences of the pair of rank m
      const uint32_t groups = (cur + 63) / 64;
      uint32_t carry = 0, chosen = 0;
      for (uint32_t g = 0; g < groups; ++g) {
        const uint32_t k = g * 64 + lane;
        const uint64_t mm = __ballot(k + 1 < cur && rk[k] == m);
        const uint64_t S = select_leftmost(mm, carry);
        carry = (uint32_t)(S >> 63);
        chosen += __popcll(S);
        if (lane == 0) sel[g] = S;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // merge, compact in place (new index <= old index), re-probe next to merges
      const uint32_t nid = 256u + m;
      uint32_t removed = 0;
      uint64_t prev_S = 0;
      for (uint32_t g = 0; g < groups; ++g) {
        const uint64_t S = sel[g];
        const uint64_t S_next = g + 1 < groups ? sel[g + 1] : 0ull;
        const uint64_t R = (S << 1) | (prev_S >> 63);  // bit j: position 64g + j is absorbed
        const uint32_t k = g * 64 + lane;
        const bool alive = k < cur && !((R >> lane) & 1ull);
        uint32_t nsym = 0, nrk = kNoRank;
        if (alive) {
          const bool chose = (S >> lane) & 1ull;
          nsym = chose ? nid : sym[k];
          const uint32_t kn = chose ? k + 2 : k + 1;  // next surviving position
          if (kn < cur) {
            const uint32_t jn = kn - g * 64;  // 1..65
            const bool chose_n = jn < 64 ? ((S >> jn) & 1ull) : ((S_next >> (jn - 64)) & 1ull);
            if (chose || chose_n) {
              const uint32_t sn = chose_n ? nid : sym[kn];
              nrk = merge_rank(T, nsym, sn);
            } else {
              nrk = rk[k];
            }
          }
        }
        const uint32_t idx = k - removed - (uint32_t)__popcll(R & lt_mask);
        __builtin_amdgcn_wave_barrier();
        if (alive) {
          sym[idx] = nsym;
          rk[idx] = nrk;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const uint32_t in_range = k < cur ? 1u : 0u;
        removed += (uint32_t)__popcll(__ballot(in_range && ((R >> lane) & 1ull)));
        prev_S = S;
      }
      cur -= chosen;
    }
    int32_t* out = B.staging + dest;
    for (uint32_t k = lane; k < cur; k += 64) out[k] = (int32_t)sym[k];
    if (lane == 0) B.chunk_cnt[c] += cur;
  }
}

}  // namespace

void launch_bpe(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((n + kTile - 1) / kTile);
  if (tiles) bpe_kernel<<<tiles, kThreads, 0, s>>>(text, n, t, b);
}

void launch_bpe_long(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s) {
  if (n) bpe_long_kernel<<<kLongWaves / (kThreads / 64), kThreads, 0, s>>>(text, n, t, b);
}

}  // namespace tok
