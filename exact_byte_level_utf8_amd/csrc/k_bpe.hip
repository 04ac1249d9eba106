// Merge stage: byte-level BPE of every piece by lowest merge rank.
//
// BPE never crosses a piece boundary, so pieces are independent; inside a
// piece the merges are ordered: while some adjacent pair has a rank, the
// lowest rank wins, the leftmost pair on equal rank, and the pair becomes ID
// 256 + rank (GraphTok, section 4 "Warp-cooperative BPE").
//
// piece_kernel (one thread per 4 bytes): resolves the pieces that need no
// merge loop -- a 1-byte piece is its byte's ID, and a 2..13-byte piece that is
// a whole vocabulary string whose own BPE is that token (checked for every
// string at load) is one probe of the whole-piece table (TokTier, "Exact GPU
// Tokenization": whole-piece vocabulary hits) -- and appends every other piece
// to one of three device work lists by length, with one atomic per wave.
//
// merge_kernel (persistent waves, items dealt round-robin): takes the long
// list first, then the 17..64-byte list (one wave per piece, one symbol per
// lane), then the 2..16-byte list (four pieces per wave, one 16-lane row each).
// A round takes the row minimum of (rank, position), chooses every leftmost
// non-overlapping occurrence of that pair value at once, compacts the row with
// a lane permute, and re-probes only the pairs next to a merge (TokTier:
// merging all leftmost non-overlapping occurrences of the minimum-rank pair
// equals iterated single merges, and only pairs adjacent to a completed merge
// are re-probed; GraphTok: a round takes every other pair of a chain).  Pieces
// longer than 64 bytes run the same rounds over arrays in global memory.
//
// Every piece's tokens go to staging[start ..] and their count to cnt8[start];
// each chunk's token total accumulates in chunk_cnt[start / 16].
#include "tok_internal.h"
#include "bpe_util.h"
#include "wg_scan.h"

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

// Whole-piece probe: token ID of the bytes p[0..len), 2 <= len <= 13, or kNoRank.
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

__global__ void __launch_bounds__(kThreads)
piece_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B) {
  constexpr int kChunksPerWg = kPieceTile / kChunk;  // 64
  constexpr int kTextLds = kPieceTile + kWaveMax + 16;
  constexpr int kFlagLds = kChunksPerWg + 6;
  __shared__ uint8_t s_text[kTextLds];
  __shared__ uint16_t s_flags[kFlagLds];

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint64_t base = (uint64_t)blockIdx.x * kPieceTile;
  const uint64_t c0 = (uint64_t)blockIdx.x * kChunksPerWg;
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

  const uint32_t lc = tid >> 2, q = tid & 3u;  // chunk within the workgroup, quarter of it
  const uint64_t c = c0 + lc;
  const uint32_t w = c < n_chunks ? s_flags[lc] : 0u;
  const uint32_t mine = (w >> (4 * q)) & 15u;
  uint32_t hits = 0, kinds = 0, lens = 0, packed = 0;
#pragma unroll
  for (uint32_t b = 0; b < 4; ++b) {
    if (!((mine >> b) & 1u)) continue;
    const uint32_t bit = 4 * q + b;
    const uint64_t s = c * kChunk + bit;
    uint64_t e = ~0ull;
    const uint32_t above = w & ~((2u << bit) - 1u);
    if (above) {
      e = c * kChunk + __builtin_ctz(above);
    } else {
      for (uint32_t j = 1; j <= 4; ++j) {
        const uint32_t wj = s_flags[lc + j];
        if (wj) {
          e = (c + j) * kChunk + __builtin_ctz(wj);
          break;
        }
      }
    }
    if (e > n) e = n;
    const uint64_t len = e - s;
    const uint8_t* p = s_text + (s - base);
    uint32_t id = kNoRank;
    if (len == 1) id = p[0];
    else if (len <= (uint64_t)kWordMax && T.word_slots) id = word_lookup(T, p, (uint32_t)len);
    if (id != kNoRank) {
      B.staging[s] = (int32_t)id;
      B.cnt8[s] = 1;
      ++hits;
      continue;
    }
    const uint32_t list = len <= (uint64_t)kRowMax ? 0u : len <= (uint64_t)kWaveMax ? 1u : 2u;
    kinds |= (list + 1) << (2 * b);
    lens |= (list == 2 ? 0u : (uint32_t)len) << (8 * b);
    packed += 1u << (10 * list);
  }
  // list slots: one atomic per wave and list, lanes take consecutive slots
  const uint32_t incl = wave_incl_scan(packed, AddOp());
  const uint32_t excl = incl - packed;
  const uint32_t tot = __shfl(incl, 63, 64);
  uint32_t b0 = 0, b1 = 0, b2 = 0;
  if (lane == 63) {
    if (tot & 1023u) b0 = atomicAdd(&B.ctr->n_list[0], tot & 1023u);
    if ((tot >> 10) & 1023u) b1 = atomicAdd(&B.ctr->n_list[1], (tot >> 10) & 1023u);
    if ((tot >> 20) & 1023u) b2 = atomicAdd(&B.ctr->n_list[2], (tot >> 20) & 1023u);
  }
  uint32_t slot0 = __shfl(b0, 63, 64) + (excl & 1023u);
  uint32_t slot1 = __shfl(b1, 63, 64) + ((excl >> 10) & 1023u);
  uint32_t slot2 = __shfl(b2, 63, 64) + ((excl >> 20) & 1023u);
#pragma unroll
  for (uint32_t b = 0; b < 4; ++b) {
    const uint32_t kind = (kinds >> (2 * b)) & 3u;
    if (!kind) continue;
    const uint2 item = make_uint2((uint32_t)(c * kChunk + 4 * q + b), (lens >> (8 * b)) & 255u);
    if (kind == 1) B.list[0][slot0++] = item;
    else if (kind == 2) B.list[1][slot1++] = item;
    else B.list[2][slot2++] = item;
  }
  hits += __shfl_xor(hits, 1, 64);
  hits += __shfl_xor(hits, 2, 64);
  if (q == 0 && c < n_chunks) B.chunk_cnt[c] = hits;
}

// BPE of one piece per row of ROW lanes (ROW = 16: four pieces per wave; ROW =
// 64: one piece per wave), one symbol per lane, in rounds.  Called by all 64
// lanes; rows without a piece pass active = false.
template <int ROW>
__device__ void merge_rows(const Tables& T, const uint8_t* __restrict__ text, uint64_t s, uint32_t len,
                           bool active, const Bufs& B) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t k = lane & (ROW - 1);
  const uint32_t row_base = lane - k;
  const uint64_t row_bits = ROW == 64 ? ~0ull : (0xFFFFull << row_base);
  const uint64_t below = ((1ull << lane) - 1ull) & row_bits;
  uint32_t cur = active ? len : 0u;
  uint32_t sym = k < cur ? (uint32_t)text[s + k] : 0u;
  const uint32_t nx = __shfl_down(sym, 1, ROW);
  uint32_t rk = k + 1 < cur ? T.pair_rank[(sym << 8) | nx] : kNoRank;
  for (;;) {
    if (k + 1 >= cur) rk = kNoRank;
    uint32_t key = rk == kNoRank ? 0xFFFFFFFFu : ((rk << 6) | k);
#pragma unroll
    for (int d = ROW / 2; d >= 1; d >>= 1) key = min(key, (uint32_t)__shfl_xor(key, d, ROW));
    const bool live = key != 0xFFFFFFFFu;
    if (__ballot(live) == 0) break;
    const uint32_t r = key >> 6;
    const uint64_t S = select_leftmost(__ballot(live && rk == r), 0);
    const bool chose = (S >> lane) & 1ull;
    const bool gone = k > 0 && ((S >> (lane - 1)) & 1ull);
    const uint32_t nsym = chose ? 256u + r : sym;
    const uint32_t n1 = __shfl_down(nsym, 1, ROW);
    const uint32_t n2 = __shfl_down(nsym, 2, ROW);
    uint32_t nrk = rk;
    if (live && !gone && k < cur) {
      const uint32_t kn = chose ? k + 2 : k + 1;  // next surviving position
      nrk = kNoRank;
      if (kn < cur) {
        const bool chose_n = (S >> (row_base + kn)) & 1ull;
        nrk = (chose || chose_n) ? merge_rank(T, nsym, chose ? n2 : n1) : rk;
      }
    }
    const uint32_t nk = k - (uint32_t)__popcll((S << 1) & below);
    const uint32_t dst = !live ? lane : ((gone || k >= cur) ? row_base + ROW - 1 : row_base + nk);
    sym = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nsym);
    rk = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nrk);
    if (live) cur -= (uint32_t)__popcll(S & row_bits);
  }
  if (active && k < cur) B.staging[s + k] = (int32_t)sym;
  if (active && k == 0) {
    B.cnt8[s] = (uint8_t)cur;
    atomicAdd(&B.chunk_cnt[s / kChunk], cur);
  }
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
      const uint32_t wl = __builtin_amdgcn_readfirstlane(__shfl(wv, l, 64));
      return (cb + l) * kChunk + __builtin_ctz(wl);
    }
  }
  return n;
}

// One wave merges a piece longer than 64 bytes with the same rounds, its
// symbols and pair ranks in global memory (workspace indexed by the piece's
// bytes, so pieces never share it), compacting in place.
__device__ void merge_long(const Tables& T, const uint8_t* __restrict__ text, uint64_t n, uint64_t s,
                           const Bufs& B) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const uint64_t e = next_start(B.flags, n, s);
  uint32_t* sym = B.ws_sym + s;
  uint32_t* rk = B.ws_rk + s;
  uint64_t* sel = B.ws_sel + s;
  uint32_t cur = __builtin_amdgcn_readfirstlane((uint32_t)(e - s));
  for (uint32_t k = lane; k < cur; k += 64) {
    const uint32_t a = text[s + k];
    sym[k] = a;
    rk[k] = k + 1 < cur ? T.pair_rank[(a << 8) | text[s + k + 1]] : kNoRank;
  }
  for (;;) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    uint32_t m = kNoRank;
    for (uint32_t k = lane; k + 1 < cur; k += 64) m = min(m, rk[k]);
    m = __builtin_amdgcn_readfirstlane(wave_min(m));
    if (m == kNoRank) break;
    const uint32_t groups = (cur + 63) / 64;
    uint32_t carry = 0, chosen = 0;
    for (uint32_t g = 0; g < groups; ++g) {
      const uint32_t k = g * 64 + lane;
      const uint64_t S = select_leftmost(__ballot(k + 1 < cur && rk[k] == m), carry);
      carry = (uint32_t)(S >> 63);
      chosen += (uint32_t)__popcll(S);
      if (lane == 0) sel[g] = S;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
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
        const uint32_t kn = chose ? k + 2 : k + 1;
        if (kn < cur) {
          const uint32_t jn = kn - g * 64;  // 1..65
          const bool chose_n = jn < 64 ? ((S >> jn) & 1ull) : ((S_next >> (jn - 64)) & 1ull);
          if (chose || chose_n) nrk = merge_rank(T, nsym, chose_n ? nid : sym[kn]);
          else nrk = rk[k];
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
      removed += (uint32_t)__popcll(__ballot(k < cur && ((R >> lane) & 1ull)));
      prev_S = S;
    }
    cur -= chosen;
  }
  for (uint32_t k = lane; k < cur; k += 64) B.staging[s + k] = (int32_t)sym[k];
  if (lane == 0) {
    B.cnt8[s] = (uint8_t)(cur < 255 ? cur : 255);  // only the chunk's last piece can be long
    atomicAdd(&B.chunk_cnt[s / kChunk], cur);
  }
}

__global__ void __launch_bounds__(kThreads)
merge_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t n1 = B.ctr->n_list[0], n2 = B.ctr->n_list[1], n3 = B.ctr->n_list[2];
  const uint32_t total = n3 + n2 + (n1 + 3) / 4;
  // Items are dealt to waves round-robin, with every value that steers the
  // loop in scalar registers: a work item taken by one lane and broadcast by a
  // shuffle counts as divergent to the compiler, which then splits the loop
  // per lane and separates the lanes of a wave.
  const uint32_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * kThreads + threadIdx.x) >> 6);
  const uint32_t n_waves = (gridDim.x * kThreads) >> 6;
  for (uint32_t item = wave; item < total; item += n_waves) {
    if (item < n3) {
      merge_long(T, text, n, B.list[2][item].x, B);
    } else if (item < n3 + n2) {
      const uint2 it = B.list[1][item - n3];
      merge_rows<64>(T, text, it.x, it.y, true, B);
    } else {
      const uint32_t i = (item - n3 - n2) * 4 + (lane >> 4);
      const bool act = i < n1;
      const uint2 it = act ? B.list[0][i] : make_uint2(0u, 0u);
      merge_rows<16>(T, text, it.x, it.y, act, B);
    }
  }
}

}  // namespace

void launch_pieces(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s) {
  const uint32_t blocks = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
  if (blocks) piece_kernel<<<blocks, kThreads, 0, s>>>(text, n, t, b);
}

void launch_merge(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s) {
  if (!n) return;
  uint64_t blocks = (n + 1023) / 1024;
  if (blocks < 16) blocks = 16;
  if (blocks > 2048) blocks = 2048;
  merge_kernel<<<(uint32_t)blocks, kThreads, 0, s>>>(text, n, t, b);
}

}  // namespace tok
