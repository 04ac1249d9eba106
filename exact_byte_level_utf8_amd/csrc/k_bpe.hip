// Merge stage: byte-level BPE of every piece by lowest merge rank.
//
// BPE never crosses a piece boundary, so pieces are independent; inside a
// piece the merges are ordered: while some adjacent pair has a rank, the
// lowest rank wins, the leftmost pair on equal rank, and the pair becomes ID
// 256 + rank (GraphTok, section 4 "Warp-cooperative BPE").  The flag words
// this stage reads also cut pieces where no token can span a byte boundary
// (no_token_spans): the parts are independent units of BPE, and below
// "piece" means such a unit.
//
// piece_kernel: one workgroup per 1 KiB of piece starts, in three phases.
//   1. One thread per 2 bytes resolves the pieces that need no merge loop: a
//      1-byte piece is its byte's ID, and a 2..28-byte piece that is a whole
//      vocabulary string whose own BPE is that token (checked for every string
//      at load) is one probe of a whole-piece table (TokTier, section 4 "GPU
//      BPE": whole-piece vocabulary hits).  The probes are first compacted
//      into lists in LDS, one per table, and then run one per lane, so a wave
//      waits for one memory round trip.  Every other piece goes to a work
//      list in LDS by length.  With added-token literals folded in, a taken
//      literal is one piece (the flags inside it are masked) whose token is
//      the literal's ID.
//   2. The workgroup's waves merge the listed pieces of up to 64 bytes:
//      33..64-byte pieces first (one wave per piece, one symbol per lane),
//      then 17..32-byte pieces (two per wave, one 32-lane row each), then
//      2..16-byte pieces (four per wave, one 16-lane row each).
//      A round takes the row minimum of (rank, position), chooses every
//      leftmost non-overlapping occurrence of that pair value at once,
//      compacts the row with a lane permute, and re-probes only the pairs next
//      to a merge (TokTier: merging all leftmost non-overlapping occurrences of
//      the minimum-rank pair equals iterated single merges, and only pairs
//      adjacent to a completed merge are re-probed; GraphTok: a round takes
//      every other pair of a chain).
//   2b. Then the whole workgroup merges each piece longer than 64 bytes in
//      turn (long_merge.h): its symbols in an LDS pool that overlays the
//      length-class and probe lists (dead by then), or in the byte-indexed
//      workspace in global memory for pieces larger than the pool.  Its
//      tokens end in that workspace.
//   3. The tile's tokens are compacted in order (in LDS) and written as one
//      run from the tile's first piece start, with the tile's count, which is
//      also added to the sums of its groups of 64 and 4096 tiles; the
//      documents that start in the tile get their offsets within that run.
//      The assembly kernel then places the runs (k_assemble.hip).
#include "tok_internal.h"
#include "bpe_util.h"
#include "long_merge.h"
#include "merge_table.h"
#include "wg_scan.h"

#pragma clang diagnostic ignored "-Wbitwise-instead-of-logical"

namespace tok {
namespace {

// NW dwords holding the LDS bytes text[off .. off + 4 NW), read with NW + 1
// aligned dword loads and byte funnel shifts; bytes at or past len are zero.
template <int NW>
__device__ inline void key_words(const uint8_t* text, uint32_t off, uint32_t len, uint32_t (&w)[NW]) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(text) + (off >> 2);
  const uint32_t sh = off & 3u;
  uint32_t d[NW + 1];
#pragma unroll
  for (int i = 0; i <= NW; ++i) d[i] = a[i];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t v = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
    const int valid = (int)len - 4 * i;  // bytes of this word inside the piece
    w[i] = valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
  }
}

// Whole-piece probe of a 2..13-byte piece at text[off]: its token ID, or kNoRank.
__device__ inline uint32_t word_lookup(const Tables& T, const uint8_t* text, uint32_t off, uint32_t len) {
  uint32_t w[4];
  key_words<4>(text, off, len, w);
  const uint64_t a = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  const uint64_t b = ((uint64_t)w[2] | ((uint64_t)(w[3] & 0xFFu) << 32)) | ((uint64_t)len << 40);
  const ulonglong2* slots = reinterpret_cast<const ulonglong2*>(T.word_slots);
  uint32_t h = word_hash(a, b) & T.word_buckets;
  constexpr uint64_t kKeyMask = (1ull << 44) - 1;
  for (uint32_t probe = 0; probe <= T.word_buckets; ++probe) {
    const ulonglong2* bk = slots + (size_t)h * kBucket;
    const ulonglong2 s0 = bk[0], s1 = bk[1], s2 = bk[2], s3 = bk[3];
    if (s0.x == a && (s0.y & kKeyMask) == b) return (uint32_t)(s0.y >> 44);
    if (s1.x == a && (s1.y & kKeyMask) == b) return (uint32_t)(s1.y >> 44);
    if (s2.x == a && (s2.y & kKeyMask) == b) return (uint32_t)(s2.y >> 44);
    if (s3.x == a && (s3.y & kKeyMask) == b) return (uint32_t)(s3.y >> 44);
    if (s3.y == 0) return kNoRank;  // slots fill in order within a bucket
    h = (h + 1) & T.word_buckets;
  }
  return kNoRank;
}

// Whole-piece probe of a 14..28-byte piece at text[off]: its token ID, or
// kNoRank.  A bucket is four 32-byte slots, one 128-byte line.
__device__ inline uint32_t long_lookup(const Tables& T, const uint8_t* text, uint32_t off, uint32_t len) {
  uint32_t w[7];
  key_words<7>(text, off, len, w);
  const uint64_t k0 = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  const uint64_t k1 = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
  const uint64_t k2 = (uint64_t)w[4] | ((uint64_t)w[5] << 32);
  const uint64_t k3 = (uint64_t)w[6] | ((uint64_t)len << 32);
  const ulonglong2* slots = reinterpret_cast<const ulonglong2*>(T.long_slots);
  uint32_t h = long_hash(k0, k1, k2, k3) & T.long_buckets;
  constexpr uint64_t kKeyMask = (1ull << 37) - 1;
  for (uint32_t probe = 0; probe <= T.long_buckets; ++probe) {
    const ulonglong2* bk = slots + (size_t)h * kBucket * 2;
    uint64_t last = 0;
#pragma unroll
    for (uint32_t j = 0; j < kBucket; ++j) {
      const ulonglong2 lo = bk[2 * j], hi = bk[2 * j + 1];
      if (lo.x == k0 && lo.y == k1 && hi.x == k2 && (hi.y & kKeyMask) == k3) return (uint32_t)(hi.y >> 37);
      last = hi.y;
    }
    if (last == 0) return kNoRank;  // slots fill in order within a bucket
    h = (h + 1) & T.long_buckets;
  }
  return kNoRank;
}

// Row minimum over 16 lanes with DPP row rotations (every lane gets it).
__device__ inline uint32_t row16_min(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // row_ror:2
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

// Value of lane + 1 (next) and lane + 2 (next2) of the same row of ROW lanes,
// by DPP: row_shl inside a 16-lane row, wave_shl across the wave.  Lanes whose
// source lies past the row get 0 (callers never use those).
template <int ROW>
__device__ inline uint32_t row_next(uint32_t v) {
  if (ROW == 16) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xF, 0xF, false);  // row_shl:1
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xF, 0xF, false);                  // wave_shl:1
}
template <int ROW>
__device__ inline uint32_t row_next2(uint32_t v) {
  if (ROW == 16) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xF, 0xF, false);  // row_shl:2
  return row_next<64>(row_next<64>(v));
}

__device__ inline uint32_t wave_min(uint32_t v) {
  v = row16_min(v);
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Set bits of the wave mask x in this lane's row of ROW lanes (row_base: the
// row's first lane), all of them or only those below lane k of the row; the
// counts come from the lane number, so no per-lane 64-bit mask stays live.
template <int ROW>
__device__ inline uint32_t row_count(uint64_t x, uint32_t row_base) {
  if (ROW == 64) return (uint32_t)__popcll(x);
  return (uint32_t)__popc((uint32_t)(x >> row_base) & (ROW >= 32 ? 0xFFFFFFFFu : (1u << (ROW & 31)) - 1u));
}
template <int ROW>
__device__ inline uint32_t row_count_below(uint64_t x, uint32_t row_base, uint32_t k) {
  if (ROW == 64) return __builtin_amdgcn_mbcnt_hi((uint32_t)(x >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)x, 0u));
  return (uint32_t)__popc((uint32_t)(x >> row_base) & ((1u << k) - 1u));
}

// Value of lane k + D (row_up) or k - D (row_down) of the same row of ROW
// lanes, or kNoRank where that lane lies outside the row.
template <int ROW, int D>
__device__ inline uint32_t row_up(uint32_t v, uint32_t k) {
  if (ROW == 16) return (uint32_t)__builtin_amdgcn_update_dpp((int)kNoRank, (int)v, 0x100 + D, 0xF, 0xF, false);
  uint32_t x = v;
#pragma unroll
  for (int i = 0; i < D; ++i) x = (uint32_t)__builtin_amdgcn_update_dpp((int)kNoRank, (int)x, 0x130, 0xF, 0xF, false);
  return k + D < (uint32_t)ROW ? x : kNoRank;
}
template <int ROW, int D>
__device__ inline uint32_t row_down(uint32_t v, uint32_t k) {
  if (ROW == 16) return (uint32_t)__builtin_amdgcn_update_dpp((int)kNoRank, (int)v, 0x110 + D, 0xF, 0xF, false);
  uint32_t x = v;
#pragma unroll
  for (int i = 0; i < D; ++i) x = (uint32_t)__builtin_amdgcn_update_dpp((int)kNoRank, (int)x, 0x138, 0xF, 0xF, false);
  return k >= (uint32_t)D ? x : kNoRank;
}

// BPE of one piece per row of ROW lanes (ROW = 16: four pieces per wave; ROW =
// 32: two; ROW = 64: one), one symbol per lane, in rounds.  Called by all 64
// lanes; rows without a piece pass active = false.  p: the piece's bytes;
// tok_out / cnt_out: where its tokens and their count go; chunk_total: the
// counter of the chunk the piece starts in (all three in LDS).
//
// A round merges every pair of the row's lowest rank and every sheltered
// pair (x, y) of rank r: walking left from x over at most two pairs ranked
// above r reaches a token that no merge ranked below r takes as its right
// operand (x itself counts), or the piece start, and likewise to the right
// of y with left operands.  No merge ranked below r can then reach x or y, so
// textbook BPE merges (x, y) before anything changes them; adjacent merged
// pairs always share one rank, and runs of them keep the leftmost
// non-overlapping pairs.  Each lane carries its token's lowest ranks as right
// operand (ml) and as left operand (mr).
template <int ROW>
__device__ void merge_rows(const Tables& T, const uint8_t* p, uint32_t len, bool active, uint32_t* tok_out,
                           uint8_t* cnt_out, uint32_t* chunk_total) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t k = lane & (ROW - 1);
  const uint32_t row_base = lane - k;
  uint32_t cur = active ? len : 0u;
  uint32_t sym = k < cur ? (uint32_t)p[k] : 0u;
  const uint32_t nx = row_next<ROW>(sym);
  uint32_t rk = k + 1 < cur ? T.pair_rank[(sym << 8) | nx] : kNoRank;
  // held across the rounds (the empty asm keeps the compiler from reloading
  // it from the kernel arguments in every round)
  const uint32_t* __restrict__ tok_min = T.tok_min;
  __asm__ volatile("" : "+s"(tok_min));
  const uint32_t min_shift = T.min_shift;
  const uint2 m0 = token_mins(tok_min, min_shift, sym);
  uint32_t ml = m0.x, mr = m0.y;
  for (;;) {
    if (k + 1 >= cur) rk = kNoRank;
    if (k >= cur) ml = mr = kNoRank;
    uint32_t key = rk == kNoRank ? 0xFFFFFFFFu : ((rk << 6) | k);
    key = row16_min(key);
    if (ROW == 64) {
      const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)key, 0),
                             (uint32_t)__builtin_amdgcn_readlane((int)key, 16));
      const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)key, 32),
                             (uint32_t)__builtin_amdgcn_readlane((int)key, 48));
      key = min(a, b);
    } else if (ROW == 32) {
      const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)key, 0),
                             (uint32_t)__builtin_amdgcn_readlane((int)key, 16));
      const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)key, 32),
                             (uint32_t)__builtin_amdgcn_readlane((int)key, 48));
      key = lane < 32u ? a : b;
    }
    const bool live = key != 0xFFFFFFFFu;
    if (__ballot(live) == 0) break;
    const uint32_t low = key >> 6;
    // shelter of the pair (k, k + 1).  The neighbours' values are read with
    // every lane active (a DPP read from an inactive lane yields the
    // fallback, which would pass for "no rank") and combined without
    // branches.
    const uint32_t rl1 = row_down<ROW, 1>(rk, k), rl2 = row_down<ROW, 2>(rk, k);
    const uint32_t ml1 = row_down<ROW, 1>(ml, k), ml2 = row_down<ROW, 2>(ml, k);
    const uint32_t rr1 = row_up<ROW, 1>(rk, k), rr2 = row_up<ROW, 2>(rk, k);
    const uint32_t mr1 = row_up<ROW, 1>(mr, k), mr2 = row_up<ROW, 2>(mr, k), mr3 = row_up<ROW, 3>(mr, k);
    const bool left = (ml > rk) | ((rl1 > rk) & ((ml1 > rk) | ((rl2 > rk) & (ml2 > rk))));
    const bool right = (mr1 > rk) | ((rr1 > rk) & ((mr2 > rk) | ((rr2 > rk) & (mr3 > rk))));
    const bool take = (rk != kNoRank) & ((rk == low) | (left & right));
    const uint64_t S = select_leftmost(__ballot(take), 0);
    const bool chose = (S >> lane) & 1ull;
    const bool gone = k > 0 && ((S >> (lane - 1)) & 1ull);
    const uint32_t nsym = chose ? 256u + rk : sym;
    uint32_t nml = ml, nmr = mr;
    if (chose) {
      const uint2 m = token_mins(tok_min, min_shift, nsym);
      nml = m.x;
      nmr = m.y;
    }
    const uint32_t n1 = row_next<ROW>(nsym);
    const uint32_t n2 = row_next2<ROW>(nsym);
    // the pair starting at this symbol after the round: gone past the end,
    // new next to a merge (one probe), or unchanged
    const uint32_t kn = chose ? k + 2 : k + 1;  // next surviving position
    const bool here = live && !gone && k < cur;
    const bool chose_n = kn < cur && ((S >> ((row_base + kn) & 63u)) & 1ull);
    uint32_t nrk = here && kn >= cur ? kNoRank : rk;
    if (here && kn < cur && (chose || chose_n)) nrk = merge_rank(T, nsym, chose ? n2 : n1);
    const uint32_t nk = k - row_count_below<ROW>(S << 1, row_base, k);
    const uint32_t dst = !live ? lane : ((gone || k >= cur) ? row_base + ROW - 1 : row_base + nk);
    sym = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nsym);
    rk = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nrk);
    ml = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nml);
    mr = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)nmr);
    if (live) cur -= row_count<ROW>(S, row_base);
  }
  if (active && k < cur) tok_out[k] = sym;
  if (active && k == 0) {
    *cnt_out = (uint8_t)cur;
    atomicAdd(chunk_total, cur);
  }
}

// Byte offset of the first piece start after s, or n (one wave).
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

constexpr uint32_t kXcds = 8;    // XCDs of the device; workgroups are dealt to them in turn
constexpr uint32_t kXcdCus = 32;  // compute units per XCD
constexpr uint32_t kLine = 128;   // L2 line bytes

// Read one dword of every L2 line of this workgroup's share of a read-only
// table, so that the merge rounds find the table in this XCD's L2 (each XCD
// has its own L2, and every kernel starts with it cold).  The workgroups that
// run at once on one XCD split the table between them; a thread reads at most
// `most` lines.  Returns the xor of what it read, so that the loads are kept.
template <int NT>
__device__ inline uint32_t touch_lines(const void* table, uint64_t bytes, uint32_t most) {
  constexpr uint32_t kAtOnce = kXcdCus * (2048 / NT);  // resident workgroups per XCD at 8 waves per SIMD
  const uint32_t lines = (uint32_t)((bytes + kLine - 1) / kLine);
  const uint32_t on_xcd = min((gridDim.x + kXcds - 1) / kXcds, kAtOnce);
  const uint32_t share = (lines + on_xcd - 1) / on_xcd;
  const uint32_t lo = (blockIdx.x / kXcds % on_xcd) * share;
  const uint32_t hi = min(lo + share, lines);
  const uint8_t* t = static_cast<const uint8_t*>(table);
  uint32_t x = 0;
  for (uint32_t i = 0; i < most; ++i) {
    const uint32_t l = lo + i * NT + threadIdx.x;
    if (l < hi) x ^= *reinterpret_cast<const uint32_t*>(t + (size_t)l * kLine);
  }
  return x;
}

// LIT: added-token literals folded in (B.lit); a separate instantiation keeps
// their checks out of every other call.
template <int NT, bool LIT>
__global__ void __launch_bounds__(NT, 8)
piece_kernel(const uint8_t* __restrict__ text, uint64_t n, Tables T, Bufs B, const uint64_t* __restrict__ doc_off,
             uint32_t n_docs, uint64_t* __restrict__ out_off) {
  constexpr int kChunksPerWg = kPieceTile / kChunk;  // 64
  constexpr int kPerChunk = NT / kChunksPerWg;  // threads per chunk
  constexpr int kBytesPer = kChunk / kPerChunk;             // 2 bytes per thread
  constexpr int kTextLds = kPieceTile + kWaveMax + 16;
  static_assert(kTextLds % 4 == 0, "the tile bytes are loaded as dwords");
  constexpr int kFlagLds = kChunksPerWg + 6;
  constexpr int kTokLds = kPieceTile + kWaveMax;
  // pieces of 2..16 bytes in four length classes (13-16, 9-12, 5-8, 2-4),
  // merged longest class first; a class of minimum length L holds at most
  // 1024 / L pieces
  constexpr int kCapA = kPieceTile / 13 + 1, kCapB = kPieceTile / 9 + 1, kCapC = kPieceTile / 5 + 1;
  constexpr int kCapD = kPieceTile / 2;
  constexpr int kCapH = kPieceTile / (kRowMax + 1) + 1, kCap1 = kPieceTile / (kHalfMax + 1) + 1;
  constexpr int kCap2 = kPieceTile / (kWaveMax + 1) + 1;  // pieces over 64 bytes: at most 16 start in a tile
  constexpr int kCapPS = kPieceTile / 2, kCapPL = kPieceTile / (kWordMax + 1) + 1;
  // the length-class lists and the probe lists of 2..13-byte and 14..28-byte
  // pieces live in one pool; once phase 2 is done the pool holds the
  // symbols of one long piece at a time (16 bytes per symbol: as many as the
  // workgroup's LDS share allows at full occupancy)
  constexpr int kListWords = kCapA + kCapB + kCapC + kCapD + kCapH + kCap1 + kCapPS + kCapPL;
  constexpr int kLongE = NT == 512 ? 2 : 3;                // long-piece symbols per thread and chunk
  constexpr int kLongSyms = NT == 512 ? 2048 : NT * kLongE;  // long-piece symbols held in LDS (whole chunks)
  constexpr int kWaveSyms = kLongSyms / (NT / kWave);        // a wave's share of them (256 or 192)
  static_assert(kWaveSyms % (kWave * kLongE) == 0, "a wave's share is whole chunks");
  constexpr int kPoolWords = kListWords > 4 * kLongSyms ? kListWords : 4 * kLongSyms;
  __shared__ __attribute__((aligned(16))) uint8_t s_text[kTextLds];
  __shared__ uint16_t s_flags[kFlagLds];
  __shared__ uint16_t s_litst[kFlagLds];  // taken literals' first bytes (literal IDs folded in)
  __shared__ uint32_t s_tok[kTokLds];
  __shared__ uint8_t s_cnt8[kPieceTile];
  __shared__ __attribute__((aligned(16))) uint32_t s_pool[kPoolWords];
  uint32_t* const s_la = s_pool;
  uint32_t* const s_lb = s_la + kCapA;
  uint32_t* const s_lc = s_lb + kCapB;
  uint32_t* const s_ld = s_lc + kCapC;
  uint32_t* const s_lh = s_ld + kCapD;
  uint32_t* const s_list1 = s_lh + kCapH;
  uint32_t* const s_probe_s = s_list1 + kCap1;
  uint32_t* const s_probe_l = s_probe_s + kCapPS;
  __shared__ uint32_t s_list2[kCap2];
  __shared__ uint32_t s_cnt[kChunksPerWg], s_excl[kChunksPerWg];
  __shared__ uint32_t s_n[9], s_next, s_next2, s_nbig, s_first, s_doc0;
  __shared__ uint32_t s_big[kCap2], s_biglen[kCap2];  // long pieces set aside for the whole workgroup
  __shared__ uint32_t s_lscan[NT / kWave];
  __shared__ uint32_t s_lat[kCap2];  // phase 3: run position of each long piece

  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  if (tid < 9) s_n[tid] = 0;
  if (tid == 0) {
    s_next = 0;
    s_next2 = 0;
    s_nbig = 0;
  }
  const uint32_t tile = blockIdx.x;
  const uint64_t base = (uint64_t)tile * kPieceTile;
  const uint64_t c0 = (uint64_t)tile * kChunksPerWg;
  const uint64_t n_chunks = (n + kChunk - 1) / kChunk;
  // tile bytes as dwords (all loads in flight before the first wait); bytes
  // past the text are zero
  {
    constexpr int kTextWords = kTextLds / 4;
    const bool aligned = (reinterpret_cast<uintptr_t>(text) & 3u) == 0;
    uint32_t* s_text32 = reinterpret_cast<uint32_t*>(s_text);
#pragma unroll
    for (int r = 0; r < (kTextWords + NT - 1) / NT; ++r) {
      const int k = r * NT + (int)tid;
      if (k < kTextWords) {
        const uint64_t p = base + 4u * (uint32_t)k;
        uint32_t v = 0;
        if (aligned && p + 4 <= n) {
          v = *reinterpret_cast<const uint32_t*>(text + p);
        } else {
          for (uint32_t i = 0; i < 4; ++i)
            if (p + i < n) v |= (uint32_t)text[p + i] << (8 * i);
        }
        s_text32[k] = v;
      }
    }
  }
  for (int k = tid; k < kFlagLds; k += NT) {
    const uint64_t c = c0 + k;
    uint32_t f = c < n_chunks ? B.flags[c] : 0u, ls = 0;
    if (LIT && c < n_chunks) {  // a taken literal is one piece: no start inside it
      const uint4 mk = reinterpret_cast<const uint4*>(B.lit.mark)[c];  // the chunk's 16 marks
      const uint32_t w[4] = {mk.x, mk.y, mk.z, mk.w};
      uint32_t inside = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t v = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        ls |= (uint32_t)(v == 1u) << i;
        inside |= (uint32_t)(v == 2u) << i;
      }
      f &= ~inside;
    }
    s_flags[k] = (uint16_t)f;
    if (LIT) s_litst[k] = (uint16_t)ls;
  }
  // the merge and byte-pair tables into this XCD's L2 while phase 1 runs
  const uint32_t warm = touch_lines<NT>(T.merge_slots, (uint64_t)T.merge_buckets * kBucket * 8, 2) ^
                        touch_lines<NT>(T.pair_rank, 256u * 256u * 4u, 1);
  __syncthreads();

  // a piece that needs the merge loop goes to the list of its length class
  auto list_piece = [&](uint32_t item) {
    const uint32_t len = item >> 16;
    if (len > (uint32_t)kWaveMax) s_list2[atomicAdd(&s_n[5], 1u)] = item & 0xFFFFu;
    else if (len > (uint32_t)kHalfMax) s_list1[atomicAdd(&s_n[4], 1u)] = item;
    else if (len > (uint32_t)kRowMax) s_lh[atomicAdd(&s_n[8], 1u)] = item;
    else if (len >= 13u) s_la[atomicAdd(&s_n[0], 1u)] = item;
    else if (len >= 9u) s_lb[atomicAdd(&s_n[1], 1u)] = item;
    else if (len >= 5u) s_lc[atomicAdd(&s_n[2], 1u)] = item;
    else s_ld[atomicAdd(&s_n[3], 1u)] = item;
  };

  // phase 1a: a single byte is its own ID; a 2..28-byte piece goes to the
  // probe list of its whole-piece table, a longer one to the merge lists.
  // Thread (lc, q) owns bytes 2q, 2q + 1 of chunk lc.
  {
    const uint32_t lc = tid / kPerChunk, q = tid % kPerChunk;
    const uint32_t w = c0 + lc < n_chunks ? s_flags[lc] : 0u;
    const uint32_t mine = (w >> (kBytesPer * q)) & ((1u << kBytesPer) - 1u);
    // ends: the next piece start in this chunk, else in the next four chunks
    // (a piece with no start within 64 bytes is long, or runs to the end)
    const uint64_t c = c0 + lc;
    const uint32_t w1 = s_flags[lc + 1], w2 = s_flags[lc + 2], w3 = s_flags[lc + 3], w4 = s_flags[lc + 4];
    const uint32_t far = w1 ? 16u + __builtin_ctz(w1) : w2 ? 32u + __builtin_ctz(w2)
                       : w3 ? 48u + __builtin_ctz(w3) : w4 ? 64u + __builtin_ctz(w4) : 0xFFFFu;
    uint32_t hits = 0;
#pragma unroll
    for (uint32_t b = 0; b < (uint32_t)kBytesPer; ++b) {
      if (!((mine >> b) & 1u)) continue;
      const uint32_t bit = kBytesPer * q + b;
      const uint32_t above = w & ~((2u << bit) - 1u);
      const uint32_t endrel = above ? (uint32_t)__builtin_ctz(above) : far;
      const uint64_t s0 = c * kChunk + bit;
      const uint64_t e = min(endrel == 0xFFFFu ? ~0ull : c * kChunk + endrel, n);
      const uint32_t len = (uint32_t)min(e - s0, (uint64_t)0xFFFF);
      const uint32_t off = (uint32_t)(s0 - base);
      const uint32_t item = off | (len << 16);
      if (LIT && ((s_litst[lc] >> bit) & 1u)) {  // a taken literal: its ID
        s_tok[off] = (uint32_t)B.lit.id_at[s0];
        s_cnt8[off] = 1;
        ++hits;
      } else if (len == 1u) {
        s_tok[off] = s_text[off];
        s_cnt8[off] = 1;
        ++hits;
      } else if (T.word_slots && len <= (uint32_t)kWordMax) {
        s_probe_s[atomicAdd(&s_n[6], 1u)] = item;
      } else if (T.long_slots && len <= (uint32_t)kLongMax) {
        s_probe_l[atomicAdd(&s_n[7], 1u)] = item;
      } else {
        list_piece(item);
      }
    }
#pragma unroll
    for (int d = 1; d < kPerChunk; d <<= 1) hits += __shfl_xor(hits, d, 64);
    if (q == 0) s_cnt[lc] = hits;
  }
  __asm__ volatile("" : : "v"(warm));  // keeps the table reads; they arrive with the tile bytes
  __syncthreads();

  // phase 1b: one whole-piece probe per lane, all in flight at once.  The
  // long-table probes start at a wave boundary, so a wave probes one table.
  {
    const uint32_t ns = s_n[6], nl = s_n[7];
    const uint32_t l0 = (ns + kWave - 1) & ~(uint32_t)(kWave - 1);
    for (uint32_t t = tid; t < l0 + nl; t += NT) {
      const bool lng = t >= l0;
      if (!lng && t >= ns) continue;
      const uint32_t item = lng ? s_probe_l[t - l0] : s_probe_s[t];
      const uint32_t off = item & 0xFFFFu, len = item >> 16;
      const uint32_t id = lng ? long_lookup(T, s_text, off, len) : word_lookup(T, s_text, off, len);
      if (id != kNoRank) {
        s_tok[off] = id;
        s_cnt8[off] = 1;
        atomicAdd(&s_cnt[off / kChunk], 1u);
      } else {
        list_piece(item);
      }
    }
  }
  __syncthreads();

  // phase 2: the waves take items in order, longest pieces first: 33..64
  // bytes (a wave each), then pairs of 17..32-byte pieces (a 32-lane row
  // each), then groups of four 2..16-byte pieces by length class (a 16-lane
  // row each).  The item index comes from an LDS counter through
  // readfirstlane, so every branch on it is uniform across the wave.
  const uint32_t n2 = __builtin_amdgcn_readfirstlane(s_n[5]);
  {
    const uint32_t n1 = __builtin_amdgcn_readfirstlane(s_n[4]);
    const uint32_t nh = __builtin_amdgcn_readfirstlane(s_n[8]);
    const uint32_t ca = __builtin_amdgcn_readfirstlane(s_n[0]), cb = __builtin_amdgcn_readfirstlane(s_n[1]);
    const uint32_t cc = __builtin_amdgcn_readfirstlane(s_n[2]), cd = __builtin_amdgcn_readfirstlane(s_n[3]);
    const uint32_t eh = n1 + (nh + 1) / 2;
    const uint32_t ea = eh + (ca + 3) / 4, eb = ea + (cb + 3) / 4, ec = eb + (cc + 3) / 4;
    const uint32_t items = ec + (cd + 3) / 4;
    for (;;) {
      // every lane adds 1, so a grab moves the counter by 64
      const uint32_t item = __builtin_amdgcn_readfirstlane(atomicAdd(&s_next, 1u)) / (uint32_t)kWave;
      if (item >= items) break;
      if (item < n1) {
        const uint32_t it = s_list1[item];
        const uint32_t off = it & 0xFFFFu;
        merge_rows<64>(T, s_text + off, it >> 16, true, s_tok + off, &s_cnt8[off], &s_cnt[off / kChunk]);
      } else if (item < eh) {
        const uint32_t i = (item - n1) * 2 + (lane >> 5);
        const bool act = i < nh;
        const uint32_t it = act ? s_lh[i] : 0u;
        const uint32_t off = it & 0xFFFFu;
        merge_rows<32>(T, s_text + off, it >> 16, act, s_tok + off, &s_cnt8[off], &s_cnt[off / kChunk]);
      } else {
        // length class of the item: bounds and counts are wave-uniform
        const bool ia = item < ea, ib = !ia && item < eb, ic = !ia && !ib && item < ec;
        const uint32_t first = ia ? eh : ib ? ea : ic ? eb : ec;
        const uint32_t cnt = ia ? ca : ib ? cb : ic ? cc : cd;
        const uint32_t* lst = ia ? s_la : ib ? s_lb : ic ? s_lc : s_ld;
        const uint32_t i = (item - first) * 4 + (lane >> 4);
        const bool act = i < cnt;
        const uint32_t it = act ? lst[i] : 0u;
        const uint32_t off = it & 0xFFFFu;
        merge_rows<16>(T, s_text + off, it >> 16, act, s_tok + off, &s_cnt8[off], &s_cnt[off / kChunk]);
      }
    }
  }
  __syncthreads();

  // phase 2b: every piece over 64 bytes.  Its tokens end in ws_sym[start ..]
  // and its count in the chunk total (a long piece is its chunk's last), with
  // a count byte of 0 marking it for phase 3.  First the waves take the
  // pieces in turn, each merging one that fits its share of the LDS pool
  // (kWaveSyms symbols) with wave scans, all waves at once; a longer piece is
  // set aside, and those are then merged by the whole workgroup one after
  // another (uniform loop: the rounds hold barriers), in the pool when they
  // fit it, else in the workspace at the piece's bytes.
  if (n2) {  // uniform
    uint32_t* const s_wpool = s_pool + (tid / kWave) * (4u * kWaveSyms);  // this wave's share
    for (;;) {
      // every lane adds 1, so a grab moves the counter by 64
      const uint32_t k = __builtin_amdgcn_readfirstlane(atomicAdd(&s_next2, 1u)) / (uint32_t)kWave;
      if (k >= n2) break;
      const uint32_t off = s_list2[k];
      const uint64_t s = base + off;
      const uint32_t len = __builtin_amdgcn_readfirstlane((uint32_t)(next_start(B.flags, n, s) - s));
      if (len > (uint32_t)kWaveSyms) {
        if (lane == 0) {
          const uint32_t j = atomicAdd(&s_nbig, 1u);
          s_big[j] = k;
          s_biglen[j] = len;
        }
        continue;
      }
      // a round costs the wave the same whatever its active lanes: pieces of
      // up to 128 symbols take two per lane, longer ones kLongE
      uint32_t* const w_rk = s_wpool + kWaveSyms;
      uint2* const w_mm = reinterpret_cast<uint2*>(s_wpool + 2 * kWaveSyms);
      const uint32_t cnt =
          kLongE > 2 && len <= 2u * kWave
              ? longp::long_piece<longp::WaveGroup, 2>(text, s, len, T, s_wpool, w_rk, w_mm, B.ws_sym + s, nullptr)
              : longp::long_piece<longp::WaveGroup, kLongE>(text, s, len, T, s_wpool, w_rk, w_mm, B.ws_sym + s,
                                                            nullptr);
      if (lane == 0) {
        s_cnt8[off] = 0;
        atomicAdd(&s_cnt[off / kChunk], cnt);
      }
    }
    __syncthreads();  // the pool is free, and the set-aside list complete
    const uint32_t nbig = __builtin_amdgcn_readfirstlane(s_nbig);
    for (uint32_t j = 0; j < nbig; ++j) {
      const uint32_t off = s_list2[s_big[j]];
      const uint64_t s = base + off;
      const uint32_t len = __builtin_amdgcn_readfirstlane(s_biglen[j]);
      uint32_t cnt;
      if (len <= (uint32_t)kLongSyms)
        cnt = longp::long_piece<longp::WgGroup<NT>, kLongE>(text, s, len, T, s_pool, s_pool + kLongSyms,
                                                            reinterpret_cast<uint2*>(s_pool + 2 * kLongSyms),
                                                            B.ws_sym + s, s_lscan);
      else
        cnt = longp::long_piece<longp::WgGroup<NT>, kLongE>(text, s, len, T, B.ws_sym + s, B.ws_rk + s,
                                                            reinterpret_cast<uint2*>(B.ws_sel + s), B.ws_sym + s,
                                                            s_lscan);
      if (tid == 0) {
        s_cnt8[off] = 0;
        s_cnt[off / kChunk] += cnt;
      }
      __syncthreads();  // the pool is reused by the next piece
    }
  }

  // phase 3: the tile's tokens as one run from its first piece start (the
  // thread index again through an empty asm, so that no address computed
  // before the merge phase is kept, and spilled, across it)
  uint32_t t2 = threadIdx.x;
  __asm__ volatile("" : "+v"(t2));
  if (t2 < (uint32_t)kChunksPerWg) {  // wave 0, all lanes
    const uint32_t v = s_cnt[t2];
    const uint32_t incl = wave_incl_scan(v, AddOp(), 0u);
    s_excl[t2] = incl - v;
    const uint32_t total = __builtin_amdgcn_readlane((int)incl, 63);
    const uint64_t has = __ballot(c0 + t2 < n_chunks && s_flags[t2] != 0);
    uint64_t first = base;
    if (has) {
      const uint32_t l = (uint32_t)__builtin_ctzll(has);
      first = base + l * kChunk + __builtin_ctz((uint32_t)__builtin_amdgcn_readlane((int)s_flags[t2], (int)l));
    }
    if (t2 == 0) {
      s_first = (uint32_t)first;
      B.tile_cnt[tile] = total;
      B.tile_first[tile] = (uint32_t)first;
      atomicAdd(&B.sum1[tile >> kSum1Shift], total);
      atomicAdd(&B.sum2[tile >> kSum2Shift], total);
    }
  }
  if (doc_off && tid == kWave)
    s_doc0 = first_doc_at_or_after(doc_off, B.n_docs_dev ? *B.n_docs_dev : n_docs, base);
  __syncthreads();

  // every thread writes the tokens of the pieces that start in its two bytes:
  // its position in the run is its chunk's offset plus the counts of the
  // earlier pieces of the chunk (a scan over the chunk's eight threads).  A
  // piece longer than 64 bytes is its chunk's last piece; its count is what
  // the chunk's total leaves, and its tokens are in the long-piece workspace.
  {
    int32_t* run = B.staging + (uint32_t)__builtin_amdgcn_readfirstlane(s_first);  // unsigned: the builtin is signed
    // this thread's piece starts, read again from LDS rather than kept live
    // across the merge phase (the empty asm keeps the compiler from reusing,
    // and so spilling, addresses computed before it)
    uint32_t t3 = threadIdx.x;
    __asm__ volatile("" : "+v"(t3));
    const uint32_t lc = t3 / kPerChunk, q = t3 % kPerChunk;
    const uint32_t w = c0 + lc < n_chunks ? s_flags[lc] : 0u;
    const uint32_t mine = (w >> (kBytesPer * q)) & ((1u << kBytesPer) - 1u);
    uint32_t own = 0;
#pragma unroll
    for (uint32_t b = 0; b < (uint32_t)kBytesPer; ++b)
      if ((mine >> b) & 1u) own += s_cnt8[lc * kChunk + kBytesPer * q + b];
    uint32_t incl = own;
#pragma unroll
    for (int d = 1; d < kPerChunk; d <<= 1) {
      const uint32_t up = __shfl_up(incl, d, kPerChunk);
      if (q >= (uint32_t)d) incl += up;
    }
    uint32_t at = s_excl[lc] + (incl - own);
    const uint32_t chunk_end = s_excl[lc] + s_cnt[lc];
#pragma unroll
    for (uint32_t b = 0; b < (uint32_t)kBytesPer; ++b) {
      if (!((mine >> b) & 1u)) continue;
      const uint32_t off = lc * kChunk + kBytesPer * q + b;
      const uint32_t k = s_cnt8[off];
      if (k == 0) {  // long piece: its chunk's last; copied below by the whole workgroup
        uint32_t m = 0;
        while (s_list2[m] != off) ++m;
        s_lat[m] = at;
        at = chunk_end;
      } else {
        for (uint32_t j = 0; j < k; ++j) run[at + j] = (int32_t)s_tok[off + j];
        at += k;
      }
    }
  }

  if (n2) {  // uniform
    __syncthreads();
    int32_t* run = B.staging + (uint32_t)__builtin_amdgcn_readfirstlane(s_first);  // unsigned: the builtin is signed
    for (uint32_t m = 0; m < n2; ++m) {
      const uint32_t off = s_list2[m], at = s_lat[m];
      const uint32_t lc = off / kChunk, c = s_excl[lc] + s_cnt[lc] - at;  // the chunk's tokens from `at` on
      const uint32_t* src = B.ws_sym + base + off;
      for (uint32_t j = threadIdx.x; j < c; j += NT) run[at + j] = (int32_t)src[j];
    }
  }

  // offsets, within this tile's run, of the documents that start in the tile
  if (doc_off) {
    const uint32_t nd = B.n_docs_dev ? *B.n_docs_dev : n_docs;  // the count read on the device, if given
    for (uint32_t d = s_doc0 + tid; d <= nd; d += NT) {
      const uint64_t p = doc_off[d];
      if (p >= n || p >= base + kPieceTile) break;
      if (p < base) continue;  // only with unordered offsets, which the call rejects
      const uint32_t off = (uint32_t)(p - base), lc2 = off / kChunk;
      uint32_t before = s_flags[lc2] & ((1u << (off % kChunk)) - 1u);
      uint32_t loc = s_excl[lc2];
      while (before) {
        loc += s_cnt8[lc2 * kChunk + __builtin_ctz(before)];
        before &= before - 1;
      }
      out_off[d] = loc;
    }
  }
}

}  // namespace

void launch_pieces(const uint8_t* text, uint64_t n, Tables t, Bufs b, const uint64_t* doc_off,
                   uint32_t n_docs, uint64_t* out_off, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t blocks = (uint32_t)((n + kPieceTile - 1) / kPieceTile);
  if (!blocks) return;
  // up to one tile per workgroup slot of the device (four 512-thread
  // workgroups per CU) every tile starts at once with 8 waves; larger inputs
  // use 4-wave workgroups, so twice as many tiles are in flight per CU
  const bool lit = b.lit.mark != nullptr;
  if (blocks <= kPieceSmallGrid) {
    auto k = lit ? piece_kernel<512, true> : piece_kernel<512, false>;
    launch_on(k, dim3(blocks), dim3(512), s, e0, e1, text, n, t, b, doc_off, n_docs, out_off);
  } else {
    auto k = lit ? piece_kernel<256, true> : piece_kernel<256, false>;
    launch_on(k, dim3(blocks), dim3(256), s, e0, e1, text, n, t, b, doc_off, n_docs, out_off);
  }
}

}  // namespace tok
