// Internal declarations shared by the HIP sources of the tokenizer library.
//
// Data layout in HBM for one call over N input bytes (C = ceil(N / 16) chunks,
// G = ceil(N / 1024) tiles):
//   flags      uint16[C + 8]   bit i of word c: byte 16c + i starts a piece
//   staging    int32[N + 64]   each tile's IDs in order, from the tile's first
//                              piece start (a piece of b bytes yields at most b
//                              tokens, so the tiles' runs never overlap)
//   tile_cnt   uint32[G]       IDs of the pieces that start in tile t
//   tile_first uint32[G]       byte offset of tile t's first piece start
//   sum1       uint32[G / 64]  tile counts summed over aligned groups of 64 tiles
//   sum2       uint32[G / 4096] the same over groups of 4096 tiles
//   ws_sym     uint32[N + 64]  tokens of the pieces longer than 64 bytes,
//                              indexed by the piece's bytes; with ws_rk
//                              uint32[N + 64] and ws_sel uint64[N + 64] (per
//                              token: lowest operand ranks) the merge
//                              workspace of pieces too long for the LDS pool
// and, in pinned host memory mapped into the device, one Counters block that
// the host reads after its one synchronization of the call.
// Everything else a tile needs (its bytes, piece lists, tokens, counts) lives
// in LDS for the lifetime of its workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tok {

constexpr int kPretokSmallGrid = 1024;  // largest pre-tokenization grid run with 8-wave workgroups
constexpr int kChunk = 16;           // bytes per flag word
constexpr int kHalo = 64;            // context bytes loaded on each side of a tile
constexpr int kWordMax = 13;         // longest piece the short whole-piece table holds
constexpr int kLongMax = 28;         // longest piece the long whole-piece table holds
constexpr int kRowMax = 16;          // longest piece merged by one 16-lane row
constexpr int kHalfMax = 32;         // longest piece merged by one 32-lane row
constexpr int kWaveMax = 64;         // longest piece merged by one wave in registers
constexpr int kPretokTile = 1024;    // bytes per workgroup of the pre-tokenization pass
constexpr int kHandCountWord = 16;   // Bufs::hand_tick: the count's word, 128 bytes after the call number
constexpr int kHandTickWords = 32;
constexpr int kPieceTile = 1024;     // bytes per workgroup of the piece pass
constexpr uint32_t kPieceSmallGrid = 1024;  // piece-pass grids up to this use 512-thread workgroups
constexpr uint32_t kNoRank = 0xFFFFFFFFu;

// Units of BPE.  A merge joins two tokens, so a token that spans a byte
// boundary has the boundary's two bytes inside it.  Where no token can span
// the boundary, every token sequence BPE passes through has a boundary
// there, the pair straddling it never has a rank, and the rounds on each
// side are those of each side alone: BPE of the piece is the BPE of the bytes
// before the boundary followed by that of the bytes from it.  So a piece
// splits there into units of BPE that merge independently.
//
// The unit table (kUnitTabWords words, built at load) decides it from the
// four bytes around the boundary before byte i: bits [0, 65536) are set for
// every byte pair (a, b) some token holds; bits [65536, 131072) for every
// two-byte token; then kTriBits bits hold, hashed, every three-byte string
// inside some token.  A token spanning the boundary is the two bytes i - 1,
// i alone, or it holds the bytes i - 2 .. i or i - 1 .. i + 1; with none of
// these in the vocabulary nothing spans it.  A hash collision only keeps a
// boundary that could have been cut, so the cuts stay exact.
constexpr int kJoinWords = 65536 / 32;
constexpr int kTriLog = 20;
constexpr uint32_t kTriBits = 1u << kTriLog;
constexpr int kUnitTabWords = 2 * kJoinWords + (int)(kTriBits / 32);

// Bit of the three bytes x, y, z (key x | y << 8 | z << 16) in the table.
__host__ __device__ inline uint32_t tri_slot(uint32_t key) { return (key * 0x9E3779B1u) >> (32 - kTriLog); }

// w: bytes i - 2, i - 1, i, i + 1 (low to high; bytes past either end of
// the text are 0, which can only keep a boundary).
__device__ inline bool no_token_spans(const uint32_t* __restrict__ tab, uint32_t w) {
  const uint32_t pair = ((w >> 8) & 0xFFu) << 8 | ((w >> 16) & 0xFFu);
  const uint32_t h1 = tri_slot(w & 0xFFFFFFu), h2 = tri_slot(w >> 8);
  const uint32_t* tri = tab + 2 * kJoinWords;
  const uint32_t held = tab[pair >> 5], two = tab[kJoinWords + (pair >> 5)];  // all four reads at once
  const uint32_t t1 = tri[h1 >> 5], t2 = tri[h2 >> 5];
  if (!((held >> (pair & 31u)) & 1u)) return true;
  if ((two >> (pair & 31u)) & 1u) return false;
  return !((t1 >> (h1 & 31u)) & 1u) && !((t2 >> (h2 & 31u)) & 1u);
}
constexpr uint64_t kEmptySlot = ~0ull;
constexpr uint32_t kBucket = 4;      // hash-table slots probed with one set of loads

// classes
enum : uint32_t { kL = 0, kN = 1, kW = 2, kO = 3 };

// Result of the device repair's match and splice.
enum : uint32_t {
  kRepairSpliced = 1,
  kRepairNone = 2,
  kRepairSession = 3,
  kRepairCapacity = 4,
  kRepairEncodeError = 5,  // the window encode reported an error: nothing matched or written
};
struct RepairOut {
  uint64_t gen;     // call number of the last match that finished
  uint32_t status;  // kRepair*
  uint32_t pad;
  uint64_t total;   // IDs of the repaired session (spliced or capacity)
  uint64_t kept;    // stored IDs kept
  uint64_t splice;  // byte where the window's IDs take over
};

// Results of a call, written by the kernels into host memory.  Each call has
// a number (gen, never 0); an error is reported by storing that number, so no
// word needs clearing between calls and any number of workgroups may report.
struct Counters {
  uint64_t err_utf8;  // gen of the last call that found malformed UTF-8
  uint64_t err_docs;  // gen of the last call whose document offsets were invalid
  uint64_t done;      // gen of the last call whose assembly finished
  uint32_t total;     // tokens in the output of that call
  uint32_t lits;      // added-token literals taken by the last literal pass
  uint64_t lit_done;  // gen of the last call whose literal selection finished
  uint64_t ins_done;  // gen of the last call whose literal insertion finished
  RepairOut rp;       // the last device repair match
};

// Store a call number into the host-visible counters.
__device__ inline void report(uint64_t* word, uint64_t gen) {
  __hip_atomic_store(word, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

constexpr uint32_t kSum1Shift = 6;   // tiles per sum1 group: 64
constexpr uint32_t kSum2Shift = 12;  // tiles per sum2 group: 4096

// Read-only device tables built by tok_load.
struct Tables {
  const uint64_t* merge_slots;  // (left << 44 | right << 24 | rank), kEmptySlot = empty
  uint32_t merge_buckets;       // buckets, kBucket slots each (at most half the slots hold a merge)
  const uint32_t* pair_rank;    // [256 * 256] rank of byte pair (a, b), or kNoRank
  const uint64_t* word_slots;   // 2 x uint64 per slot, see word_hash()
  uint32_t word_buckets;        // buckets - 1; word_slots == nullptr disables the table
  const uint64_t* long_slots;   // 4 x uint64 per slot, see long_hash()
  uint32_t long_buckets;        // buckets - 1; long_slots == nullptr disables the table
  const uint32_t* tok_len;      // bytes of each token ID
  const uint32_t* tok_min;      // per token: lowest rank of a merge taking it as right operand (x), as left (y),
                                // 16 bits each (x high), shifted right by min_shift; 0xFFFF: none
  uint32_t min_shift;
  uint32_t max_tok_len;         // bytes of the longest token
};

// Per-call device buffers.
// Added-token literals folded into the piece pass (k_added.hip): the taken
// literals, marked by the pre-tokenization kernels on their way in (one
// literal per thread over the grid, before anything else) and read by the
// piece pass.  mark == nullptr: no literals to fold.
struct LitMarks {
  const uint64_t* sel;    // the taken literals in order, (first byte << 32 | literal index)
  const uint32_t* count;  // how many (on the device)
  const uint32_t* off;    // literal i's bytes are off[i] .. off[i + 1]
  const int32_t* ids;     // literal i's ID
  uint8_t* mark;          // 1 at a taken literal's first byte, 2 on its others (0 elsewhere: cleared before)
  int32_t* id_at;         // the literal's ID at its first byte
};

__device__ inline void mark_literals(const LitMarks& m) {
  if (!m.mark) return;
  const uint32_t k = *m.count;
  for (uint32_t j = blockIdx.x * blockDim.x + threadIdx.x; j < k; j += gridDim.x * blockDim.x) {
    const uint64_t a = m.sel[j];
    const uint32_t li = (uint32_t)a;
    const uint64_t S = a >> 32, E = S + (m.off[li + 1] - m.off[li]);
    m.id_at[S] = m.ids[li];
    m.mark[S] = 1;
    for (uint64_t b = S + 1; b < E; ++b) m.mark[b] = 2;
  }
}

struct Bufs {
  uint16_t* flags;
  int32_t* staging;
  uint32_t* tile_cnt;
  uint32_t* tile_first;
  uint32_t* sum1;
  uint32_t* sum2;
  uint32_t* ws_sym;
  uint32_t* ws_rk;
  uint64_t* ws_sel;
  Counters* ctr;  // device address of the host-mapped counters
  uint64_t gen;   // this call's number
  // Hand-over of the case-splitting pre-tokenization (k_pretok_case.hip):
  // hand_tick: kHandTickWords words; [0] the calls so far, and
  // [kHandCountWord] (on its own cache line) the workgroups of the current
  // call that have read that number; zero when allocated, and the count is
  // back to zero after every call, so they persist across calls and are not
  // per-call scratch.  hand_state: per tile, (tag << 32 | cursor), the first
  // piece start at or after the tile's end, tagged with the call's number
  // (1 + calls so far, modulo 2^32 - 1); zeroed when allocated.  hand_wait:
  // wall-clock ticks a tile waits for its predecessor's word before finding
  // the cursor itself (0: it never waits).
  uint64_t* hand_tick;
  uint64_t* hand_state;
  uint64_t hand_wait;
  const uint32_t* n_docs_dev;  // if set, the document count, read on the device (overrides n_docs)
  LitMarks lit;  // added-token literals folded into the piece pass (lit.mark == nullptr: none)
};

// A token's lowest ranks as right operand (x) and as left operand (y), from
// the packed table, floored to a multiple of 2^shift.  A floor never exceeds
// the rank, so a test "lowest rank > r" that passes on it passes on the rank
// too.  "None" (0xFFFF) comes out as 0xFFFF << shift, which the table's shift
// keeps above every rank, so it needs no case of its own.
__device__ inline uint2 token_mins(const uint32_t* __restrict__ tok_min, uint32_t shift, uint32_t t) {
  const uint32_t v = tok_min[t];
  return make_uint2((v >> 16) << shift, (v & 0xFFFFu) << shift);
}

// Hash of the merge pair (left, right): multiplicative hashing of the
// 40-bit key, high bits.
__host__ __device__ inline uint32_t merge_hash(uint32_t left, uint32_t right) {
  const uint64_t key = ((uint64_t)left << 20) | right;
  return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> 32);
}

// First bucket of the pair among nb buckets (the hash scaled to [0, nb), so
// nb need not be a power of two), and the bucket probed after h.
__host__ __device__ inline uint32_t merge_bucket(uint32_t left, uint32_t right, uint32_t nb) {
  return (uint32_t)(((uint64_t)merge_hash(left, right) * nb) >> 32);
}
__host__ __device__ inline uint32_t next_bucket(uint32_t h, uint32_t nb) { return h + 1 == nb ? 0u : h + 1; }

// Whole-piece key of a byte string of 2..13 bytes: a = bytes 0..7 (little
// endian, zero padded), b = bytes 8..12 | len << 40.  A stored slot adds the
// token ID in bits 44..63 of b.
__host__ __device__ inline uint32_t word_hash(uint64_t a, uint64_t b) {
  return (uint32_t)(((a ^ (b * 0x9E3779B97F4A7C15ull)) * 0xC2B2AE3D27D4EB4Full) >> 32);
}

// Whole-piece key of a byte string of 14..28 bytes: k0, k1, k2 = bytes 0..23
// (little endian), k3 = bytes 24..27 (zero padded) | len << 32.  A stored
// slot adds the token ID in bits 37..63 of k3.
__host__ __device__ inline uint32_t long_hash(uint64_t k0, uint64_t k1, uint64_t k2, uint64_t k3) {
  const uint64_t h = (k0 ^ (k1 * 0x9E3779B97F4A7C15ull)) * 0xC2B2AE3D27D4EB4Full ^ (k2 + (k3 << 7));
  return (uint32_t)((h * 0xFF51AFD7ED558CCDull) >> 32);
}

// First index d in [0, n_docs] with doc_off[d] >= x (n_docs + 1 if none).
__device__ inline uint32_t first_doc_at_or_after(const uint64_t* doc_off, uint32_t n_docs, uint64_t x) {
  uint32_t lo = 0, hi = n_docs + 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (doc_off[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Launch kernel k on stream s, between event records e0 and e1 when the
// stage is timed.
template <typename... KArgs, typename... Args>
inline void launch_on(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                      Args... args) {
  if (e0) (void)hipEventRecord(e0, s);
  k<<<grid, block, 0, s>>>(args...);
  if (e1) (void)hipEventRecord(e1, s);
}

// Kernel launchers (defined in the .hip files); e0 / e1: optional events
// around the stage's kernel.
void launch_empty_batch(Bufs b, const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off, hipStream_t s);
// unit_tab: nullptr for piece starts only; else the unit table, and a flag
// also marks every byte before which no token can span the boundary (at
// non-ASCII byte pairs).
void launch_pretok(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                   int pattern, const uint32_t* unit_tab, Bufs b, hipStream_t s, hipEvent_t e0 = nullptr,
                   hipEvent_t e1 = nullptr);
// The case-splitting family's pre-tokenization (k_pretok_case.hip), called by
// launch_pretok for that pattern.
void launch_pretok_case(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                        const uint32_t* unit_tab, Bufs b, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
void launch_pieces(const uint8_t* text, uint64_t n, Tables t, Bufs b, const uint64_t* doc_off,
                   uint32_t n_docs, uint64_t* out_off, hipStream_t s, hipEvent_t e0 = nullptr,
                   hipEvent_t e1 = nullptr);
// spans: optional uint32 per output ID, the byte where its token starts
// (tok_len is read only when spans is set).
void launch_assemble(uint64_t n, Bufs b, int32_t* out, uint32_t* spans, const uint32_t* tok_len, uint64_t cap,
                     const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off, hipStream_t s,
                     hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

}  // namespace tok
