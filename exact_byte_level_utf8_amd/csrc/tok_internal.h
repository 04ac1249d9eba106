// Internal declarations shared by the HIP sources of the tokenizer library.
//
// Data layout in HBM for one call over N input bytes (C = ceil(N / 16) chunks,
// G = ceil(N / 4096) tiles):
//   flags      uint16[C + 8]   bit i of word c: byte 16c + i starts a piece
//   staging    int32[N + 64]   tokens of the piece that starts at byte s, at
//                              staging[s ..] (a piece of b bytes yields at most
//                              b tokens, so every piece owns its slot)
//   cnt8       uint8[N + 64]   token count of the piece that starts at byte s
//                              (read only for pieces that are not the last of
//                              their chunk, which are under 16 bytes)
//   chunk_cnt  uint32[C]       tokens of the pieces that start in chunk c
//   chunk_excl uint32[C]       exclusive prefix of chunk_cnt (output offsets)
//   list1/2/3  uint2[...]      pieces left for merging: 2..16 bytes, 17..64
//                              bytes, longer (start, length; 0 = not yet known)
//   ws_sym/rk  uint32[N + 64]  merge workspace of long pieces, indexed by byte
//   ws_sel     uint64[N + 64]  round selections of long pieces, indexed by byte
//   scan_state uint64[G]       decoupled look-back state of the count scan
//   ctr        Counters        status and device-side counts
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tok {

constexpr int kTile = 4096;          // bytes per workgroup tile
constexpr int kThreads = 256;        // threads per workgroup
constexpr int kChunk = 16;           // bytes per thread (one flag word)
constexpr int kHalo = 64;            // context bytes loaded on each side of a tile
constexpr int kWordMax = 13;         // longest piece the whole-piece table holds
constexpr int kRowMax = 16;          // longest piece merged by one 16-lane row
constexpr int kWaveMax = 64;         // longest piece merged by one wave in registers
constexpr int kPieceTile = 1024;     // bytes per workgroup of the piece pass (4 per thread)
constexpr uint32_t kNoRank = 0xFFFFFFFFu;
constexpr uint64_t kEmptySlot = ~0ull;

// classes
enum : uint32_t { kL = 0, kN = 1, kW = 2, kO = 3 };

// status bits
enum : uint32_t { kStUtf8 = 1u, kStSpin = 2u, kStDocOff = 4u };

struct Counters {
  uint32_t status;      // kSt* bits, OR-ed by kernels
  uint32_t n_list[3];   // entries in the merge lists (2..16, 17..64, longer)
  uint32_t work;        // next merge work item
  uint32_t k3_ticket;   // tile ticket of the count scan
  uint32_t total;       // tokens in the output
  uint32_t pad;
};

// Read-only device tables built by tok_load.
struct Tables {
  const uint64_t* merge_slots;  // (left << 44 | right << 24 | rank), kEmptySlot = empty
  uint32_t merge_mask;          // slots - 1 (power of two)
  const uint32_t* pair_rank;    // [256 * 256] rank of byte pair (a, b), or kNoRank
  const uint64_t* word_slots;   // 2 x uint64 per slot, see word_key()
  uint32_t word_mask;           // slots - 1; 0 with word_slots == nullptr disables
  const uint32_t* tok_len;      // bytes of each token ID
};

// Per-call device buffers.
struct Bufs {
  uint16_t* flags;
  int32_t* staging;
  uint8_t* cnt8;
  uint32_t* chunk_cnt;
  uint32_t* chunk_excl;
  uint2* list[3];
  uint32_t* ws_sym;
  uint32_t* ws_rk;
  uint64_t* ws_sel;
  unsigned long long* scan_state;
  Counters* ctr;
};

__host__ __device__ inline uint64_t mix64(uint64_t x) {
  x ^= x >> 31;
  x *= 0x7FB5D329728EA185ull;
  x ^= x >> 27;
  x *= 0x81DADEF4BC2DD44Dull;
  x ^= x >> 33;
  return x;
}

__host__ __device__ inline uint32_t merge_hash(uint32_t left, uint32_t right) {
  return (uint32_t)mix64(((uint64_t)left << 20) | right);
}

// Whole-piece key of a byte string of 2..13 bytes: a = bytes 0..7 (little
// endian, zero padded), b = bytes 8..12 | len << 40.  A stored slot adds the
// token ID in bits 44..63 of b.
__host__ __device__ inline uint32_t word_hash(uint64_t a, uint64_t b) {
  return (uint32_t)mix64(a * 0x9E3779B97F4A7C15ull ^ (b + 0x632BE59BD9B4E019ull));
}

// Kernel launchers (defined in the .hip files).
void launch_reset(Bufs b, uint32_t n_tiles, const uint64_t* doc_off, uint32_t n_docs, uint64_t n,
                  hipStream_t s);
void launch_pretok(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs,
                   int pattern, Bufs b, hipStream_t s);
void launch_pieces(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s);
void launch_merge(const uint8_t* text, uint64_t n, Tables t, Bufs b, hipStream_t s);
void launch_assemble(uint64_t n, int32_t* out, uint64_t cap, Bufs b, hipStream_t s);
void launch_doc_offsets(uint64_t n, const uint64_t* doc_off, uint32_t n_docs, uint64_t* out_off,
                        Tables t, Bufs b, hipStream_t s);

}  // namespace tok
