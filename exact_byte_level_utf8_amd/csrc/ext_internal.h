// Internal declarations of the passes around the tokenization pipeline:
// the added-token literal pass (k_added.hip) and the device side of append
// repair (k_repair.hip).  Kept apart from tok_internal.h, which holds what the
// pipeline's own kernels use.
#pragma once

#include "tok_internal.h"

namespace tok {

// Device tables of the added-token literals (set by tok_set_added_tokens).
struct Literals {
  const uint8_t* bytes;   // literal i is bytes[off[i] .. off[i + 1])
  const uint32_t* off;
  const int32_t* ids;
  const uint32_t* key2;   // [65536] by first two bytes: (first << 16 | count) into order, longest first
  const uint16_t* order;  // literal indices of two or more bytes, grouped by key2
  const int32_t* key1;    // [256] the one-byte literal of each byte, or -1
  const uint32_t* first;  // [8] bit b: some literal starts with byte b
  const uint64_t* by_id;  // (id << 32 | literal index), sorted by ID
  uint32_t n;
};

// Per-call buffers of the literal pass (sized by the context's capacity and
// document count).  The k taken literals cut the caller's documents into
// parts: each literal is a part, and so is each stretch between two cuts.
struct LitBufs {
  uint64_t* cand;       // per tile: up to kLitTile (position << 32 | literal) in position order
  uint32_t* tile_cnt;   // candidates found in each tile
  uint64_t* sel;        // taken literals, in order
  uint64_t* cut;        // parts + 1 cut points: document boundaries, literal starts and ends, merged
  int32_t* part_lit;    // per part: the ID of the taken literal it is, or -1
  uint32_t* doc_part;   // per document boundary: its index among the cut points
  uint64_t* out_off;    // the parts' output offsets from the pipeline
  uint32_t* fin;        // final output offset of each part (and the total)
  uint32_t* misc;       // [0] tokens the pipeline produced, [1] literals taken k, [2] parts, [3] documents,
                        // [4] selection workgroups finished (zeroed by the match kernel)
  int32_t* ids;         // the pipeline's output, before the literal IDs go in
  uint32_t* spans;      // with span export: the first byte of each of those IDs
  // Literal IDs folded into the piece pass (calls without span export): a
  // taken literal is then one piece whose token is its ID, and the pipeline's
  // output is the result.  lmark[b]: 1 where a taken literal starts, 2 on
  // its later bytes, else 0 (the match kernel clears its tile's bytes, the
  // pre-tokenization kernel marks the taken literals on its way in);
  // lid_at[b]: the ID of the literal that starts at b (meaningful only where
  // lmark[b] is 1).
  uint8_t* lmark;
  int32_t* lid_at;
  uint32_t fold;        // this call folds the literal IDs in
};

constexpr int kLitTile = 1024;  // bytes per workgroup of the literal match
constexpr int kLitMax = 64;     // longest added-token literal, bytes
constexpr uint32_t kLitMaxCount = 4096;

// Arguments of the device repair's match and splice (one workgroup).
struct RepairArgs {
  const uint8_t* win;  // text[ws0, new_len) on the device
  uint64_t ws0, ws, margin, old_len, new_len;
  const int32_t* fresh;          // IDs of the window text[ws, new_len)
  const uint32_t* fspan;         // their first bytes, counted from ws
  const uint32_t* fresh_total;   // how many (the window encode's count word)
  int32_t* session;              // stored IDs on the device, spliced in place
  uint64_t n_session, cap;
  const uint32_t* tok_len;
  const uint8_t* tok_bytes;      // token t is tok_bytes[tok_off[t] .. + tok_len[t])
  const uint64_t* tok_off;
  uint32_t vocab, max_tok_len;  // max_tok_len: the longest token or literal
  int pattern;                   // TOK_PAT_GPT2, TOK_PAT_LLAMA3 or TOK_PAT_O200K
  Literals L;                    // added-token literals (L.n == 0: none); their IDs name no token
  uint32_t* st_off;              // scratch: first byte of the r-th stored record from the end
  uint64_t* splice;              // device words: [0] first window record to copy, [1] session
                                 // index it goes to, [2] how many (0: nothing to copy)
  uint64_t max_fresh;            // bound on the window's record count (its byte count)
  RepairOut* out;                // host-mapped result
  const uint64_t* err_utf8;      // host-mapped error words of the window encode: when either holds
  const uint64_t* err_docs;      // gen, the window's IDs are not a result and the session is left alone
  uint64_t gen;
};

// Launchers (defined in k_added.hip and k_repair.hip).
void launch_literal_pass(const uint8_t* text, uint64_t n, const uint64_t* doc_off, uint32_t n_docs, Literals L,
                         LitBufs lb, Counters* ctr, uint64_t gen, hipStream_t s);
void launch_literal_insert(uint64_t n, Literals L, LitBufs lb, int32_t* out, uint32_t* spans, uint64_t cap,
                           uint64_t* out_off, Counters* ctr, uint64_t gen, hipStream_t s);
// With the literal IDs folded into the piece pass: the caller's document
// offsets (n_docs + 1 of them) from the pipeline's part offsets.
void launch_literal_doc_offsets(LitBufs lb, uint64_t* out_off, uint32_t n_docs, hipStream_t s);
// The match kernel, then, for a window of more than a few thousand records,
// the copy of the window's IDs after the splice (a grid sized by a.max_fresh).
void launch_repair_match(const RepairArgs& a, hipStream_t s);

}  // namespace tok
