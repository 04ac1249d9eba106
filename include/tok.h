/*
 * tok.h -- C ABI of the exact byte-level BPE tokenizer for AMD Instinct MI355X
 * (gfx950).
 *
 * One output contract for every call: the returned token IDs equal the full
 * tokenization of the request text under one frozen configuration (TokTier,
 * section 5.2 "Exactness" and Appendix A, Definition A.2; Delta Tokenizer, the
 * contract shared by all of its request paths; GraphTok, section 3
 * "Background", where exactness means the complete ordered ID sequence).  A
 * call that cannot honour the contract returns an error code and writes no
 * partial answer the caller could mistake for a result: a failure costs work,
 * never exactness (TokTier, section 3, the repair search may miss a boundary
 * but never accepts a wrong one).
 *
 * Configuration (fixed at tok_load):
 *   - merges: n_merges ordered pairs (left, right) of token IDs, in rank order.
 *     IDs 0..255 are the single bytes; merge r creates ID 256 + r.  Ranks are
 *     keyed by the ordered ID pair (GraphTok, section 4: the lowest rank wins,
 *     the leftmost pair on equal rank).
 *   - pattern: the pre-tokenizer family, TOK_PAT_GPT2, TOK_PAT_LLAMA3 or TOK_PAT_O200K.
 *     encode(x) = concatenation over the pre-tokenization pieces p of x, in
 *     order, of bpe(bytes(p)) (TokTier, Appendix A, Definition A.2 and
 *     Lemma A.3).
 *
 * Text is UTF-8.  Malformed input (overlong forms, surrogates, values above
 * U+10FFFF, truncated or stray continuation bytes, a sequence cut by a document
 * boundary) is rejected as a whole with TOK_E_UTF8: the pages define
 * tokenization over Unicode text, so a byte string that is not UTF-8 has no
 * reference result to match.
 *
 * Threading: a context serves one caller at a time (GraphTok, section 5
 * "Implementation", one context per dispatcher).  Device-pointer calls enqueue
 * their work on the given stream and return after that stream has completed
 * it; the call's count and error status come back through pinned host memory
 * written by the kernels, so a call costs one stream synchronization.
 *
 * Ownership: every pointer argument is owned by the caller and is not retained
 * after the call returns; the context owns all of its device memory.
 */
#ifndef EXACT_BYTE_LEVEL_UTF8_TOK_H
#define EXACT_BYTE_LEVEL_UTF8_TOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tok_ctx tok_ctx;

/* Status codes. */
#define TOK_OK 0
#define TOK_E_ARG 1        /* null pointer, non-monotone offsets, bad flag  */
#define TOK_E_BADMERGES 2  /* operand >= 256 + rank, repeated pair, too many */
#define TOK_E_PATTERN 3    /* pattern id not supported                      */
#define TOK_E_UTF8 4       /* malformed UTF-8 anywhere in the input         */
#define TOK_E_CAPACITY 5   /* output buffer too small; *n_out = required    */
#define TOK_E_TOOLONG 6    /* input longer than TOK_MAX_BYTES               */
#define TOK_E_DEVICE 7     /* a HIP runtime call failed                     */
#define TOK_E_NOMEM 8      /* device or pinned host allocation failed       */
#define TOK_E_SESSION 9    /* repair: stored IDs do not spell the old text  */

/* Pre-tokenizer families. */
#define TOK_PAT_GPT2 0   /* 's|'t|'re|'ve|'m|'ll|'d| ?L+| ?N+| ?[^\s L N]+|\s+(?!\S)|\s+ */
#define TOK_PAT_LLAMA3 1 /* (?i:contractions)|[^\r\n L N]?L+|N{1,3}| ?[^\s L N]+[\r\n]*|\s*[\r\n]+|\s+(?!\S)|\s+ */
/* Case-splitting family (the o200k lineage as TokTier, section 4, describes it:
 * the Llama-3 style with a case-boundary rule inside letter runs, marks
 * joining letters and contractions as a suffix of a letter piece):
 * P?H*T+S?|P?H+T*S?|N{1,3}| ?[^\s L N]+[\r\n]*|\s*[\r\n]+|\s+(?!\S)|\s+ with H = upper-case or
 * caseless letters or marks, T = lower-case or caseless letters or marks,
 * P = one char that is not CR, LF, a letter or a number, S = an optional
 * case-insensitive 's 't 're 've 'm 'll 'd. */
#define TOK_PAT_O200K 2

/* Largest input of one call, in bytes (token counts and offsets are 32-bit
 * on the device). */
#define TOK_MAX_BYTES 0xFFFF0000ull
/* Largest merge list: token IDs are 20-bit fields in the device tables. */
#define TOK_MAX_MERGES 1040000ull

/*
 * tok_opts -- per-context options of tok_load (the survey's load options;
 * the repair parameters are per-tokenizer values in the pages: TokTier,
 * section 3 "Incremental repair", a first window of w = 512 characters
 * doubled at most five times before the full re-encode; Delta Tokenizer,
 * Table S1, the certificate's margin and bound).  A NULL opts means the
 * defaults below; tok_opts_default fills a struct with them.
 *
 * device:           HIP device ordinal the context runs on (default 0).
 * initial_bytes:    input bytes the per-call device scratch covers from the
 *                   start (0, the default: allocated by the first call and
 *                   grown in powers of two, as every call does when its input
 *                   is larger).
 * repair_window:    code points of the stored text in the first repair
 *                   window (default 512; 1 .. 2^24).
 * repair_doublings: window doublings before the whole text is encoded
 *                   (default 5; at most 24).
 * repair_margin:    code points into the window that a certifying boundary
 *                   must lie (default 8; at most 2^20).  Any value is exact
 *                   (the certificate holds for every left context); a margin
 *                   keeps the splice away from the window's cut.
 * handoff_wait_us:  TOK_PAT_O200K only: microseconds a 1 KiB tile of the
 *                   pre-tokenization waits for the previous tile's cursor
 *                   (the first piece start past that tile) before finding it
 *                   itself by walking back to the cut its segment started at
 *                   (default 1000000; at most 10^7).  The wait always ends
 *                   well before this in practice; 0 makes every tile walk
 *                   back (slow on long stretches without a cut, for tests).
 *                   Results never depend on it.
 */
typedef struct tok_opts {
  int32_t device;
  uint32_t repair_window;
  uint64_t initial_bytes;
  uint32_t repair_doublings;
  uint32_t repair_margin;
  uint32_t handoff_wait_us;
} tok_opts;

void tok_opts_default(tok_opts* opts);

/*
 * tok_load -- validate a configuration and build its device tables.
 *
 * merges:   host array of 2 * n_merges uint32: (left, right) of merge r at
 *           [2r, 2r+1].  Copied; the caller may free it on return.
 * pattern:  TOK_PAT_GPT2, TOK_PAT_LLAMA3 or TOK_PAT_O200K.
 * opts:     load options (above), or NULL for the defaults.  Read during the
 *           call only.
 * out:      receives the context (NULL on error).
 *
 * Builds, on the device: the (left, right) -> rank open-addressing table, a
 * direct byte-pair rank table, the token byte lengths, and whole-piece
 * tables of vocabulary strings of 2..28 bytes whose own BPE is the single token
 * (the whole-vocabulary-hit shortcut of TokTier, section 4 "GPU BPE", applied only where it
 * provably cannot change an ID: each string is checked by running the GPU
 * merge kernels on it once at load).
 *
 * Errors: TOK_E_ARG (null out, merges NULL with n_merges > 0, an option out
 * of its range), TOK_E_BADMERGES (left or right >= 256 + r, a repeated pair,
 * n_merges > TOK_MAX_MERGES), TOK_E_PATTERN, TOK_E_DEVICE, TOK_E_NOMEM.
 */
int tok_load(const uint32_t* merges, size_t n_merges, int pattern, const tok_opts* opts, tok_ctx** out);

/* Release the context and all its device and pinned memory.  NULL is a no-op. */
void tok_free(tok_ctx* ctx);

/* Static message for a status code. */
const char* tok_strerror(int code);

/*
 * tok_encode -- exact encode of one request held in host memory.
 *
 * text, len: UTF-8 request (len may be 0; text may be NULL when len is 0).
 * ids, cap:  host output buffer of cap int32.  cap >= len always suffices
 *            (every token covers at least one byte).
 * n_out:     receives the token count T (also on TOK_E_CAPACITY, where it is
 *            the required cap; nothing is written to ids then).
 *
 * The text is staged through pinned memory to the context's stream; the
 * pipeline runs on the device; the count and then the IDs come back.
 * Errors: TOK_E_ARG, TOK_E_TOOLONG, TOK_E_UTF8 (*n_out = 0), TOK_E_CAPACITY,
 * TOK_E_DEVICE, TOK_E_NOMEM.
 */
int tok_encode(tok_ctx* ctx, const uint8_t* text, size_t len, int32_t* ids, size_t cap,
               size_t* n_out);

/*
 * tok_encode_dev -- as tok_encode with device-resident input and output: no
 * host/device transfer of text or IDs (GraphTok, section 5, the device
 * buffer handoff).  d_text: len bytes on the context's device; d_ids: cap
 * int32 on the device; stream: hipStream_t to enqueue on (NULL = the
 * context's own stream, a blocking stream: it runs after work queued before
 * the call on the legacy default stream).  On TOK_E_CAPACITY the first cap IDs are written and
 * *n_out is the full count; on TOK_E_UTF8 the content of d_ids is unspecified.
 */
int tok_encode_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, int32_t* d_ids, size_t cap,
                   size_t* n_out, void* stream);

/*
 * tok_encode_dev_noalloc -- tok_encode_dev that allocates nothing, for
 * callers that cannot allocate device memory during a call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, results and errors as tok_encode_dev, for len up to
 * TOK_NOALLOC_MAX_BYTES (else TOK_E_TOOLONG, before any device work).  Every
 * per-call device buffer comes from one fixed array that the library holds on
 * each GPU it runs on until the process ends (about 20 MiB); the call makes
 * no hipMalloc, hipFree or other allocation.  All calls on one GPU share that
 * array, so calls that overlap on one GPU (from any context or thread) race:
 * the caller must serialize them.  Added-token literals are not supported
 * here (TOK_E_ARG when the context has any): their pass needs more buffers.
 * The array's address is looked up at tok_load; TOK_E_DEVICE if that failed.
 */
#define TOK_NOALLOC_MAX_BYTES 0x100000ull
int tok_encode_dev_noalloc(tok_ctx* ctx, const uint8_t* d_text, size_t len, int32_t* d_ids, size_t cap,
                           size_t* n_out, void* stream);

/*
 * tok_encode_batch -- encode n_docs independent documents in one pipeline
 * pass (GraphTok, section 5 "Implementation", the batch entry point; TokTier,
 * section 4 "GPU BPE", multi-document batches).  Document i is text[doc_off[i] .. doc_off[i+1]);
 * documents are hard boundaries: no piece, code point or token spans two of
 * them; an empty document yields no IDs.
 *
 * doc_off: host array of n_docs + 1 non-decreasing byte offsets with
 *          doc_off[0] = 0 (the text length is doc_off[n_docs]).
 * ids,cap: host output, concatenated IDs of all documents in order.
 * out_off: host array of n_docs + 1: document i's IDs are
 *          ids[out_off[i] .. out_off[i+1]).  out_off[n_docs] is the total.
 * Errors: as tok_encode, plus TOK_E_ARG for offsets that decrease, do not
 * start at 0, or n_docs == 0.  On TOK_E_CAPACITY out_off is filled and ids
 * is untouched.
 */
int tok_encode_batch(tok_ctx* ctx, const uint8_t* text, const uint64_t* doc_off, size_t n_docs,
                     int32_t* ids, size_t cap, uint64_t* out_off);

/*
 * tok_encode_batch_dev -- as tok_encode_batch with device-resident text
 * (d_text, len bytes), offsets (d_doc_off: n_docs + 1 uint64 on the device;
 * the device checks d_doc_off[0] == 0, d_doc_off[n_docs] == len and that they
 * never decrease, else TOK_E_ARG), IDs and output offsets (d_out_off: n_docs
 * + 1 uint64 on the device).  n_out receives the total count.  stream as in
 * tok_encode_dev.
 */
int tok_encode_batch_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, const uint64_t* d_doc_off,
                         size_t n_docs, int32_t* d_ids, size_t cap, uint64_t* d_out_off,
                         size_t* n_out, void* stream);

/*
 * tok_encode_spans_dev -- tok_encode_dev / tok_encode_batch_dev that also
 * exports, for every ID, the byte where its token starts (span export:
 * TokTier, section 7 "Session-state construction" and Appendix E, "Route C:
 * GPU full tokenization with span export": each ID's token byte length is
 * gathered and a cumulative sum gives the offsets, on the device).
 *
 * d_doc_off, n_docs: as tok_encode_batch_dev (then d_out_off receives the
 *            per-document output offsets), or NULL / 0 for one request
 *            (d_out_off is then ignored and may be NULL).
 * d_ids, d_spans, cap: device arrays of cap int32 IDs and cap uint32 byte
 *            offsets.  d_spans[k] counts from the start of d_text (in a batch
 *            too, not from the document's start); token k covers
 *            d_text[d_spans[k] .. d_spans[k] + its byte length), and the
 *            tokens of a document tile it without gaps.
 * Errors, stream, capacity: as tok_encode_dev (on TOK_E_CAPACITY the first
 * cap IDs and offsets are written).
 */
int tok_encode_spans_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len, const uint64_t* d_doc_off,
                         size_t n_docs, int32_t* d_ids, uint32_t* d_spans, size_t cap, uint64_t* d_out_off,
                         size_t* n_out, void* stream);

/*
 * tok_encode_spans -- tok_encode with span export into host memory: ids and
 * spans are host arrays of cap entries; spans[k] is the byte of text where
 * token k starts.  Errors as tok_encode (on TOK_E_CAPACITY neither array is
 * written).
 */
int tok_encode_spans(tok_ctx* ctx, const uint8_t* text, size_t len, int32_t* ids, uint32_t* spans, size_t cap,
                     size_t* n_out);

/*
 * tok_pretokenize_dev -- the pre-tokenization stage alone, for split-level
 * checks (TokTier, section 5.2, compares pieces before IDs).  Writes one
 * uint16 per 16-byte chunk of d_text to d_flags (ceil(len / 16) words on the
 * device): bit i of word c is set iff byte 16c + i starts a piece.  A
 * document start always starts a piece.  d_doc_off / n_docs as in
 * tok_encode_batch_dev, or NULL / 0 for one document.  Added-token literals
 * are not applied here: this is the pattern's stage alone.
 */
int tok_pretokenize_dev(tok_ctx* ctx, const uint8_t* d_text, size_t len,
                        const uint64_t* d_doc_off, size_t n_docs, uint16_t* d_flags, void* stream);

/*
 * tok_repair -- exact encode of a session after an append, from the session's
 * stored IDs (TokTier, section 3, windowed repair with a splice certificate,
 * and Appendix A, Definition A.4, Theorem A.5, Corollary A.6; Delta Tokenizer,
 * reference-identical tokenization of session deltas).
 *
 * text:        host bytes text[0 .. new_len): the stored text A =
 *              text[0 .. old_len) followed by the appended text B.
 * session_ids: host array of cap int32; on entry session_ids[0 .. n_session)
 *              must equal the encode of A; on success session_ids[0 .. *n_out)
 *              equals the encode of A + B, spliced in place (a prefix of the
 *              stored IDs is left untouched).
 * info:        optional; receives where the accepted window started, the splice
 *              byte, the number of stored IDs kept, the window doublings and
 *              whether the whole text was encoded.
 *
 * The last w code points of A plus B are encoded on the device (w = 512,
 * doubling up to five times); a run of equal (offset, ID) records of the
 * stored and the fresh encode is accepted if it holds at least two tokens,
 * spans more bytes than the longest token and contains, at least 8 code points
 * into the window, a synchronizing transition (tok_sync_boundary); the
 * result is the stored IDs up to the end of the last such run followed by the
 * fresh IDs.  Without such a run the whole text is encoded.  Work is O(w +
 * |B|): the stored IDs are walked back from their end through the token byte
 * lengths.
 *
 * Errors: TOK_E_ARG (null pointers, old_len > new_len, n_session > cap),
 * TOK_E_TOOLONG, TOK_E_SESSION (the walked-back stored IDs do not spell the
 * tail of A, or do not cover it, or exactly one of old_len and n_session is
 * 0), TOK_E_UTF8, TOK_E_CAPACITY (*n_out = required cap; session_ids is
 * unchanged), TOK_E_DEVICE, TOK_E_NOMEM.
 */
typedef struct tok_repair_info {
  uint64_t window_start;  /* first byte of the accepted window (0 after a full encode) */
  uint64_t splice_byte;   /* end of the accepted equal run                          */
  uint64_t kept;          /* stored IDs kept                                        */
  uint32_t widenings;     /* window doublings done                                  */
  uint32_t full;          /* 1 if the whole text was encoded                        */
} tok_repair_info;

int tok_repair(tok_ctx* ctx, int32_t* session_ids, size_t n_session, size_t cap, const uint8_t* text,
               size_t old_len, size_t new_len, size_t* n_out, tok_repair_info* info);

/*
 * tok_repair_dev -- tok_repair for a session whose IDs live in device memory
 * (TokTier, section 3 and Appendix A as for tok_repair; "Delta-aware routing" and
 * Appendix E: the match and splice run on the device, so the IDs never cross
 * to the host).
 *
 * d_session_ids: device array of cap int32 (the context's device); on entry
 *                d_session_ids[0 .. n_session) must equal the encode of
 *                text[0 .. old_len); on success d_session_ids[0 .. *n_out)
 *                equals the encode of text[0 .. new_len), spliced in place.
 * text:          host bytes text[0 .. new_len), as for tok_repair.
 *
 * Each attempt copies the window text[ws - (longest token, rounded up to 4
 * bytes) .. new_len) to the device, encodes text[ws .. new_len) with span
 * export, and one workgroup then walks the stored IDs back from their end
 * through the token byte lengths (checking that they spell the text),
 * matches the (byte offset, ID) records, picks the splice exactly as
 * tok_repair does and writes the window's IDs after it: one synchronization
 * per attempt.  The window widening, the gates and the full-encode fallback
 * are tok_repair's, with added-token literals too.
 * Runs on the context's own stream, ordered after work on the legacy default
 * stream.
 *
 * Errors: as tok_repair; on TOK_E_CAPACITY (*n_out = required cap) and on
 * every other error the session IDs are left unchanged.
 */
int tok_repair_dev(tok_ctx* ctx, int32_t* d_session_ids, size_t n_session, size_t cap, const uint8_t* text,
                   size_t old_len, size_t new_len, size_t* n_out, tok_repair_info* info);

/*
 * tok_sync_boundary -- 1 if a byte where code point prev_cp is followed by
 * code point cp is a synchronizing transition of the pattern family: a class
 * change such that, for any text before it, the pieces from that byte on are
 * those of the text from that byte alone, and the pieces before it do not
 * depend on the text after cp (the stable boundary of TokTier, section 3 and
 * Appendix A).  No context needed; never touches the device.
 */
int tok_sync_boundary(int pattern, uint32_t prev_cp, uint32_t cp);

/*
 * tok_set_added_tokens -- added-token literals (special tokens such as
 * "<|endoftext|>") that take precedence over the pattern (TokTier, section 4
 * "Single-request path": a leftmost-longest literal pass extracts added and
 * special tokens before the tokenizer family handles the remaining segments;
 * GraphTok, section 4 "Design": added entries take precedence over ordinary
 * pre-tokenization, their IDs are emitted directly and only the unmatched
 * regions reach the family predicate).
 *
 * Literal i is bytes[off[i] .. off[i+1]) (off: n + 1 non-decreasing host
 * offsets, off[0] = 0) with token ID ids[i] >= 0 (any value; usually at or
 * above the vocabulary size).  Each literal is 1..64 bytes of well-formed
 * UTF-8; no string twice; n <= 4096.  n = 0 removes the literals.
 *
 * Afterwards every encode call scans the text left to right: at the
 * first position where some literal matches, the longest one there is taken
 * and its ID emitted, and the scan goes on after it; each segment between
 * taken literals is encoded as a request of its own (its pieces and merges
 * never reach across a literal).  Literals are matched on the raw bytes, with
 * no whitespace stripping, word-boundary or normalization options.  The
 * literal pass and the insertion of the literal IDs run on the device in the
 * same stream as the pipeline (still one synchronization per call).
 * tok_repair also refuses a cut inside any literal occurrence, taken or not
 * (Delta Tokenizer, section 3, the cut guard), and counts a literal's length
 * in its gates; it encodes the whole text when a literal's ID is also a
 * vocabulary ID or another literal's.  tok_repair_dev does the same on the
 * device.  The batch calls apply the
 * pass within each document (a literal never spans two documents), and span
 * export covers literals (a literal's span is its first byte).
 *
 * Errors: TOK_E_ARG (null pointers, a length of 0 or over 64, a negative ID, a
 * repeated string, n > 4096), TOK_E_UTF8 (a literal is not well-formed UTF-8),
 * TOK_E_NOMEM, TOK_E_DEVICE.  On error no literals are set.
 */
int tok_set_added_tokens(tok_ctx* ctx, const uint8_t* bytes, const uint64_t* off, size_t n, const int32_t* ids);

/*
 * tok_fill_scratch -- diagnostic: fill every per-call device buffer the
 * context holds (pipeline scratch, literal-pass buffers, staging of the
 * host-memory calls) with the byte value (0..255) and wait for it.  No call's
 * result depends on what an earlier call left in those buffers; tests poison
 * them between calls of different sizes to show it (GraphTok, section 6.2,
 * stale state across replays).  Device tables and the caller's buffers are
 * not touched.  Errors: TOK_E_ARG (null context, value out of range),
 * TOK_E_DEVICE.
 */
int tok_fill_scratch(tok_ctx* ctx, int value);

/* Context facts. */
typedef struct tok_info {
  uint32_t pattern;
  uint32_t n_merges;
  uint32_t vocab_size;     /* 256 + n_merges                                 */
  uint32_t max_token_len;  /* longest token, bytes                           */
  uint32_t n_whole;        /* whole-piece table entries (self-encoding)      */
  uint32_t n_not_self;     /* 2..28-byte vocab strings whose BPE differs     */
  uint64_t config_hash;    /* FNV-1a over pattern and merges                 */
} tok_info;

int tok_get_info(const tok_ctx* ctx, tok_info* info);

/*
 * Token byte lengths, for host-side offset arithmetic: writes min(n,
 * vocab_size) lengths to len_out (host).  Returns the vocabulary size.
 */
size_t tok_token_lengths(const tok_ctx* ctx, uint32_t* len_out, size_t n);

/*
 * Stage timing (GraphTok, section 6.11, the per-stage profile).
 * tok_set_profiling(ctx, stages): stages is a bit mask of the stages to time
 * (0 = off); in every later call a pair of HIP events brackets the kernel of
 * each timed stage on the stream it runs on (timing-only events, without a
 * system-scope fence).  tok_stage_ms writes the last call's stage durations in ms, 0 for
 * stages not timed: [0] pre-tokenization (with the per-call set-up of the
 * later passes), [1] piece pass (single bytes, whole-piece hits, merge
 * rounds of the remaining pieces, the longer ones by the whole workgroup,
 * one run of IDs per 1 KiB tile), [2] assembly (output offsets of the runs
 * and their copy).  Returns the number
 * of stages written (at most n).  tok_set_profiling: TOK_E_ARG for a null
 * context or a negative mask.
 */
/*
 * Graph replay (GraphTok, section 4 "Design", graph-resident execution, and
 * section 5 "Implementation", captured execution).  tok_set_graph(ctx, 1)
 * turns it on: a call whose shape -- text and output pointers, sizes,
 * document offsets, stream -- was met before replays one HIP graph of the
 * three kernels captured for that shape, instead of three launches; a shape
 * met for the first time runs eagerly.  At most 8 graphs are held (least
 * recently used evicted); growing the context's buffers drops them all, and
 * so does tok_set_graph(ctx, 0), the default.  Calls with stage timing on,
 * tok_pretokenize_dev and empty batches always run eagerly.  Results are the
 * same either way.  A replay reuses the launch geometry of its shape, so
 * graphs are keyed by exact size rather than by power-of-two capacity class.
 * tok_set_graph: TOK_E_ARG for a null context or on outside {0, 1}.
 * tok_graph_count: the number of graphs held (0 for a null context).
 */
int tok_set_graph(tok_ctx* ctx, int on);
size_t tok_graph_count(const tok_ctx* ctx);

#define TOK_STAGE_PRETOK 1
#define TOK_STAGE_PIECES 2
#define TOK_STAGE_ASSEMBLE 4
#define TOK_STAGES_ALL 7
int tok_set_profiling(tok_ctx* ctx, int stages);
int tok_stage_ms(const tok_ctx* ctx, float* ms, int n);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_BYTE_LEVEL_UTF8_TOK_H */
