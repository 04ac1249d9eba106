// tok_encode_dev_noalloc: tok_encode_dev for callers that cannot allocate
// device memory during a call (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// Every per-call buffer of the pipeline (flag words, tile runs, tile counts
// and group sums, the long-piece workspace) is carved from one
// file-scope device array sized for TOK_NOALLOC_MAX_BYTES of input.  Each GPU
// the library runs on holds its own copy of the array until the process
// ends.  Host code never passes the array's name to a kernel: its device
// address is looked up once per device, at the first tok_load on that device
// (with the device current), and kept per device.  All calls on one GPU share
// the array, so calls that overlap on one GPU race; the kernels clear what
// must start at zero (the group sums) in every call.  The hand-over words of
// the case-splitting pre-tokenization (a call counter, a count of the
// workgroups that read it, and per-tile cursors tagged with it) start at zero with the array and are kept consistent by
// every call.
#include <mutex>

#include "ctx.h"

namespace {

constexpr uint64_t kNaMax = TOK_NOALLOC_MAX_BYTES;
constexpr uint64_t kNaTiles = kNaMax / kPieceTile;

constexpr uint64_t up256(uint64_t x) { return (x + 255) & ~255ull; }

// byte offsets of the buffers within the array (each 256-byte aligned)
constexpr uint64_t kOffFlags = 0;
constexpr uint64_t kOffStaging = up256(kOffFlags + (kNaMax / kChunk + 8) * 2);
constexpr uint64_t kOffTileCnt = up256(kOffStaging + (kNaMax + 64) * 4);
constexpr uint64_t kOffTileFirst = up256(kOffTileCnt + kNaTiles * 4);
constexpr uint64_t kOffSum1 = up256(kOffTileFirst + kNaTiles * 4);
constexpr uint64_t kOffSum2 = up256(kOffSum1 + ((kNaTiles >> kSum1Shift) + 1) * 4);
constexpr uint64_t kOffWsSym = up256(kOffSum2 + ((kNaTiles >> kSum2Shift) + 1) * 4);
constexpr uint64_t kOffWsRk = up256(kOffWsSym + (kNaMax + 64) * 4);
constexpr uint64_t kOffWsSel = up256(kOffWsRk + (kNaMax + 64) * 4);
constexpr uint64_t kOffHandTick = up256(kOffWsSel + (kNaMax + 64) * 8);
constexpr uint64_t kOffHandState = up256(kOffHandTick + kHandTickWords * 8);
constexpr uint64_t kScratchBytes = up256(kOffHandState + (kNaMax / kPretokTile + 1) * 8);
static_assert(kScratchBytes < (24ull << 20), "the no-allocation scratch stays near 20 MiB");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

}  // namespace

// The array's device address on `device` (which is current), looked up on
// the first call for that device; nullptr if the lookup failed.
uint8_t* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[device] = static_cast<uint8_t*>(p);
  }
  return g_ptr[device];
}

extern "C" {

int tok_encode_dev_noalloc(tok_ctx* ctx, const uint8_t* d_text, size_t len, int32_t* d_ids, size_t cap,
                           size_t* n_out, void* stream) {
  if (!ctx || !n_out || (!d_text && len) || (!d_ids && cap)) return TOK_E_ARG;
  *n_out = 0;
  if (len > TOK_NOALLOC_MAX_BYTES) return TOK_E_TOOLONG;
  if (ctx->n_lit) return TOK_E_ARG;  // the literal pass needs buffers this array does not hold
  if (len == 0) return TOK_OK;
  DeviceGuard g(ctx->device);
  uint8_t* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    base = ctx->device >= 0 && ctx->device < kMaxDevices ? g_ptr[ctx->device] : nullptr;
  }
  if (!base) return TOK_E_DEVICE;  // tok_load looks the address up; it failed there
  Bufs bb{};
  bb.flags = reinterpret_cast<uint16_t*>(base + kOffFlags);
  bb.staging = reinterpret_cast<int32_t*>(base + kOffStaging);
  bb.tile_cnt = reinterpret_cast<uint32_t*>(base + kOffTileCnt);
  bb.tile_first = reinterpret_cast<uint32_t*>(base + kOffTileFirst);
  bb.sum1 = reinterpret_cast<uint32_t*>(base + kOffSum1);
  bb.sum2 = reinterpret_cast<uint32_t*>(base + kOffSum2);
  bb.ws_sym = reinterpret_cast<uint32_t*>(base + kOffWsSym);
  bb.ws_rk = reinterpret_cast<uint32_t*>(base + kOffWsRk);
  bb.ws_sel = reinterpret_cast<uint64_t*>(base + kOffWsSel);
  bb.hand_tick = reinterpret_cast<uint64_t*>(base + kOffHandTick);  // zero at load, kept by every call
  bb.hand_state = reinterpret_cast<uint64_t*>(base + kOffHandState);
  bb.hand_wait = ctx->b.hand_wait;
  bb.ctr = ctx->d_ctr;
  bb.n_docs_dev = nullptr;
  bb.gen = ++ctx->gen;
  hipStream_t s = stream ? (hipStream_t)stream : ctx->stream;
  ctx->enqueue(d_text, len, nullptr, 0, d_ids, nullptr, cap, nullptr, s, bb, true, nullptr);
  HIP_OK(hipGetLastError());
  HIP_OK(hipStreamSynchronize(s));
  ctx->collect_stage_times(kStages);
  const volatile Counters* c = ctx->h_ctr;
  if (c->err_utf8 == bb.gen) return TOK_E_UTF8;
  if (c->done != bb.gen) return TOK_E_DEVICE;
  *n_out = c->total;
  return c->total > cap ? TOK_E_CAPACITY : TOK_OK;
}

}  // extern "C"
