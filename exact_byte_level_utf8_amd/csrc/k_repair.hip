// Device side of append repair over a session kept in device memory
// (tok_repair_dev): after the window [ws, new_len) is encoded with span
// export, one workgroup matches the window's (byte offset, ID) records
// against the stored ones, picks the splice and writes it into the session
// buffer, so the IDs never cross to the host (TokTier, section 3, windowed
// repair with a splice certificate; Appendix A, Definition A.4, Theorem A.5,
// Corollary A.6; "Delta-aware routing" and Appendix E, the match and splice moved onto
// the device).  The decisions are those of the host repair, record for
// record:
//   - stored records: walked back from the session's end through the token
//     byte lengths (a suffix scan) until they cover [ws, old_len); each must
//     spell its bytes of the text, else the session does not match;
//   - a window record is equal when a stored record starts at the same byte
//     with the same ID; runs of consecutive equal records are the candidates;
//   - a run qualifies with at least two records, more bytes than the longest
//     token (or added-token literal), and a record starting at a
//     synchronizing transition at least 8 code points into the window and
//     before old_len, with no literal occurrence across it;
//   - the last qualifying run is kept: stored IDs up to its end, then the
//     window's IDs after it.
// Only window records that start before old_len can equal a stored one, so
// the match passes stop there; a long tail of window IDs after the splice
// (a long append) is copied by a second, grid-wide kernel.
#include "ext_internal.h"
#include "pretok_rules.h"
#include "sync_rules.h"
#include "wg_scan.h"
#include "uniclass.inc"
#include "uniclass_case.inc"

namespace tok {
namespace {

constexpr uint32_t kRpThreads = 1024;
// Window IDs after the splice up to this many are copied by the match
// kernel itself; longer tails (a long append) by a grid-wide copy.
constexpr uint32_t kInlineCopy = 8 * kRpThreads;

__device__ inline uint32_t rp_class(uint32_t cp) {
  if (cp < 0x80) return ascii_class(cp);
  if (cp < TOK_CLS_LOW) return (kClsLow[cp >> 2] >> (2 * (cp & 3u))) & 3u;
  if (cp >= 0x110000) return kO;
  const uint32_t blk = kClsBlock[cp >> 8];
  return (kClsBits[blk * 64 + ((cp & 255u) >> 2)] >> (2 * (cp & 3u))) & 3u;
}

__device__ inline uint32_t rp_case(uint32_t cp) {
  if (cp < TOK_CLS_LOW) return (kCaseLow[cp >> 1] >> (4 * (cp & 1u))) & 15u;
  if (cp >= 0x110000) return 6u;
  const uint32_t blk = kCaseBlock[cp >> 8];
  return (kCaseBits[blk * 128 + ((cp & 255u) >> 1)] >> (4 * (cp & 1u))) & 15u;
}

// Code point whose lead byte is at index i of w[0, n) (valid UTF-8 there).
__device__ inline uint32_t rp_cp(const uint8_t* w, uint64_t n, uint64_t i) {
  const uint32_t b0 = w[i];
  if (b0 < 0x80) return b0;
  const uint32_t len = b0 >= 0xF0 ? 4 : b0 >= 0xE0 ? 3 : 2;
  uint32_t cp = b0 & (0x7Fu >> len);
  for (uint32_t k = 1; k < len && i + k < n; ++k) cp = (cp << 6) | (w[i + k] & 0x3Fu);
  return cp;
}

// Bytes of an ID: a vocabulary token, or an added-token literal (A.L.n > 0;
// literal IDs name no token).  False for an ID that is neither.
__device__ inline bool id_bytes(const RepairArgs& A, int32_t id, const uint8_t** b, uint32_t* len) {
  if (id >= 0 && (uint32_t)id < A.vocab) {
    *b = A.tok_bytes + A.tok_off[id];
    *len = A.tok_len[id];
    return true;
  }
  if (id < 0 || A.L.n == 0) return false;
  uint32_t lo = 0, hi = A.L.n;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if ((uint32_t)(A.L.by_id[mid] >> 32) < (uint32_t)id) lo = mid + 1;
    else hi = mid;
  }
  if (lo == A.L.n || (uint32_t)(A.L.by_id[lo] >> 32) != (uint32_t)id) return false;
  const uint32_t li = (uint32_t)A.L.by_id[lo];
  *b = A.L.bytes + A.L.off[li];
  *len = A.L.off[li + 1] - A.L.off[li];
  return true;
}

__device__ inline uint32_t id_len(const RepairArgs& A, int32_t id) {
  const uint8_t* b = nullptr;
  uint32_t len = 0;
  return id_bytes(A, id, &b, &len) ? len : 0u;
}

// Some added-token literal occurrence, taken or not, covers bytes b - 1 and b
// (a cut there is refused: Delta Tokenizer, section 3, the cut guard).  The
// window starts at least the longest literal before any b asked about.
__device__ inline bool inside_literal(const RepairArgs& A, uint64_t b) {
  const Literals& L = A.L;
  for (uint64_t p = b - min(b - A.ws0, (uint64_t)kLitMax - 1); p < b; ++p) {
    const uint32_t b0 = A.win[p - A.ws0];
    if (!((L.first[b0 >> 5] >> (b0 & 31u)) & 1u) || p + 1 >= A.new_len) continue;
    const uint32_t e = L.key2[b0 | ((uint32_t)A.win[p + 1 - A.ws0] << 8)];
    for (uint32_t c = 0; c < (e & 0xFFFFu); ++c) {
      const uint32_t li = L.order[(e >> 16) + c];
      const uint32_t a = L.off[li], len = L.off[li + 1] - a;
      if (p + len <= b || p + len > A.new_len) continue;
      uint32_t k = 2;
      while (k < len && A.win[p + k - A.ws0] == L.bytes[a + k]) ++k;
      if (k == len) return true;
    }
  }
  return false;
}

// Stored record whose first byte is `off`, as its distance r from the
// session's end (st_off[r] falls as r grows), or -1.
__device__ inline int32_t find_stored(const uint32_t* st_off, uint32_t n_st, uint64_t off) {
  uint32_t lo = 0, hi = n_st;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (st_off[mid] > off) lo = mid + 1;
    else hi = mid;
  }
  return lo < n_st && st_off[lo] == off ? (int32_t)lo : -1;
}

__global__ void __launch_bounds__(kRpThreads) repair_match_kernel(RepairArgs A) {
  __shared__ uint32_t s_scan[kRpThreads / kWave];
  __shared__ uint32_t s_bad, s_nst, s_best, s_F;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    s_bad = 0;
    s_nst = 0xFFFFFFFFu;
    s_best = 0;
    s_F = *(volatile const uint32_t*)A.fresh_total;  // host-mapped: one read
    A.splice[2] = 0;  // the copy kernel after this one moves nothing unless a splice sets it
    // the window encode found malformed UTF-8 (or bad part offsets): its IDs
    // are no result, so nothing is matched and the session stays as it was
    const uint64_t e1 = __hip_atomic_load(A.err_utf8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t e2 = __hip_atomic_load(A.err_docs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (e1 == A.gen || e2 == A.gen) s_bad = 2;
  }
  __syncthreads();
  if (s_bad == 2) {  // uniform: read after the barrier
    if (tid == 0) {
      A.out->status = kRepairEncodeError;
      __threadfence_system();
      report(&A.out->gen, A.gen);
    }
    return;
  }
  __syncthreads();  // every lane has read s_bad before the stored-record pass may set it
  const uint32_t F = s_F;
  const uint64_t wn = A.new_len - A.ws0;  // bytes in the device window
  const uint64_t need = A.old_len - A.ws;  // stored bytes to cover

  // Fo = the window records starting before old_len (fspan rises with k;
  // records start on distinct bytes, so at most `need` of them): the
  // answer lies in [lo, hi]; each step samples the range at 1,024 evenly
  // spaced records at once and keeps the gap after the last one before
  // old_len.
  uint32_t lo = 0, hi = (uint32_t)min((uint64_t)F, need);
  while (lo < hi) {  // uniform: every thread gets the same count
    const uint32_t step = (hi - lo + kRpThreads - 1) / kRpThreads;
    const uint64_t k = lo + (uint64_t)tid * step;
    const int below = k < hi && A.ws + A.fspan[k] < A.old_len;
    const uint32_t c = (uint32_t)__syncthreads_count(below);
    if (c == 0) break;  // record lo starts at or after old_len
    const uint32_t nlo = lo + (c - 1) * step + 1;
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + (uint64_t)c * step);
    lo = nlo;
  }
  const uint32_t Fo = lo;

  // stored records, from the session's end: r-th from the end has session
  // index n_session - 1 - r and starts at old_len - (bytes of the last r + 1)
  uint32_t carry = 0;
  for (uint32_t r0 = 0;; r0 += kRpThreads) {  // uniform: s_nst and carry are shared
    const uint32_t r = r0 + tid;
    const bool have = r < A.n_session;
    const int32_t id = have ? A.session[A.n_session - 1 - r] : 0;
    const uint8_t* tb = nullptr;
    uint32_t len = 0;
    const bool id_ok = have && id_bytes(A, id, &tb, &len);
    uint32_t tot = 0;
    const uint32_t before = wg_excl_scan<kRpThreads>(len, 0u, AddOp(), s_scan, &tot);
    const uint64_t s_end = (uint64_t)carry + before;  // bytes after this record
    if (have && s_end < need) {                       // the record reaches into [ws, old_len)
      bool bad = !id_ok || s_end + len > A.old_len;
      if (!bad) {
        const uint64_t off = A.old_len - s_end - len;
        A.st_off[r] = (uint32_t)off;
        for (uint32_t k = 0; k < len && !bad; ++k) bad = tb[k] != A.win[off - A.ws0 + k];
        if (s_end + len >= need) atomicMin(&s_nst, r + 1);
      }
      if (bad) s_bad = 1u;
    }
    carry += tot;
    __syncthreads();
    const bool stop = s_bad || s_nst != 0xFFFFFFFFu || r0 + kRpThreads >= A.n_session;
    __syncthreads();  // every lane has read the shared words before the next pass may write them
    if (stop) break;
  }
  const uint32_t n_st = s_nst;
  if (s_bad || n_st == 0xFFFFFFFFu) {  // IDs that do not spell the text, or do not cover it
    if (tid == 0) {
      A.out->status = kRepairSession;
      __threadfence_system();
      report(&A.out->gen, A.gen);
    }
    return;
  }

  // equal records, runs, certificates; best = 1 + the last qualifying run end
  auto equal_at = [&](int64_t k) -> bool {
    if (k < 0 || k >= (int64_t)Fo) return false;
    const uint64_t off = A.ws + A.fspan[k];
    const int32_t r = find_stored(A.st_off, n_st, off);
    return r >= 0 && A.session[A.n_session - 1 - (uint32_t)r] == A.fresh[k];
  };
  uint32_t c_start = 0, c_cert = 0;  // 1 + index of the last run start / certified record so far
  for (uint32_t k0 = 0; k0 < Fo; k0 += kRpThreads) {
    const uint32_t k = k0 + tid;
    const bool eq = equal_at(k);
    const bool start = eq && !equal_at((int64_t)k - 1);
    const bool end = eq && !equal_at((int64_t)k + 1);
    bool cert = false;
    uint64_t off = 0;
    if (eq) {
      off = A.ws + A.fspan[k];
      if (off >= A.margin && off < A.old_len) {
        const uint64_t i = off - A.ws0;
        uint64_t j = i - 1;
        while (j > 0 && (A.win[j] & 0xC0u) == 0x80u) --j;
        const uint32_t x = rp_cp(A.win, wn, j), y = rp_cp(A.win, wn, i);
        cert = (A.pattern == 2 ? sync_transition_case(x, rp_case(x), y, rp_case(y))
                               : sync_transition_of(A.pattern == 0, x, rp_class(x), y, rp_class(y))) &&
               (A.L.n == 0 || !inside_literal(A, off));
      }
    }
    uint32_t t1 = 0, t2 = 0;
    const uint32_t ls = MaxOp()(c_start, wg_excl_scan<kRpThreads>(start ? k + 1 : 0u, 0u, MaxOp(), s_scan, &t1));
    const uint32_t lc = MaxOp()(c_cert, wg_excl_scan<kRpThreads>(cert ? k + 1 : 0u, 0u, MaxOp(), s_scan, &t2));
    if (end) {
      const uint32_t s = start ? k + 1 : ls;  // 1 + index of this run's first record
      const uint32_t c = cert ? k + 1 : lc;
      const uint32_t m = k + 2 - s;
      const uint64_t bytes = off + id_len(A, A.fresh[k]) - (A.ws + A.fspan[s - 1]);
      if (c >= s && m >= 2 && bytes > A.max_tok_len) atomicMax(&s_best, k + 1);
    }
    c_start = MaxOp()(c_start, t1);
    c_cert = MaxOp()(c_cert, t2);
  }
  __syncthreads();
  const uint32_t best = s_best;
  if (best == 0) {
    if (tid == 0) {
      A.out->status = kRepairNone;
      __threadfence_system();
      report(&A.out->gen, A.gen);
    }
    return;
  }
  const uint32_t kl = best - 1;
  const uint64_t end_off = A.ws + A.fspan[kl] + id_len(A, A.fresh[kl]);
  const int32_t r = find_stored(A.st_off, n_st, A.ws + A.fspan[kl]);
  const uint64_t keep_s = A.n_session - (uint32_t)r;  // stored IDs through the run's last record
  const uint64_t total = keep_s + (F - best);
  if (total <= A.cap && F - best <= kInlineCopy)  // a short tail: copied here
    for (uint32_t i = tid; i < F - best; i += kRpThreads) A.session[keep_s + i] = A.fresh[best + i];
  if (tid == 0) {
    if (total <= A.cap && F - best > kInlineCopy) {  // the copy kernel after this one moves them
      A.splice[0] = best;
      A.splice[1] = keep_s;
      A.splice[2] = F - best;
    }
    A.out->status = total <= A.cap ? kRepairSpliced : kRepairCapacity;
    A.out->total = total;
    A.out->kept = keep_s;
    A.out->splice = end_off;
    __threadfence_system();
    report(&A.out->gen, A.gen);
  }
}

// session[at + i] = fresh[from + i] for i < count, with (from, at, count)
// as the match kernel left them; 16 IDs per thread.
constexpr uint32_t kCopyThreads = 256, kCopyPer = 16;

__global__ void __launch_bounds__(kCopyThreads) repair_copy_kernel(const int32_t* fresh, int32_t* session,
                                                                   const uint64_t* splice) {
  const uint64_t from = splice[0], at = splice[1], count = splice[2];
  const uint64_t base = (uint64_t)blockIdx.x * kCopyThreads * kCopyPer;
  if (base >= count) return;
  const uint64_t end = min(count, base + (uint64_t)kCopyThreads * kCopyPer);
  for (uint64_t i = base + threadIdx.x; i < end; i += kCopyThreads) session[at + i] = fresh[from + i];
}

}  // namespace

void launch_repair_match(const RepairArgs& a, hipStream_t s) {
  repair_match_kernel<<<1, kRpThreads, 0, s>>>(a);
  const uint64_t per = (uint64_t)kCopyThreads * kCopyPer;
  const uint32_t grid = (uint32_t)((a.max_fresh + per - 1) / per);
  if (a.max_fresh > kInlineCopy) repair_copy_kernel<<<grid, kCopyThreads, 0, s>>>(a.fresh, a.session, a.splice);
}

}  // namespace tok
