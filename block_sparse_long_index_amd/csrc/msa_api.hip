// msa_api.hip -- the C ABI declared in include/msa.h: host-side validation,
// workspace sizing and the launches.  No device memory is allocated here.
#include "msa.h"
#include "msa_internal.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kDefaultWindow = int64_t(1) << 20;  // rows per inversion (one sequence)
constexpr int64_t kMaxElems = int64_t(1) << 46;

bool pow2_upto(int v, int hi) { return v >= 1 && v <= hi && (v & (v - 1)) == 0; }

int check_dims(const msa_dims_t* d) {
  if (!d) return fail(MSA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->B < 1 || d->T < 1 || d->N < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "B, T, N must be >= 1 (B=%lld T=%lld N=%lld)",
                (long long)d->B, (long long)d->T, (long long)d->N);
  if (d->T > d->N)
    return fail(MSA_ERR_INVALID_ARGUMENT, "T (%lld) exceeds N (%lld)", (long long)d->T,
                (long long)d->N);
  if (d->Hq < 1 || d->G < 1 || d->Hq % d->G != 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "Hq (%d) must be a positive multiple of G (%d)",
                d->Hq, d->G);
  if (d->k < 1 || d->Bk < 1 || d->d_h < 1 || d->d_I < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k, Bk, d_h, d_I must be >= 1");
  if (d->d_h != 128 || d->d_I != 128)
    return fail(MSA_ERR_UNSUPPORTED, "only d_h = d_I = 128 (got %d, %d)", d->d_h, d->d_I);
  if (d->Bk != 128 && d->Bk != 64 && d->Bk != 32)
    return fail(MSA_ERR_UNSUPPORTED, "Bk must be 32, 64 or 128 (got %d)", d->Bk);
  // at most 2048 selected keys per query and group: k <= 16 / 32 / 64
  if (d->k > 2048 / d->Bk)
    return fail(MSA_ERR_UNSUPPORTED, "k * Bk > 2048 (k = %d, Bk = %d)", d->k, d->Bk);
  if (!pow2_upto(d->G, 16)) return fail(MSA_ERR_UNSUPPORTED, "G must be 1, 2, 4, 8 or 16");
  if (!pow2_upto(d->Hq / d->G, 16))
    return fail(MSA_ERR_UNSUPPORTED, "Hq / G must be 1, 2, 4, 8 or 16");
  if (d->B > 65535) return fail(MSA_ERR_UNSUPPORTED, "B > 65535");
  // block counts of one sequence live in LDS during the inversion (64 KB)
  if (d->N > (int64_t(1) << 21)) return fail(MSA_ERR_UNSUPPORTED, "N > 2^21");
  if ((d->N + d->Bk - 1) / d->Bk > 16384)
    return fail(MSA_ERR_UNSUPPORTED, "more than 16384 blocks per sequence");
  const int64_t NB = (d->N + d->Bk - 1) / d->Bk;
  if (d->B * d->T * d->Hq > kMaxElems / 128 || d->B * d->G * d->N > kMaxElems / 128 ||
      d->B * d->G * d->T * NB > kMaxElems || d->B * d->G * NB > (int64_t(1) << 30))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large");
  return MSA_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(MSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15)
    return fail(MSA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return MSA_OK;
}

const msa::PagedCache kContiguous = {nullptr, nullptr, 0, 0};

// The page table and lengths of a paged call (device arrays; their contents
// are the caller's, see msa.h).
int check_paged(const msa_dims_t* d, int64_t num_pages, const int32_t* table,
                const int64_t* lens, msa::PagedCache* pc) {
  if (d->Bk != 128)
    return fail(MSA_ERR_UNSUPPORTED, "paged caches have 128-token pages (Bk = %d)", d->Bk);
  if (d->T != 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "paged calls are decode only (T == 1, got %lld)",
                (long long)d->T);
  if (num_pages < 1 || num_pages > (int64_t(1) << 31))
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages %lld out of range", (long long)num_pages);
  if (!table || (reinterpret_cast<uintptr_t>(table) & 3))
    return fail(MSA_ERR_INVALID_ARGUMENT, "block_table is NULL or not 4-byte aligned");
  if (!lens || (reinterpret_cast<uintptr_t>(lens) & 7))
    return fail(MSA_ERR_INVALID_ARGUMENT, "seq_lens is NULL or not 8-byte aligned");
  pc->table = table;
  pc->lens = lens;
  pc->pages = num_pages;
  pc->nb = static_cast<int32_t>((d->N + d->Bk - 1) / d->Bk);
  return MSA_OK;
}

#define MSA_TRY(x)               \
  do {                           \
    const int rc_ = (x);         \
    if (rc_ != MSA_OK) return rc_; \
  } while (0)

int64_t nblocks(const msa_dims_t* d) { return (d->N + d->Bk - 1) / d->Bk; }

// Calls whose kernels only take 128-key blocks (the fused selection on fp8
// inputs, paged caches).
int need_bk128(const msa_dims_t* d, const char* what) {
  if (d->Bk != 128) return fail(MSA_ERR_UNSUPPORTED, "%s needs Bk = 128 (got %d)", what, d->Bk);
  return MSA_OK;
}

// Prefill selection with Bk < 128: the scores of a window of rows are
// materialised, then ranked.  Rows per window for a workspace of ws bytes.
int64_t select_window(const msa_dims_t* d, size_t ws) {
  const int64_t per_row = d->B * d->G * nblocks(d) * int64_t(sizeof(float));
  const int64_t w = static_cast<int64_t>(ws) / per_row;
  return w < d->T ? w : d->T;
}

// Default: windows of up to 1 GB of scores.
size_t select_window_ws(const msa_dims_t* d) {
  const int64_t per_row = d->B * d->G * nblocks(d) * int64_t(sizeof(float));
  int64_t w = (int64_t(1) << 30) / per_row;
  if (w < 1) w = 1;
  if (w > d->T) w = d->T;
  return static_cast<size_t>(w * per_row);
}

size_t decode_select_ws(const msa_dims_t* d) {
  return static_cast<size_t>(d->B * d->G * nblocks(d)) * sizeof(float);
}

int64_t default_window(const msa_dims_t* d) {
  return d->T < kDefaultWindow ? d->T : kDefaultWindow;
}

// Rows per attention stage: the largest power of two >= 1024 whose partials
// fit a byte budget.  A bigger stage gathers more queries per KV block (fewer
// block loads and fewer partly filled chunks) but writes more partials before
// they are read back; 512 MB is best at 128K tokens, and from 4096 blocks on,
// where a stage's queries are spread over many more blocks, 1 GB is.
int64_t stage_rows_for(const msa_dims_t* d, int64_t window) {
  const int64_t per_row = int64_t(d->k) * (d->Hq / d->G) * 256;
  const int64_t budget = nblocks(d) >= 4096 ? int64_t(1) << 30 : int64_t(1) << 29;
  int64_t rows = 1024;
  while (rows * 2 * per_row <= budget) rows *= 2;
  return window < rows ? window : rows;
}

size_t prefill_ws(const msa_dims_t* d, int64_t window) {
  return msa::attn_workspace_bytes(window, stage_rows_for(d, window), d->N, d->G, d->Hq / d->G,
                                   d->k, d->Bk, false);
}

// Backward: the prefill's inversion and partial buffers (the dq partials take
// the place of the partial O), then D = dO . O for every (row, head).
size_t rowdot_bytes(const msa_dims_t* d) {
  return ((static_cast<size_t>(d->B * d->T * d->Hq) * sizeof(float)) + 255) & ~size_t(255);
}

size_t backward_ws(const msa_dims_t* d, int64_t window) {
  return rowdot_bytes(d) + prefill_ws(d, window);
}

// Index-branch KL backward: the proxy lse of every (row, group), one stage's
// teacher (fp32 per (row, slot, key)), then the prefill's inversion and
// partial buffers.
size_t lpx_bytes(const msa_dims_t* d) {
  return ((static_cast<size_t>(d->B * d->T * d->G) * sizeof(float)) + 255) & ~size_t(255);
}

size_t teach_bytes(const msa_dims_t* d, int64_t window) {
  return ((static_cast<size_t>(stage_rows_for(d, window) * d->k * d->Bk) * sizeof(float)) + 255) &
         ~size_t(255);
}

size_t index_kl_ws(const msa_dims_t* d, int64_t window) {
  return lpx_bytes(d) + teach_bytes(d, window) + prefill_ws(d, window);
}

// Fused training backward: D = dO . O, the proxy lse, one stage's teacher,
// then the prefill's inversion and partials.

size_t train_ws(const msa_dims_t* d, int64_t window) {
  return rowdot_bytes(d) + lpx_bytes(d) + teach_bytes(d, window) + prefill_ws(d, window);
}

// The one-call prefill (msa_prefill): windows of about T / 4 query rows, at
// least 16384 (smaller windows fill the attention's chunks too thinly to
// gain from the overlap), a multiple of 4096, at most 64 windows; the
// selection of a window overlaps the attention of the one before.  When that
// makes fewer than four windows the whole prefill is one window: the overlap
// does not pay there, and the windows' smaller launches cost more than one
// selection and one attention over all rows (32K rows: 6.33 ms in three
// windows in order, 5.62 ms as one).
constexpr int kMaxPipeWindows = 64;

#ifndef MSA_PIPE_SPLIT
#define MSA_PIPE_SPLIT 4
#endif
int64_t pipe_window(const msa_dims_t* d) {
  int64_t w = (d->T + MSA_PIPE_SPLIT - 1) / MSA_PIPE_SPLIT;
  if (w < 16384) w = 16384;
  w = ((w + 4095) / 4096) * 4096;
  if ((d->T + w - 1) / w > kMaxPipeWindows) w = (d->T + kMaxPipeWindows - 1) / kMaxPipeWindows;
  if (w >= d->T) return d->T;
  int64_t bounds[msa::kMaxPrefillWindows + 1];
  if (msa::prefill_windows(d->T, w, bounds, msa::kMaxPrefillWindows) < 4) return d->T;
  return w;
}

// Rows of block scores the one-call prefill materialises at a time (Bk < 128).
int64_t pipe_score_rows(const msa_dims_t* d) {
  const int64_t per_row = d->B * d->G * nblocks(d) * int64_t(sizeof(float));
  int64_t r = (int64_t(1) << 30) / per_row;
  if (r < 1) r = 1;
  const int64_t w = pipe_window(d);
  return r < w ? r : w;
}

size_t pipe_score_bytes(const msa_dims_t* d) {
  if (d->Bk == 128) return 0;
  const size_t b = static_cast<size_t>(pipe_score_rows(d) * d->B * d->G * nblocks(d)) * 4;
  return (b + 255) & ~size_t(255);
}

// Workspace of the one-call prefill: the selection's item counters (one per
// window), the score rows (Bk < 128), then the attention's.
constexpr size_t kPipeCounterBytes = 512;
static_assert(kPipeCounterBytes >= sizeof(int32_t) * msa::kMaxPrefillWindows, "counters");

size_t pipe_ws(const msa_dims_t* d) {
  return kPipeCounterBytes + pipe_score_bytes(d) + prefill_ws(d, pipe_window(d));
}

size_t decode_ws(const msa_dims_t* d) {
  return msa::attn_workspace_bytes(d->B, d->B, d->N, d->G, d->Hq / d->G, d->k, d->Bk, true);
}

// One-call decode (msa_decode): the block scores of the scan, then either the
// fused step (one workgroup per (sequence, group): selection, attention and
// merge) or, for batches of fewer rows than that needs to fill the chip, the
// separate top-k, attention and combine launches (whose partials follow the
// scores in the workspace).
#ifndef MSA_STEP_MIN_ROWS
#define MSA_STEP_MIN_ROWS 128
#endif
constexpr int64_t kStepMinRows = MSA_STEP_MIN_ROWS;

size_t decode_scores_bytes(const msa_dims_t* d) {
  return (decode_select_ws(d) + 255) & ~size_t(255);
}

size_t decode1_ws(const msa_dims_t* d) {
  return decode_scores_bytes(d) + (d->B * d->G >= kStepMinRows
                                       ? msa::decode_step_scratch_bytes(d->B, d->G, d->Hq)
                                       : decode_ws(d));
}

}  // namespace

extern "C" {

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MSA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_err; }

int msa_timing_begin(int64_t max_launches) {
  if (max_launches < 1 || max_launches > (int64_t(1) << 20))
    return fail(MSA_ERR_INVALID_ARGUMENT, "max_launches %lld outside [1, 2^20]",
                (long long)max_launches);
  if (msa::timing_enabled())
    return fail(MSA_ERR_INVALID_ARGUMENT, "a timing session is already open");
  const hipError_t e = msa::timing_start(max_launches);
  return e == hipSuccess ? MSA_OK : hip_fail(e, "msa_timing_begin");
}

int msa_timing_end(double* total_ms, int64_t* launches, int nkinds) {
  if (!total_ms || !launches || nkinds < 1 || nkinds > MSA_KERNEL_KINDS)
    return fail(MSA_ERR_INVALID_ARGUMENT, "total_ms, launches NULL or nkinds %d outside [1, %d]",
                nkinds, MSA_KERNEL_KINDS);
  if (!msa::timing_enabled()) return fail(MSA_ERR_INVALID_ARGUMENT, "no timing session is open");
  int64_t dropped = 0;
  const hipError_t e = msa::timing_stop(total_ms, launches, nkinds, &dropped);
  if (e != hipSuccess) return hip_fail(e, "msa_timing_end");
  if (dropped > 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "%lld launches were not timed (max_launches too small)",
                (long long)dropped);
  return MSA_OK;
}

size_t msa_workspace_bytes(int op, const msa_dims_t* d) {
  char saved[sizeof g_err];
  memcpy(saved, g_err, sizeof g_err);
  const int rc = check_dims(d);
  memcpy(g_err, saved, sizeof g_err);
  if (rc != MSA_OK) return 0;
  switch (op) {
    case MSA_OP_INDEX_SCORES: return 0;
    case MSA_OP_SELECT_BLOCKS:
      return d->T == 1 ? decode_select_ws(d) : (d->Bk == 128 ? 0 : select_window_ws(d));
    case MSA_OP_SELECT_FROM_SCORES: return 0;
    case MSA_OP_ATTN_PREFILL: return prefill_ws(d, default_window(d));
    case MSA_OP_ATTN_DECODE: return d->T == 1 ? decode_ws(d) : 0;
    case MSA_OP_ATTN_BACKWARD: return backward_ws(d, default_window(d));
    case MSA_OP_INDEX_KL_BACKWARD: return index_kl_ws(d, default_window(d));
    case MSA_OP_TRAIN_BACKWARD: return train_ws(d, default_window(d));
    case MSA_OP_PREFILL: return d->T > 1 ? pipe_ws(d) : 0;
    case MSA_OP_DECODE: return d->T == 1 ? decode1_ws(d) : 0;
  }
  return 0;
}

static int index_scores_impl(const msa_dims_t* d, const void* qI, const void* kI, float* S,
                             void* stream, bool fp8, const char* name) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(S, "S"));
  if (fp8) MSA_TRY(need_bk128(d, name));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d->T == 1)
    e = msa::launch_decode_scan(fp8, qI, kI, S, d->B, d->N, d->G, d->Bk, kContiguous, st);
  else
    e = msa::launch_index_tiles(true, fp8, qI, kI, S, nullptr, d->B, d->T, 0, d->T, d->N, d->G,
                                d->Bk, d->k, st);
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

static int select_blocks_impl(const msa_dims_t* d, const void* qI, const void* kI, int32_t* idx,
                              void* ws, size_t ws_bytes, void* stream, bool fp8,
                              const char* name) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(idx, "idx"));
  if (fp8) MSA_TRY(need_bk128(d, name));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d->T == 1) {
    const size_t need = decode_select_ws(d);
    MSA_TRY(check_ptr(ws, "ws"));
    if (ws_bytes < need)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "select needs %zu workspace bytes, got %zu",
                  need, ws_bytes);
    float* S = static_cast<float*>(ws);
    e = msa::launch_decode_scan(fp8, qI, kI, S, d->B, d->N, d->G, d->Bk, kContiguous, st);
    if (e == hipSuccess)
      e = msa::launch_topk_rows(S, idx, d->B, 1, 0, 1, d->N, d->G, d->Bk, d->k, kContiguous, st);
  } else if (d->Bk == 128) {
    e = msa::launch_index_tiles(false, fp8, qI, kI, nullptr, idx, d->B, d->T, 0, d->T, d->N,
                                d->G, 128, d->k, st);
  } else {
    // the scores of a window of rows at a time, then their top-k
    MSA_TRY(check_ptr(ws, "ws"));
    const int64_t W = select_window(d, ws_bytes);
    if (W < 1)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                  "select needs at least %lld workspace bytes (one row of scores), got %zu",
                  (long long)(d->B * d->G * nblocks(d) * 4), ws_bytes);
    float* S = static_cast<float*>(ws);
    e = hipSuccess;
    for (int64_t t0 = 0; t0 < d->T && e == hipSuccess; t0 += W) {
      const int64_t Tw = d->T - t0 < W ? d->T - t0 : W;
      e = msa::launch_index_tiles(true, false, qI, kI, S, nullptr, d->B, d->T, t0, Tw, d->N,
                                  d->G, d->Bk, d->k, st);
      if (e == hipSuccess)
        e = msa::launch_topk_rows(S, idx, d->B, d->T, t0, Tw, d->N, d->G, d->Bk, d->k,
                                  kContiguous, st);
    }
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

int msa_index_scores(const msa_dims_t* d, const void* qI, const void* kI, float* S,
                     void* stream) {
  return index_scores_impl(d, qI, kI, S, stream, false, "msa_index_scores");
}

int msa_index_scores_fp8(const msa_dims_t* d, const void* qI, const void* kI, float* S,
                         void* stream) {
  return index_scores_impl(d, qI, kI, S, stream, true, "msa_index_scores_fp8");
}

int msa_select_blocks(const msa_dims_t* d, const void* qI, const void* kI, int32_t* idx,
                      void* ws, size_t ws_bytes, void* stream) {
  return select_blocks_impl(d, qI, kI, idx, ws, ws_bytes, stream, false, "msa_select_blocks");
}

int msa_select_blocks_fp8(const msa_dims_t* d, const void* qI, const void* kI, int32_t* idx,
                          void* ws, size_t ws_bytes, void* stream) {
  return select_blocks_impl(d, qI, kI, idx, ws, ws_bytes, stream, true,
                            "msa_select_blocks_fp8");
}

int msa_select_blocks_from_scores(const msa_dims_t* d, const float* S, int32_t* idx,
                                  void* stream) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(S, "S"));
  MSA_TRY(check_ptr(idx, "idx"));
  const hipError_t e = msa::launch_topk_rows(S, idx, d->B, d->T, 0, d->T, d->N, d->G, d->Bk,
                                             d->k, kContiguous,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_select_blocks_from_scores");
  return MSA_OK;
}

int msa_sparse_attn_prefill(const msa_dims_t* d, const void* q, const void* K, const void* V,
                            const int32_t* idx, void* O, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(ws, "ws"));
  // Largest window (query rows per pass) whose workspace fits.
  int64_t hi = default_window(d);
  if (prefill_ws(d, 1) > ws_bytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "prefill needs at least %zu workspace bytes (%zu for the default window), got %zu",
                prefill_ws(d, 1), prefill_ws(d, hi), ws_bytes);
  if (prefill_ws(d, hi) > ws_bytes) {
    int64_t lo = 1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (prefill_ws(d, mid) <= ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    hi = lo;
  }
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(ws, hi, stage_rows_for(d, hi), d->N, d->G, d->Hq / d->G, d->k, d->Bk,
                            false, &w);
  const hipError_t e = msa::launch_attn_prefill(q, K, V, idx, O, lse, d->B, d->T, d->N, d->Hq,
                                                d->G, d->k, d->Bk, w,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_prefill");
  return MSA_OK;
}

}  // extern "C"

namespace {

// Events of the one-call prefill's stream hand-offs: a pool per thread and
// device, created on first use and reused by every later call of that thread
// (a call enqueues all its records and waits before it returns, so a later
// call's records cannot be confused with them).
constexpr int kPoolDevices = 64;
constexpr int kPoolEvents = kMaxPipeWindows + 2;  // windows (the last one may be cut) + 1
struct EventPool {
  bool ready;
  hipEvent_t ev[kPoolEvents];
};
thread_local EventPool t_events[kPoolDevices];

int pipe_events(hipEvent_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "msa_prefill: hipGetDevice");
  if (dev < 0 || dev >= kPoolDevices)
    return fail(MSA_ERR_UNSUPPORTED, "msa_prefill: device %d >= %d", dev, kPoolDevices);
  EventPool& p = t_events[dev];
  if (!p.ready) {
    for (int i = 0; i < kPoolEvents; ++i) {
      e = hipEventCreateWithFlags(&p.ev[i], hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "msa_prefill: hipEventCreateWithFlags");
    }
    p.ready = true;
  }
  *out = p.ev;
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_prefill(const msa_dims_t* d, const void* qI, const void* kI, const void* q,
                const void* K, const void* V, int32_t* idx, void* O, float* lse, void* ws,
                size_t ws_bytes, void* stream, void* stream2) {
  MSA_TRY(check_dims(d));
  if (d->T < 2)
    return fail(MSA_ERR_INVALID_ARGUMENT,
                "msa_prefill needs T >= 2 (got %lld); one row is a decode step",
                (long long)d->T);
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(ws, "ws"));
  const size_t need = pipe_ws(d);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_prefill needs %zu workspace bytes, got %zu",
                need, ws_bytes);
  const int64_t win = pipe_window(d);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStream_t st2 = stream2 ? static_cast<hipStream_t>(stream2) : st;
  hipEvent_t* ev = nullptr;
  if (st2 != st) MSA_TRY(pipe_events(&ev));
  char* p = static_cast<char*>(ws);
  int32_t* counters = reinterpret_cast<int32_t*>(p);
  float* S = d->Bk == 128 ? nullptr : reinterpret_cast<float*>(p + kPipeCounterBytes);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(p + kPipeCounterBytes + pipe_score_bytes(d), win,
                            stage_rows_for(d, win), d->N, d->G, d->Hq / d->G, d->k, d->Bk, false,
                            &w);
  const hipError_t e = msa::launch_prefill_pipelined(
      qI, kI, q, K, V, idx, O, lse, d->B, d->T, d->N, d->Hq, d->G, d->k, d->Bk, win, S,
      pipe_score_rows(d), counters, w, st, st2, ev, kPoolEvents);
  if (e != hipSuccess) return hip_fail(e, "msa_prefill");
  return MSA_OK;
}

int msa_sparse_attn_backward(const msa_dims_t* d, const void* q, const void* K, const void* V,
                             const int32_t* idx, const void* O, const float* lse, const void* dO,
                             float* dq, float* dK, float* dV, void* ws, size_t ws_bytes,
                             void* stream) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(dO, "dO"));
  MSA_TRY(check_ptr(dq, "dq"));
  MSA_TRY(check_ptr(dK, "dK"));
  MSA_TRY(check_ptr(dV, "dV"));
  MSA_TRY(check_ptr(ws, "ws"));
  int64_t hi = default_window(d);
  if (backward_ws(d, 1) > ws_bytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "backward needs at least %zu workspace bytes (%zu for the default window), got %zu",
                backward_ws(d, 1), backward_ws(d, hi), ws_bytes);
  if (backward_ws(d, hi) > ws_bytes) {
    int64_t lo = 1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (backward_ws(d, mid) <= ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    hi = lo;
  }
  float* Dr = static_cast<float*>(ws);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(static_cast<char*>(ws) + rowdot_bytes(d), hi, stage_rows_for(d, hi),
                            d->N, d->G, d->Hq / d->G, d->k, d->Bk, false, &w);
  const hipError_t e = msa::launch_attn_backward(q, K, V, idx, O, lse, dO, dq, dK, dV, Dr, d->B,
                                                 d->T, d->N, d->Hq, d->G, d->k, d->Bk, w,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_backward");
  return MSA_OK;
}

int msa_index_kl_backward(const msa_dims_t* d, const void* qI, const void* kI, const void* q,
                          const void* K, const int32_t* idx, const float* lse, float* dqI,
                          float* dkI, float* kl, void* ws, size_t ws_bytes, void* stream) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(dqI, "dqI"));
  MSA_TRY(check_ptr(dkI, "dkI"));
  if (kl) MSA_TRY(check_ptr(kl, "kl"));
  MSA_TRY(check_ptr(ws, "ws"));
  int64_t hi = default_window(d);
  if (index_kl_ws(d, 1) > ws_bytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "index KL backward needs at least %zu workspace bytes (%zu for the default "
                "window), got %zu",
                index_kl_ws(d, 1), index_kl_ws(d, hi), ws_bytes);
  if (index_kl_ws(d, hi) > ws_bytes) {
    int64_t lo = 1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (index_kl_ws(d, mid) <= ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    hi = lo;
  }
  char* p = static_cast<char*>(ws);
  float* lpx = reinterpret_cast<float*>(p);
  p += lpx_bytes(d);
  float* teach = reinterpret_cast<float*>(p);
  p += teach_bytes(d, hi);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(p, hi, stage_rows_for(d, hi), d->N, d->G, d->Hq / d->G, d->k, d->Bk,
                            false, &w);
  const hipError_t e = msa::launch_index_kl_backward(
      qI, kI, q, K, idx, lse, dqI, dkI, kl, lpx, teach, d->B, d->T, d->N, d->Hq, d->G, d->k,
      d->Bk, w, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_index_kl_backward");
  return MSA_OK;
}

int msa_train_backward(const msa_dims_t* d, const void* q, const void* K, const void* V,
                       const void* qI, const void* kI, const int32_t* idx, const void* O,
                       const float* lse, const void* dO, float* dq, float* dK, float* dV,
                       float* dqI, float* dkI, float* kl, void* ws, size_t ws_bytes,
                       void* stream) {
  MSA_TRY(check_dims(d));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(dO, "dO"));
  MSA_TRY(check_ptr(dq, "dq"));
  MSA_TRY(check_ptr(dK, "dK"));
  MSA_TRY(check_ptr(dV, "dV"));
  MSA_TRY(check_ptr(dqI, "dqI"));
  MSA_TRY(check_ptr(dkI, "dkI"));
  if (kl) MSA_TRY(check_ptr(kl, "kl"));
  MSA_TRY(check_ptr(ws, "ws"));
  int64_t hi = default_window(d);
  if (train_ws(d, 1) > ws_bytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "training backward needs at least %zu workspace bytes (%zu for the default "
                "window), got %zu",
                train_ws(d, 1), train_ws(d, hi), ws_bytes);
  if (train_ws(d, hi) > ws_bytes) {
    int64_t lo = 1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (train_ws(d, mid) <= ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    hi = lo;
  }
  char* p = static_cast<char*>(ws);
  float* Dr = reinterpret_cast<float*>(p);
  p += rowdot_bytes(d);
  float* lpx = reinterpret_cast<float*>(p);
  p += lpx_bytes(d);
  float* teach = reinterpret_cast<float*>(p);
  p += teach_bytes(d, hi);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(p, hi, stage_rows_for(d, hi), d->N, d->G, d->Hq / d->G, d->k, d->Bk,
                            false, &w);
  const hipError_t e = msa::launch_train_backward(
      q, K, V, qI, kI, idx, O, lse, dO, dq, dK, dV, dqI, dkI, kl, Dr, lpx, teach, d->B, d->T,
      d->N, d->Hq, d->G, d->k, d->Bk, w, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_train_backward");
  return MSA_OK;
}

int msa_sparse_attn_decode(const msa_dims_t* d, const void* q, const void* K, const void* V,
                           const int32_t* idx, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  MSA_TRY(check_dims(d));
  if (d->T != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "decode needs T == 1 (got %lld)",
                             (long long)d->T);
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(ws, "ws"));
  const size_t need = decode_ws(d);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(ws, d->B, d->B, d->N, d->G, d->Hq / d->G, d->k, d->Bk, true, &w);
  const hipError_t e = msa::launch_attn_decode(q, K, V, idx, O, lse, d->B, d->N, d->Hq, d->G,
                                               d->k, d->Bk, kContiguous, w,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_decode");
  return MSA_OK;
}

}  // extern "C"

// The one-call decode over contiguous caches (pc == kContiguous) or paged
// pools (pc from check_paged): the scan, then the per-row step kernel or,
// for small batches, the separate top-k, attention and combine launches.
static int decode_impl(const msa_dims_t* d, const void* qI, const void* kI, const void* q,
                       const void* K, const void* V, int32_t* idx, void* O, float* lse, void* ws,
                       size_t ws_bytes, void* stream, bool fp8, const msa::PagedCache& pc,
                       const char* name) {
  MSA_TRY(check_dims(d));
  if (d->T != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "%s needs T == 1 (got %lld)", name,
                             (long long)d->T);
  if (fp8) MSA_TRY(need_bk128(d, name));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI, "kI"));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(ws, "ws"));
  const size_t need = decode1_ws(d);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "%s needs %zu workspace bytes, got %zu", name, need,
                ws_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* S = static_cast<float*>(ws);
  hipError_t e = msa::launch_decode_scan(fp8, qI, kI, S, d->B, d->N, d->G, d->Bk, pc,
                                         st);
  if (e == hipSuccess) {
    if (d->B * d->G >= kStepMinRows) {
      e = msa::launch_decode_step(S, q, K, V, idx, O, lse,
                                  static_cast<unsigned char*>(ws) + decode_scores_bytes(d), d->B,
                                  d->N, d->Hq, d->G, d->k, d->Bk, pc, st);
    } else {
      e = msa::launch_topk_rows(S, idx, d->B, 1, 0, 1, d->N, d->G, d->Bk, d->k, pc, st);
      if (e == hipSuccess) {
        msa::AttnWorkspace w;
        msa::attn_workspace_carve(static_cast<unsigned char*>(ws) + decode_scores_bytes(d), d->B,
                                  d->B, d->N, d->G, d->Hq / d->G, d->k, d->Bk, true, &w);
        e = msa::launch_attn_decode(q, K, V, idx, O, lse, d->B, d->N, d->Hq, d->G, d->k, d->Bk,
                                    pc, w, st);
      }
    }
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

extern "C" {

int msa_decode(const msa_dims_t* d, const void* qI, const void* kI, const void* q, const void* K,
               const void* V, int32_t* idx, void* O, float* lse, void* ws, size_t ws_bytes,
               void* stream) {
  return decode_impl(d, qI, kI, q, K, V, idx, O, lse, ws, ws_bytes, stream, false, kContiguous,
                     "msa_decode");
}

int msa_decode_fp8(const msa_dims_t* d, const void* qI, const void* kI, const void* q,
                   const void* K, const void* V, int32_t* idx, void* O, float* lse, void* ws,
                   size_t ws_bytes, void* stream) {
  return decode_impl(d, qI, kI, q, K, V, idx, O, lse, ws, ws_bytes, stream, true, kContiguous,
                     "msa_decode_fp8");
}

static int decode_paged(const msa_dims_t* d, const void* qI, const void* kI_pool, const void* q,
                        const void* K_pool, const void* V_pool, int64_t num_pages,
                        const int32_t* block_table, const int64_t* seq_lens, int32_t* idx,
                        void* O, float* lse, void* ws, size_t ws_bytes, void* stream, bool fp8,
                        const char* name) {
  MSA_TRY(check_dims(d));
  msa::PagedCache pc;
  MSA_TRY(check_paged(d, num_pages, block_table, seq_lens, &pc));
  return decode_impl(d, qI, kI_pool, q, K_pool, V_pool, idx, O, lse, ws, ws_bytes, stream, fp8,
                     pc, name);
}

int msa_decode_paged(const msa_dims_t* d, const void* qI, const void* kI_pool, const void* q,
                     const void* K_pool, const void* V_pool, int64_t num_pages,
                     const int32_t* block_table, const int64_t* seq_lens, int32_t* idx, void* O,
                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_paged(d, qI, kI_pool, q, K_pool, V_pool, num_pages, block_table, seq_lens, idx,
                      O, lse, ws, ws_bytes, stream, false, "msa_decode_paged");
}

int msa_decode_paged_fp8(const msa_dims_t* d, const void* qI, const void* kI_pool,
                         const void* q, const void* K_pool, const void* V_pool,
                         int64_t num_pages, const int32_t* block_table,
                         const int64_t* seq_lens, int32_t* idx, void* O, float* lse, void* ws,
                         size_t ws_bytes, void* stream) {
  return decode_paged(d, qI, kI_pool, q, K_pool, V_pool, num_pages, block_table, seq_lens, idx,
                      O, lse, ws, ws_bytes, stream, true, "msa_decode_paged_fp8");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode attention for callers that cannot allocate device memory: the
// partial results of the selected blocks (bf16 O, fp32 (max, sum)) live in a
// device array of this file instead of a caller workspace.  Each GPU holds its
// own copy for the life of the process; its device address is looked up once
// per device and kept.  The decode kernels write every partial they read, so
// nothing needs clearing between calls.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kScratchRows = 32768;  // partial rows: B * Hq * k
constexpr size_t kScratchOpart = static_cast<size_t>(kScratchRows) * 128 * sizeof(uint16_t);
constexpr size_t kScratchBytes = kScratchOpart + static_cast<size_t>(kScratchRows) * 8;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The current device's copy of the scratch array (its device address).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attn_decode_noalloc: device %d >= %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "msa_sparse_attn_decode_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_sparse_attn_decode_noalloc(const msa_dims_t* d, const void* q, const void* K,
                                   const void* V, const int32_t* idx, void* O, float* lse,
                                   void* stream) {
  MSA_TRY(check_dims(d));
  if (d->T != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "decode needs T == 1 (got %lld)",
                             (long long)d->T);
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K, "K"));
  MSA_TRY(check_ptr(V, "V"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  const int64_t rows = d->B * d->Hq * d->k;
  if (rows > kScratchRows)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_decode_noalloc: B * Hq * k = %lld partial rows exceed the "
                "static scratch (%lld rows)", (long long)rows, (long long)kScratchRows);
  void* base = nullptr;
  MSA_TRY(scratch_ptr(&base));
  msa::AttnWorkspace w = {};
  w.opart = static_cast<uint16_t*>(base);
  w.lpart = reinterpret_cast<float2*>(static_cast<char*>(base) + kScratchOpart);
  w.window = d->B;
  w.stage_rows = d->B;
  const hipError_t e = msa::launch_attn_decode(q, K, V, idx, O, lse, d->B, d->N, d->Hq, d->G,
                                               d->k, d->Bk, kContiguous, w,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_decode_noalloc");
  return MSA_OK;
}

static int select_paged_impl(const msa_dims_t* d, const void* qI, const void* kI_pool,
                             int64_t num_pages, const int32_t* block_table,
                             const int64_t* seq_lens, int32_t* idx, void* ws, size_t ws_bytes,
                             void* stream, bool fp8, const char* name) {
  MSA_TRY(check_dims(d));
  msa::PagedCache pc;
  MSA_TRY(check_paged(d, num_pages, block_table, seq_lens, &pc));
  MSA_TRY(check_ptr(qI, "qI"));
  MSA_TRY(check_ptr(kI_pool, "kI_pool"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(ws, "ws"));
  const size_t need = decode_select_ws(d);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "select needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* S = static_cast<float*>(ws);
  hipError_t e = msa::launch_decode_scan(fp8, qI, kI_pool, S, d->B, d->N, d->G, 128, pc, st);
  if (e == hipSuccess)
    e = msa::launch_topk_rows(S, idx, d->B, 1, 0, 1, d->N, d->G, 128, d->k, pc, st);
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

int msa_select_blocks_paged(const msa_dims_t* d, const void* qI, const void* kI_pool,
                            int64_t num_pages, const int32_t* block_table,
                            const int64_t* seq_lens, int32_t* idx, void* ws, size_t ws_bytes,
                            void* stream) {
  return select_paged_impl(d, qI, kI_pool, num_pages, block_table, seq_lens, idx, ws, ws_bytes,
                           stream, false, "msa_select_blocks_paged");
}

int msa_select_blocks_paged_fp8(const msa_dims_t* d, const void* qI, const void* kI_pool,
                                int64_t num_pages, const int32_t* block_table,
                                const int64_t* seq_lens, int32_t* idx, void* ws,
                                size_t ws_bytes, void* stream) {
  return select_paged_impl(d, qI, kI_pool, num_pages, block_table, seq_lens, idx, ws, ws_bytes,
                           stream, true, "msa_select_blocks_paged_fp8");
}

int msa_sparse_attn_decode_paged(const msa_dims_t* d, const void* q, const void* K_pool,
                                 const void* V_pool, int64_t num_pages,
                                 const int32_t* block_table, const int64_t* seq_lens,
                                 const int32_t* idx, void* O, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  MSA_TRY(check_dims(d));
  msa::PagedCache pc;
  MSA_TRY(check_paged(d, num_pages, block_table, seq_lens, &pc));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(K_pool, "K_pool"));
  MSA_TRY(check_ptr(V_pool, "V_pool"));
  MSA_TRY(check_ptr(idx, "idx"));
  MSA_TRY(check_ptr(O, "O"));
  if (lse) MSA_TRY(check_ptr(lse, "lse"));
  MSA_TRY(check_ptr(ws, "ws"));
  const size_t need = decode_ws(d);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  msa::AttnWorkspace w;
  msa::attn_workspace_carve(ws, d->B, d->B, d->N, d->G, d->Hq / d->G, d->k, d->Bk, true, &w);
  const hipError_t e = msa::launch_attn_decode(q, K_pool, V_pool, idx, O, lse, d->B, d->N,
                                               d->Hq, d->G, d->k, 128, pc, w,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_decode_paged");
  return MSA_OK;
}

}  // extern "C"
