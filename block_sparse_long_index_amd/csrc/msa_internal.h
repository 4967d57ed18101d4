// msa_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// A paged cache for decode: 128-token pages in a pool of `pages`; sequence
// b's logical block j lives in page table[b * nb + j] and the sequence holds
// lens[b] tokens.  table == nullptr: the contiguous layout, every sequence as
// long as the capacity.  Both arrays are device memory.
struct PagedCache {
  const int32_t* table;
  const int64_t* lens;
  int64_t pages;
  int32_t nb;  // table row length (blocks of capacity)
};

// Stages 1+2 (write S, blocks of Bk keys) or stages 1-3 fused (write idx,
// Bk = 128) for the query rows t0 .. t0 + Tw - 1 of T; S holds those rows
// only ([B, G, Tw, NB]).  fp8: q^I and k^I are e4m3 bytes instead of bf16
// (Bk = 128).  wgs > 0: at most that many workgroups, each looping over the
// work items (the selection then occupies at most wgs CUs).  counter
// (non-null, zero before the first of them): the workgroups take items from
// it, so several launches over the same rows share the items.
hipError_t launch_index_tiles(bool write_scores, bool fp8, const void* qI, const void* kI,
                              float* S, int32_t* idx, int64_t B, int64_t T, int64_t t0,
                              int64_t Tw, int64_t N, int G, int Bk, int k, hipStream_t st,
                              int wgs = 0, int32_t* counter = nullptr);

// Stages 1+2 for T == 1: streams the index keys, S is [B, G, 1, NB] with NB
// blocks of Bk keys (fp8 and paged caches: Bk = 128).
hipError_t launch_decode_scan(bool fp8, const void* qI, const void* kI, float* S,
                              int64_t B, int64_t N, int G, int Bk, const PagedCache& pc,
                              hipStream_t st);

// Stage 3 for the query rows t0 .. t0 + Tw - 1 of T from their scores
// S [B, G, Tw, NB] (blocks of Bk keys) into idx [B, G, T, k], k <= 64.
hipError_t launch_topk_rows(const float* S, int32_t* idx, int64_t B, int64_t T, int64_t t0,
                            int64_t Tw, int64_t N, int G, int Bk, int k, const PagedCache& pc,
                            hipStream_t st);

// Queries per KV-outer work chunk (a chunk's rows = kChunkQueries * hg).
constexpr int kChunkQueries = 128;
struct AttnWorkspace {
  int32_t* hist;       // [G * NB * nc]: unit block counts, then exclusive offsets
  int32_t* tile_sums;  // [ntiles]
  int32_t* totals;     // [4 + nstages]: entries, -, -, -, chunks per stage
  int32_t* entries;    // [window * G * k]
  int4* chunks;        // [nstages][max_chunks]
  uint16_t* opart;     // one stage's partial O: [stage_rows, k, hg, 128] bf16, unnormalised
  float2* lpart;       // [stage_rows, k, hg]: (log2-domain row max, row sum)
  int64_t window;      // query rows of one sequence per inversion
  int64_t stage_rows;  // rows of one group per KV-outer stage
  int64_t max_chunks;  // per stage
  int64_t nstages;
  int64_t nbins;       // G * NB
  int64_t nhist, ntiles;
  int32_t rq, nc;      // rows per histogram unit, units per full window
  int64_t sink;        // index of the spare partial row
};

// Bytes of workspace for a window of `window` rows of one sequence processed
// in stages of `stage_rows` rows of one group.  decode: one chunk per
// (sequence, group, slot), window = B.
size_t attn_workspace_bytes(int64_t window, int64_t stage_rows, int64_t N, int G, int hg, int k,
                            int Bk, bool decode);
void attn_workspace_carve(void* ws, int64_t window, int64_t stage_rows, int64_t N, int G, int hg,
                          int k, int Bk, bool decode, AttnWorkspace* out);

// Inversion of the selection for the query rows [t0, t0 + W) of sequence b
// into per-stage chunk lists in w; *nsub = row stages per group.
hipError_t launch_invert_window(const int32_t* idx, int64_t b, int64_t T, int64_t t0, int64_t W,
                                int64_t N, int G, int k, int Bk, const AttnWorkspace& w,
                                int32_t* nsub, hipStream_t st);
// Stage 4 backward: dq [B, T, Hq, 128], dK, dV [B, G, N, 128] (fp32, all
// overwritten) from q, O, dO [B, T, Hq, 128], K, V, idx and the forward's lse
// [B, Hq, T]; Dr: B*T*Hq floats of scratch.  Blocks of Bk keys (32, 64, 128).
hipError_t launch_attn_backward(const void* q, const void* K, const void* V,
                                const int32_t* idx, const void* O, const float* lse,
                                const void* dO, float* dq, float* dK, float* dV, float* Dr,
                                int64_t B, int64_t T, int64_t N, int Hq, int G, int k, int Bk,
                                const AttnWorkspace& w, hipStream_t st);
// Sum in slot order of per-(row, slot) bf16 partials (the backward's layout)
// for the rows of one stage and group: out [.., outer, 128] fp32 at
// (b*T + t) * outer + group.
hipError_t launch_dq_combine(const int32_t* idx, const uint16_t* part, float* out, int64_t T,
                             int64_t r0, int64_t rows, int outer, int G, int k, int rl_base,
                             int group, hipStream_t st);
// Index-branch KL alignment backward: dqI [B, T, G, 128], dkI [B, N, 128]
// (fp32, overwritten), kl [B, G, T] (nullable) from q^I, k^I, q, K, idx and
// the main lse [B, Hq, T]; lpx: B*G*T floats of scratch; teach: w.stage_rows
// * k * Bk floats of scratch (one stage's teacher).  Blocks of Bk keys.
hipError_t launch_index_kl_backward(const void* qI, const void* kI, const void* q, const void* K,
                                    const int32_t* idx, const float* lse, float* dqI, float* dkI,
                                    float* kl, float* lpx, float* teach, int64_t B, int64_t T,
                                    int64_t N, int Hq, int G, int k, int Bk,
                                    const AttnWorkspace& w, hipStream_t st);
// Pieces of the two backward launchers, for the fused training backward:
// zeroing / D = dO . O, and one stage (group g, row stage sub of the window
// of W rows at global row r0, S row stages per group) after
// launch_invert_window.  teach: [stage rows, k, Bk] fp32, written by the
// main stage (null: no teacher) or by the KL stage itself (make_teacher) and
// read by the KL stage.
hipError_t attn_bwd_prepare(const void* O, const void* dO, float* dK, float* dV, float* Dr,
                            int64_t B, int64_t T, int64_t N, int Hq, int G, hipStream_t st);
hipError_t attn_bwd_stage(const void* q, const void* K, const void* V, const int32_t* idx,
                          const float* lse, const void* dO, const float* Dr, float* dq,
                          float* dK, float* dV, float* teach, int64_t T, int64_t N, int Hq,
                          int G, int k, int Bk, const AttnWorkspace& w, int64_t r0, int64_t W,
                          int32_t S, int g, int32_t sub, hipStream_t st);
hipError_t index_kl_prepare(float* dkI, int64_t B, int64_t N, hipStream_t st);
hipError_t index_kl_stage(const void* qI, const void* kI, const void* q, const void* K,
                          const int32_t* idx, const float* lse, float* teach, bool make_teacher,
                          float* dqI,
                          float* dkI, float* kl, float* lpx, int64_t T, int64_t N, int Hq, int G,
                          int k, int Bk, const AttnWorkspace& w, int64_t r0, int64_t W, int32_t S,
                          int g, int32_t sub, hipStream_t st);
// Both training backwards in one pass over the stages (the outputs of
// launch_attn_backward and launch_index_kl_backward); teach: w.stage_rows *
// k * Bk floats of scratch.
hipError_t launch_train_backward(const void* q, const void* K, const void* V, const void* qI,
                                 const void* kI, const int32_t* idx, const void* O,
                                 const float* lse, const void* dO, float* dq, float* dK,
                                 float* dV, float* dqI, float* dkI, float* kl, float* Dr,
                                 float* lpx, float* teach, int64_t B, int64_t T, int64_t N,
                                 int Hq, int G, int k, int Bk, const AttnWorkspace& w,
                                 hipStream_t st);
hipError_t launch_attn_prefill(const void* q, const void* K, const void* V,
                               const int32_t* idx, void* O, float* lse,
                               int64_t B, int64_t T, int64_t N, int Hq, int G,
                               int k, int Bk, const AttnWorkspace& w, hipStream_t st);
// Stage 4 for the query rows [t0, t0 + W) of sequence b only (W <= w.window):
// their inversion, then their stages.  Reads only those rows' idx.
hipError_t launch_attn_prefill_rows(const void* q, const void* K, const void* V,
                                    const int32_t* idx, void* O, float* lse, int64_t b,
                                    int64_t T, int64_t t0, int64_t W, int64_t N, int Hq, int G,
                                    int k, int Bk, const AttnWorkspace& w, hipStream_t st);

// Stages 1-4 of a prefill in windows of about `win` query rows (all
// sequences): selection of window i on st, then its attention on st2 after an
// event, so that window i's attention overlaps the later windows' selection.
// Bk < 128: S holds the scores of `srows` rows of every sequence.  counters:
// kMaxPrefillWindows ints of scratch.  w: an attention workspace whose window
// is >= win.  ev: nev >= ceil(T / win) + 2 events (unused when st2 == st).
constexpr int kMaxPrefillWindows = 72;
// Window boundaries [bounds[i], bounds[i + 1]) of the pipelined prefill for
// windows of `win` rows; returns their number.
int prefill_windows(int64_t T, int64_t win, int64_t* bounds, int max_windows);
hipError_t launch_prefill_pipelined(const void* qI, const void* kI, const void* q, const void* K,
                                    const void* V, int32_t* idx, void* O, float* lse, int64_t B,
                                    int64_t T, int64_t N, int Hq, int G, int k, int Bk,
                                    int64_t win, float* S, int64_t srows, int32_t* counters,
                                    const AttnWorkspace& w, hipStream_t st, hipStream_t st2,
                                    hipEvent_t* ev, int nev);

// One-call decode after the scan: per (sequence, group) one workgroup selects
// the blocks from S [B, G, NB] (writing idx) and attends them, writing O and
// lse (nullable) directly.
// scratch: decode_step_scratch_bytes(B, G, Hq) bytes (fp32 results of the
// row parts when a row is split over two workgroups; 0 bytes otherwise).
size_t decode_step_scratch_bytes(int64_t B, int G, int Hq);
hipError_t launch_decode_step(const float* S, const void* q, const void* K, const void* V,
                              int32_t* idx, void* O, float* lse, void* scratch, int64_t B,
                              int64_t N, int Hq, int G, int k, int Bk, const PagedCache& pc,
                              hipStream_t st);

hipError_t launch_attn_decode(const void* q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse,
                              int64_t B, int64_t N, int Hq, int G, int k, int Bk,
                              const PagedCache& pc, const AttnWorkspace& w, hipStream_t st);

// Per-kernel timing (msa_timing.hip).  Kinds are the MSA_KERNEL_* ids of
// msa.h.  TimedLaunch brackets the launches made during its lifetime with
// two events on `st` when timing is on.
bool timing_enabled();
int timing_open(int kind, hipStream_t st);
void timing_close(int slot, hipStream_t st);
hipError_t timing_start(int64_t max_launches);
hipError_t timing_stop(double* ms, int64_t* launches, int nkinds, int64_t* dropped);
struct TimedLaunch {
  int slot;
  hipStream_t st;
  TimedLaunch(int kind, hipStream_t s) : slot(timing_enabled() ? timing_open(kind, s) : -1), st(s) {}
  ~TimedLaunch() { timing_close(slot, st); }
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;
};

}  // namespace msa
