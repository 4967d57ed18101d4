/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) hot path for AMD MI355X
 * (gfx950): the forward, and the two backward calls of a training step.
 * Implemented by libmsa.so (hand-written HIP kernels).
 *
 * The method (MSA study notes, dimensionstp.github.io/study-concept/msa,
 * section 2-3 "Fixed attention budget", its three displayed equations and the
 * Main Branch equation; section 3 for the branches and the kernel ideas):
 *
 *   (1) index score   s[t,g,j] = q^I[t,g] . k^I[j] / sqrt(d_I),  j <= p(t)
 *   (2) block max     S[t,g,b] = max_{j in block b, j <= p(t)} s[t,g,j]
 *   (3) selection     the local block local(t) = floor(p(t)/Bk), always,
 *                     plus the best min(k-1, local(t)) earlier blocks by S
 *   (4) main branch   O[t,h] = softmax(q[t,h] K_g^T / sqrt(d_h)) V_g over the
 *                     keys j <= p(t) of the selected blocks of h's group g
 *   training          the gradients of (4) with the selection held fixed, and
 *                     the index branch's KL alignment against the group's
 *                     mean main-branch weights (study notes sections 4-2, 4-3)
 *
 * Conventions shared by every call
 * --------------------------------
 * Positions.  Query row t (0 <= t < T) of sequence b sits at absolute position
 *   p(t) = N - T + t: prefill has T == N; decode has T == 1 and N is the cache
 *   length including the new token.
 * Groups.  Query head h belongs to group g = h / (Hq / G).  Every head of a
 *   group reads the group's selection (study notes, section 3-3).
 * Budget.  k counts the local block: at most k * Bk keys per query and group
 *   (study notes, section 2-3: a budget of 2048 tokens with the local block
 *   counted in it).
 * Ties.  Among equal block scores the lower block index wins.
 * Slot order.  idx rows list the selected blocks in ascending order; the
 *   local block is the last valid slot; unused slots hold -1.
 * Invisible blocks.  Blocks after local(t) have S = -inf and are never
 *   selected.  The local block's S is its true causal max; selection ignores
 *   it (it is forced).
 * Precision.  bf16 inputs, fp32 accumulation.  S is the fp32 value nearest the
 *   score (exact for integer-valued index inputs).  O is bf16; lse is fp32,
 *   natural log.
 * Memory.  Every pointer is a device pointer the caller owns, 16-byte aligned,
 *   to a contiguous row-major tensor of the layout given.  The library never
 *   allocates or frees device memory and keeps no pointer after returning;
 *   its only device memory of its own is the static scratch array of
 *   msa_sparse_attn_decode_noalloc.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it; nothing synchronises.  Results are ready when the
 *   stream reaches them.
 * Errors.  Arguments are validated on the host before any HIP call; on an
 *   error nothing is launched and no output is touched.  A HIP launch error
 *   returns MSA_ERR_HIP (text from msa_last_error()).
 * Supported now: d_h == d_I == 128; Bk in {32, 64, 128} with 1 <= k and
 *   k * Bk <= 2048 (the study notes' fixed budget of section 2-3, which its
 *   block-size comparison in section 4-6 keeps: k <= 16, 32, 64) and at most
 *   16384 blocks per sequence; G in {1,2,4,8,16}, Hq / G in {1,2,4,8,16};
 *   N <= 2^21.  The fp8 index calls and the paged calls take Bk == 128; the
 *   training calls take every supported Bk.
 *   Others: MSA_ERR_UNSUPPORTED.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t B;   /* sequences */
    int64_t T;   /* query rows per sequence (T <= N) */
    int64_t N;   /* keys per sequence (context length) */
    int32_t Hq;  /* query heads */
    int32_t G;   /* GQA groups = KV heads = index query heads */
    int32_t d_h; /* main-branch head dimension */
    int32_t d_I; /* index-branch dimension */
    int32_t Bk;  /* block size in tokens */
    int32_t k;   /* blocks selected per (query, group), local included */
} msa_dims_t;

enum {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARGUMENT = -1,
    MSA_ERR_UNSUPPORTED = -2,
    MSA_ERR_WORKSPACE_TOO_SMALL = -3,
    MSA_ERR_HIP = -4
};

/* Operation ids for msa_workspace_bytes. */
enum {
    MSA_OP_INDEX_SCORES = 0,
    MSA_OP_SELECT_BLOCKS = 1,
    MSA_OP_SELECT_FROM_SCORES = 2,
    MSA_OP_ATTN_PREFILL = 3,
    MSA_OP_ATTN_DECODE = 4,
    MSA_OP_ATTN_BACKWARD = 5,
    MSA_OP_INDEX_KL_BACKWARD = 6,
    MSA_OP_TRAIN_BACKWARD = 7,
    MSA_OP_PREFILL = 8,
    MSA_OP_DECODE = 9
};

/*
 * Stages 1 and 2 (study notes section 2-3, equations for s and S; section
 * 3-2 on max pooling of the causally visible token scores).
 *   qI  bf16 [B, T, G, d_I]   index queries, one per (row, group)
 *   kI  bf16 [B, N, d_I]      index keys, one shared head
 *   S   fp32 [B, G, T, ceil(N/Bk)]  out: block scores; -inf where invisible
 */
int msa_index_scores(const msa_dims_t *dims, const void *qI, const void *kI,
                     float *S, void *stream);

/*
 * Stages 1 to 3 fused: the token scores and block maxima stay on chip and
 * feed an exp-free streaming top-k (study notes section 3-5 "Exp-free
 * Top-k"; the Flash-MSA blog on hackernews.jp, section on the proxy
 * attention, for top-k kept in registers while the keys stream).
 *   qI, kI as for msa_index_scores
 *   idx int32 [B, G, T, k]    out: selected blocks (see conventions)
 *   ws / ws_bytes             scratch, >= msa_workspace_bytes(MSA_OP_SELECT_BLOCKS):
 *                             decode (T == 1) uses a row of block scores; a
 *                             prefill with Bk == 128 needs none; with Bk < 128
 *                             the block scores of a window of query rows are
 *                             materialised and ranked, window after window (the
 *                             default size holds up to 1 GB of scores; any
 *                             workspace of at least one row's scores,
 *                             B * G * ceil(N/Bk) floats, is accepted)
 */
int msa_select_blocks(const msa_dims_t *dims, const void *qI, const void *kI,
                      int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/*
 * The index branch (stages 1+2, and 1-3 fused) on 8-bit inputs.  The pages'
 * kernel co-design section (the Italian news page on MSA, last paragraph)
 * lists FP8 among the precisions of the authors' kernel; the definitions are
 * unchanged: s = (q^I . k^I) / sqrt(d_I) with the products and sums in fp32,
 * then the same block max and selection rules as msa_index_scores and
 * msa_select_blocks.
 *   qI  fp8 e4m3 (OCP e4m3fn: bias 7, no infinities) [B, T, G, d_I], one byte
 *       per value
 *   kI  fp8 e4m3 [B, N, d_I]
 *   S, idx, ws, ws_bytes, errors: as for the bf16 calls (the decode workspace
 *       is the same msa_workspace_bytes(MSA_OP_SELECT_BLOCKS))
 * Integer-valued inputs with |dot| < 2^24 are exact in any summation order,
 * so on such inputs S and idx equal the bf16 calls' on the same values.
 */
int msa_index_scores_fp8(const msa_dims_t *dims, const void *qI, const void *kI,
                         float *S, void *stream);
int msa_select_blocks_fp8(const msa_dims_t *dims, const void *qI, const void *kI,
                          int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/*
 * Stage 3 alone, from materialised block scores (study notes section 2-3,
 * the TopK equation; section 3-5 "Exp-free Top-k": only the order of raw
 * scores matters, no max/exp/sum).
 *   S   fp32 [B, G, T, ceil(N/Bk)]  as written by msa_index_scores
 *   idx int32 [B, G, T, k]          out
 */
int msa_select_blocks_from_scores(const msa_dims_t *dims, const float *S,
                                  int32_t *idx, void *stream);

/*
 * Stage 4 for prefill, scheduled KV-outer (study notes section 3-5
 * "KV-outer sparse attention": a reverse index gathers, for each KV block,
 * the queries that chose it; hot blocks are pre-split into chunks; partial
 * results are merged by a two-phase combine.  The Flash-MSA blog's backward
 * section describes the same inversion of [batch, head, query, slot] ->
 * block into [batch, head, block] -> queries.)
 *   q   bf16 [B, T, Hq, d_h]
 *   K,V bf16 [B, G, N, d_h]
 *   idx int32 [B, G, T, k]    as written by msa_select_blocks
 *   O   bf16 [B, T, Hq, d_h]  out
 *   lse fp32 [B, Hq, T]       out, may be NULL
 *   ws / ws_bytes             scratch; msa_workspace_bytes(MSA_OP_ATTN_PREFILL)
 *                             gives the size for the default query window.  A
 *                             smaller workspace (down to one query row per
 *                             window) is accepted and processes the rows in
 *                             more windows; below that: WORKSPACE_TOO_SMALL.
 */
int msa_sparse_attn_prefill(const msa_dims_t *dims, const void *q,
                            const void *K, const void *V, const int32_t *idx,
                            void *O, float *lse, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Stages 1 to 4 of a prefill in one call: msa_select_blocks, then
 * msa_sparse_attn_prefill, on the same arguments and with the same results
 * (idx bit for bit, O and lse as the prefill call computes them), scheduled
 * window by window of query rows so that the two halves overlap.  The study
 * notes (section 5-3 on efficiency) name the selection and the gather and
 * combine of the sparse attention as the overheads of a prefill; here the
 * fused selection of window i + 1 (bound by the matrix cores) runs on
 * `stream` while the attention of window i (bound by the memory traffic of
 * its gathers and partial results) runs on `stream2`.
 *   qI, kI, q, K, V, idx, O, lse   as for msa_select_blocks and
 *                                  msa_sparse_attn_prefill (idx is written)
 *   ws / ws_bytes  >= msa_workspace_bytes(MSA_OP_PREFILL)
 *   stream         the caller's stream: everything is ordered after the work
 *                  already on it, and the results are ready when it reaches
 *                  the point where the call returned
 *   stream2        a second stream of the same device for the attention
 *                  windows (it waits for each window's selection; `stream`
 *                  waits for its last window), or NULL: every launch in
 *                  order on `stream`.  Prefills of fewer than four windows
 *                  (T up to about 49152 rows) also run in order on `stream`.
 * Needs T >= 2.  Any supported Bk (with Bk < 128 the selection materialises
 * the scores of up to 1 GB of rows at a time in the workspace).
 */
int msa_prefill(const msa_dims_t *dims, const void *qI, const void *kI, const void *q,
                const void *K, const void *V, int32_t *idx, void *O, float *lse, void *ws,
                size_t ws_bytes, void *stream, void *stream2);

/*
 * Backward of stage 4 for training: the gradients of exact softmax attention
 * over each row's selected blocks, the selection held fixed (the Flash-MSA
 * blog's backward pass keeps the forward's block indices and the main
 * branch's lse, inverts the selection into block -> queries and schedules
 * the shared KV blocks from it; the study notes, section 3-3, define the
 * forward being differentiated).  With P = softmax over the support,
 * dS = P (dO.V - dO.O):  dq = dS K / sqrt(d_h), dK = dS^T q / sqrt(d_h),
 * dV = P^T dO, dK and dV summed over the heads of each group.
 *   q, O, dO  bf16 [B, T, Hq, d_h]   O and lse as written by the prefill call
 *   K, V      bf16 [B, G, N, d_h]
 *   idx       int32 [B, G, T, k]     the forward's selection
 *   lse       fp32 [B, Hq, T]        natural log (required)
 *   dq        fp32 [B, T, Hq, d_h]   out, overwritten
 *   dK, dV    fp32 [B, G, N, d_h]    out, overwritten (keys no row selects get 0)
 *   ws / ws_bytes  >= msa_workspace_bytes(MSA_OP_ATTN_BACKWARD) for the
 *                  default query window; a smaller one (down to one row per
 *                  window plus B*T*Hq floats) runs more windows.
 * Any supported block size (Bk = 32, 64, 128).  dK and dV are accumulated with
 * fp32 atomic adds, so their last bits can differ between runs; dq is summed
 * in slot order.
 */
int msa_sparse_attn_backward(const msa_dims_t *dims, const void *q, const void *K,
                             const void *V, const int32_t *idx, const void *O,
                             const float *lse, const void *dO, float *dq, float *dK,
                             float *dV, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of the index branch's KL alignment for training: per row and
 * group, over the row's support (the visible keys of its selected blocks),
 * teacher p_t = mean over the group's heads of the main attention weights
 * (detached), proxy p_x = softmax of the index scores s over the same support,
 * loss KL(p_t || p_x); its gradient on s is p_x - p_t, giving
 * dq^I = (p_x - p_t) k^I / sqrt(d_I) and dk^I += (p_x - p_t) q^I / sqrt(d_I)
 * summed over rows and groups (study notes sections 4-2 and 4-3 on the teacher
 * and the detach; the Flash-MSA blog's "KL divergence loss" section on the
 * gradient and the proxy lse recomputed over the sparse support).
 *   qI, kI    bf16 [B, T, G, d_I], [B, N, d_I]   the index branch's inputs
 *   q, K      bf16 [B, T, Hq, d_h], [B, G, N, d_h]
 *   idx       int32 [B, G, T, k]     the forward's selection
 *   lse       fp32 [B, Hq, T]        the main branch's lse from the prefill
 *   dqI       fp32 [B, T, G, d_I]    out, overwritten
 *   dkI       fp32 [B, N, d_I]       out, overwritten (keys no row selects get 0)
 *   kl        fp32 [B, G, T]         out, the loss per row and group; may be NULL
 *   ws / ws_bytes  >= msa_workspace_bytes(MSA_OP_INDEX_KL_BACKWARD) for the
 *                  default window; smaller (down to one row per window plus
 *                  B*G*T floats) runs more windows.
 * Any supported block size (Bk = 32, 64, 128).  dkI is accumulated with fp32
 * atomic adds; dqI and kl are summed in slot order.  Scaling by a loss weight
 * is the caller's.
 */
int msa_index_kl_backward(const msa_dims_t *dims, const void *qI, const void *kI,
                          const void *q, const void *K, const int32_t *idx, const float *lse,
                          float *dqI, float *dkI, float *kl, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * Both training backwards in one call, the fused proxy + main backward of
 * the Flash-MSA blog's backward pass: one inversion of the selection drives
 * both branches stage by stage, and the main branch's weights are formed
 * once.  Each stage's main backward writes the teacher of its rows (the mean
 * over the group's heads of the main weights, fp32, in the workspace); the
 * index branch's pass right after reads it instead of recomputing the main
 * scores.  Outputs and their meaning are those of msa_sparse_attn_backward
 * (dq, dK, dV) and msa_index_kl_backward (dqI, dkI, kl); the arguments are
 * the union of theirs, with the same shapes and layouts.
 *   ws / ws_bytes  >= msa_workspace_bytes(MSA_OP_TRAIN_BACKWARD) for the
 *                  default window; smaller (down to one row per window plus
 *                  B*T*(Hq+G) floats plus one stage's teacher) runs more
 *                  windows.
 * Any supported block size.  Results equal those of the two separate calls
 * up to rounding (the teacher's head sum is taken in another order) and the
 * atomic-add order of dK, dV and dkI.
 */
int msa_train_backward(const msa_dims_t *dims, const void *q, const void *K, const void *V,
                       const void *qI, const void *kI, const int32_t *idx, const void *O,
                       const float *lse, const void *dO, float *dq, float *dK, float *dV,
                       float *dqI, float *dkI, float *kl, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * Stage 4 for decode (T must be 1): split over the B * G * k selected KV
 * blocks, then the same combine (llama.cpp analysis page, section 4: block
 * scores and max pooling, local block plus top-k, then attention over the
 * gathered K/V; section 2: only the 256 B/token index keys and the selected
 * K/V blocks are read).
 *   q   bf16 [B, Hq, d_h]     (= [B, 1, Hq, d_h])
 *   K,V bf16 [B, G, N, d_h]   the KV cache, N = cache length
 *   idx int32 [B, G, 1, k]
 *   O   bf16 [B, Hq, d_h]     out
 *   lse fp32 [B, Hq]          out, may be NULL
 *   ws / ws_bytes             >= msa_workspace_bytes(MSA_OP_ATTN_DECODE)
 */
int msa_sparse_attn_decode(const msa_dims_t *dims, const void *q,
                           const void *K, const void *V, const int32_t *idx,
                           void *O, float *lse, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * msa_sparse_attn_decode without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  It allocates nothing.  The partial
 * results of the selected blocks live in a static device array of the library
 * instead (8.25 MB on each GPU the library runs on, held until the process
 * ends), which bounds the call to B * Hq * k <= 32768 partial rows (the
 * 256K x 16 decode step uses 16384); larger calls return
 * MSA_ERR_WORKSPACE_TOO_SMALL before anything is launched.  The array used is
 * the one of the current device, so `stream` must belong to it.  Every call on
 * a GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Arguments,
 * results and errors are those of msa_sparse_attn_decode; the kernels are
 * the same, so the outputs are bitwise equal to its outputs.
 */
int msa_sparse_attn_decode_noalloc(const msa_dims_t *dims, const void *q, const void *K,
                                   const void *V, const int32_t *idx, void *O, float *lse,
                                   void *stream);

/*
 * Decode over paged caches: the explicit per-sequence position -> cell ->
 * block map that the llama.cpp analysis page (section 4 on kv_unified and its
 * dense fallback, section 5 on what to build) asks for, so that sequences of
 * different lengths share one cache pool.  Token i of sequence b lives in
 * row i % Bk of page block_table[b][i / Bk]; sequence b holds seq_lens[b]
 * tokens, the last of which is the query's own (position seq_lens[b] - 1).
 * Everything else is the contiguous calls' definition for that sequence.
 *   dims          T == 1; N = the table's capacity in tokens (every
 *                 seq_lens[b] <= N); the table has ceil(N / Bk) columns
 *   num_pages     pages in each pool (1 .. 2^31)
 *   block_table   int32 [B, ceil(N / Bk)], device; page ids in [0, num_pages)
 *   seq_lens      int64 [B], device; in [1, N]
 *   kI_pool       bf16 (fp8 e4m3 for _fp8) [num_pages, Bk, d_I]
 *   K_pool/V_pool bf16 [num_pages, G, Bk, d_h]
 *   qI, q, idx, O, lse, ws: as for msa_select_blocks / msa_sparse_attn_decode
 *                 (the same workspace sizes)
 * The table and lengths are device data and are not validated on the host:
 * lengths are clamped to [1, N] and page ids to [0, num_pages) inside the
 * kernels, so bad contents give wrong results but no access outside the
 * pools.  Table columns at or past a sequence's last block are never read.
 */
int msa_select_blocks_paged(const msa_dims_t *dims, const void *qI, const void *kI_pool,
                            int64_t num_pages, const int32_t *block_table,
                            const int64_t *seq_lens, int32_t *idx, void *ws, size_t ws_bytes,
                            void *stream);
int msa_select_blocks_paged_fp8(const msa_dims_t *dims, const void *qI, const void *kI_pool,
                                int64_t num_pages, const int32_t *block_table,
                                const int64_t *seq_lens, int32_t *idx, void *ws,
                                size_t ws_bytes, void *stream);
int msa_sparse_attn_decode_paged(const msa_dims_t *dims, const void *q, const void *K_pool,
                                 const void *V_pool, int64_t num_pages,
                                 const int32_t *block_table, const int64_t *seq_lens,
                                 const int32_t *idx, void *O, float *lse, void *ws,
                                 size_t ws_bytes, void *stream);

/*
 * msa_decode over paged pools (the serving shape of the llama.cpp analysis
 * page, sections 4-5): the paged selection and the paged decode attention in
 * one call, with msa_decode's one-kernel-per-row step.  Arguments as for
 * msa_select_blocks_paged(_fp8) and msa_sparse_attn_decode_paged, the pools
 * sharing num_pages and block_table; ws / ws_bytes >= msa_workspace_bytes(
 * MSA_OP_DECODE).  idx equals msa_select_blocks_paged(_fp8)'s bit for bit, O
 * and lse are msa_decode's for the sequences the table describes.
 */
int msa_decode_paged(const msa_dims_t *dims, const void *qI, const void *kI_pool, const void *q,
                     const void *K_pool, const void *V_pool, int64_t num_pages,
                     const int32_t *block_table, const int64_t *seq_lens, int32_t *idx, void *O,
                     float *lse, void *ws, size_t ws_bytes, void *stream);
int msa_decode_paged_fp8(const msa_dims_t *dims, const void *qI, const void *kI_pool,
                         const void *q, const void *K_pool, const void *V_pool,
                         int64_t num_pages, const int32_t *block_table,
                         const int64_t *seq_lens, int32_t *idx, void *O, float *lse, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * A decode step in one call (T == 1): stages 1 to 4 with the results of
 * msa_select_blocks followed by msa_sparse_attn_decode (idx bit for bit; O
 * and lse within the decode tolerance: the slot results are merged in fp32
 * inside the chip instead of through bf16 partials).  The llama.cpp analysis
 * page (section 2) reads per step the whole index-key cache plus only the
 * selected K/V blocks; the study notes (section 3-5) scan, select, then
 * attend.  After the scan of the index keys, each (sequence, group) row is
 * one workgroup that selects its blocks, attends them with an online softmax
 * and merges its waves' results, so the selected K/V are the only other bytes
 * read and nothing is written but idx, O and lse.  Batches of fewer than 128
 * (sequence, group) rows run the separate top-k, attention and combine
 * launches instead (one workgroup per row would leave most of the chip idle).
 *   qI, kI, q, K, V, idx, O, lse   as for msa_select_blocks and
 *                                  msa_sparse_attn_decode (idx is written)
 *   ws / ws_bytes  >= msa_workspace_bytes(MSA_OP_DECODE)
 * bf16 index inputs, contiguous caches, every supported Bk.
 */
int msa_decode(const msa_dims_t *dims, const void *qI, const void *kI, const void *q,
               const void *K, const void *V, int32_t *idx, void *O, float *lse, void *ws,
               size_t ws_bytes, void *stream);

/*
 * msa_decode on 8-bit (E4M3) index inputs (the kernel co-design section of
 * the Italian news page on MSA lists FP8 among the kernel's precisions; the
 * definitions are those of msa_select_blocks_fp8): qI fp8 e4m3 [B, 1, G, d_I]
 * and kI fp8 e4m3 [B, N, d_I], one byte per value, Bk = 128 (otherwise
 * MSA_ERR_UNSUPPORTED).  idx equals msa_select_blocks_fp8's bit for bit;
 * everything else (q, K, V, O, lse, the workspace of MSA_OP_DECODE, errors)
 * as for msa_decode.
 */
int msa_decode_fp8(const msa_dims_t *dims, const void *qI, const void *kI, const void *q,
                   const void *K, const void *V, int32_t *idx, void *O, float *lse, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * Per-kernel timing, for measurement harnesses.  Between msa_timing_begin and
 * msa_timing_end every launch of the kernel kinds below, by any call on any
 * stream, is bracketed by two HIP events recorded on the stream the kernel is
 * launched on; msa_timing_end waits for those events and returns, per kind,
 * the summed elapsed milliseconds and the number of launches timed.  The
 * events are created on the current device by msa_timing_begin (room for
 * max_launches launches, 1 <= max_launches <= 2^20) and destroyed by
 * msa_timing_end.  A launch past that room is not timed, and msa_timing_end
 * then returns MSA_ERR_INVALID_ARGUMENT after filling the arrays.  Timing adds
 * two event records per timed launch; calls made with it off are unchanged.
 * Not for use under HIP graph capture.  One timing session per process.
 *   total_ms, launches  out: arrays of nkinds (<= MSA_KERNEL_KINDS) entries
 */
enum {
    MSA_KERNEL_SELECT = 0,        /* index-score tiles (fused select or score writing) */
    MSA_KERNEL_KV_OUTER = 1,      /* prefill KV-outer attention */
    MSA_KERNEL_COMBINE = 2,       /* prefill partial combine */
    MSA_KERNEL_INVERT = 3,        /* block->queries inversion (all of its kernels) */
    MSA_KERNEL_DECODE_SCAN = 4,   /* decode index-key scan */
    MSA_KERNEL_TOPK = 5,          /* top-k from materialised scores */
    MSA_KERNEL_DECODE_ATTN = 6,   /* decode split-KV attention */
    MSA_KERNEL_DECODE_COMBINE = 7,
    MSA_KERNEL_ATTN_BACKWARD = 8, /* KV-outer backward */
    MSA_KERNEL_INDEX_KL = 9,      /* index-branch KL backward passes */
    MSA_KERNEL_DECODE_STEP = 10,  /* one-call decode: selection + attention per row */
    MSA_KERNEL_KINDS = 11
};
int msa_timing_begin(int64_t max_launches);
int msa_timing_end(double *total_ms, int64_t *launches, int nkinds);

/* Scratch bytes an operation needs for these dims (0 if none); 0 also for
 * invalid dims.  Host only, no HIP call. */
size_t msa_workspace_bytes(int op, const msa_dims_t *dims);

/* Static text for a status code. */
const char *msa_status_string(int status);

/* Text of the last MSA_ERR_HIP or validation failure on this thread. */
const char *msa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
