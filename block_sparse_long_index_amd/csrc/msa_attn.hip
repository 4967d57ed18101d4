// msa_attn.hip -- main branch of MSA on gfx950: exact softmax attention over
// the selected blocks, scheduled KV-outer, and the two-phase combine.
//
// Method: MSA study notes (dimensionstp.github.io/study-concept/msa) section
// 2-3 (Main Branch equation) and section 3-3 (exact softmax over the
// selected support, per-head weights, one selection per GQA group).
// Schedule: study notes section 3-5 "KV-outer sparse attention" -- a reverse
// index gathers, for every KV block, the queries that selected it; popular
// blocks are pre-split into chunks spread over workgroups; the partial
// results are merged by a two-phase combine.  The inversion [b, g, t, slot] ->
// block into [b, g, block] -> (t, slot) is the one the Flash-MSA blog
// (hackernews.jp) describes for its backward pass; the llama.cpp analysis
// page (velog.io, section 3) illustrates the reuse of a KV block across the
// queries that chose it.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_topk.h"

#include <math.h>

namespace msa {

static_assert(kChunkQueries % 64 == 0, "a chunk's entries fill whole wave registers");
constexpr int kScanTile = 4096;    // elements per workgroup in the offset scan

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Rows of one histogram unit: about NB/8 so that writing a unit's NB bin counts
// costs no more than counting its entries; at least 256.
static int32_t unit_rows(int64_t NB) {
  int32_t r = 256;
  while (r < NB / 8) r <<= 1;
  return r;
}

// Chunks one stage can produce: its entries in chunks of kChunkQueries plus at
// most one partial chunk per block.
static int64_t stage_max_chunks(int64_t stage_rows, int64_t NB, int k) {
  const int64_t entries = stage_rows * k;
  return entries / kChunkQueries + (NB < entries ? NB : entries) + 1;
}

static void layout(int64_t window, int64_t stage_rows, int64_t N, int G, int hg, int k, int Bk,
                   bool decode, size_t* off, AttnWorkspace* w) {
  const int64_t NB = (N + Bk - 1) / Bk;
  const int32_t rq = unit_rows(NB);
  int32_t nc = 0;
  int64_t nstages = 0, maxc = 0, prow_count = 0;
  if (decode) {
    // one chunk per (sequence, group, slot); partials for every (row, group)
    nstages = 1;
    maxc = window * G * k;
    prow_count = window * G * k * hg;
  } else {
    // stages are whole histogram units, so a stage's entries are a union of
    // unit ranges of the scanned offsets
    stage_rows = ((stage_rows + rq - 1) / rq) * rq;
    nc = static_cast<int32_t>((window + rq - 1) / rq);
    nstages = G * ((window + stage_rows - 1) / stage_rows);
    maxc = stage_max_chunks(stage_rows, NB, k);
    prow_count = stage_rows * k * hg;  // one stage: stage_rows rows of one group
  }
  const int64_t nhist = static_cast<int64_t>(G) * NB * nc;
  const int64_t ntiles = (nhist + kScanTile - 1) / kScanTile;
  const int64_t entries = window * G * k;
  size_t o = 0;
  off[0] = o; o += align256(sizeof(int32_t) * (nhist > 0 ? nhist : 1));
  off[1] = o; o += align256(sizeof(int32_t) * (ntiles > 0 ? ntiles : 1));
  off[2] = o; o += align256(sizeof(int32_t) * (4 + nstages));
  off[3] = o; o += align256(sizeof(int32_t) * entries);
  off[4] = o; o += align256(sizeof(int4) * nstages * maxc);
  // one extra (sink) entry of hg rows absorbs the stores of rows past a chunk's end
  off[5] = o; o += align256(sizeof(uint16_t) * (prow_count + hg) * kHeadDim);
  off[6] = o; o += align256(sizeof(float2) * (prow_count + hg));
  off[7] = o;
  if (w) {
    w->window = window;
    w->stage_rows = stage_rows;
    w->max_chunks = maxc;
    w->nstages = nstages;
    w->nbins = static_cast<int64_t>(G) * NB;
    w->rq = rq;
    w->nc = nc;
    w->nhist = nhist;
    w->ntiles = ntiles;
    w->sink = prow_count;
  }
}

size_t attn_workspace_bytes(int64_t window, int64_t stage_rows, int64_t N, int G, int hg, int k,
                            int Bk, bool decode) {
  size_t off[8];
  layout(window, stage_rows, N, G, hg, k, Bk, decode, off, nullptr);
  return off[7];
}

void attn_workspace_carve(void* ws, int64_t window, int64_t stage_rows, int64_t N, int G, int hg,
                          int k, int Bk, bool decode, AttnWorkspace* w) {
  size_t off[8];
  layout(window, stage_rows, N, G, hg, k, Bk, decode, off, w);
  char* p = static_cast<char*>(ws);
  w->hist = reinterpret_cast<int32_t*>(p + off[0]);
  w->tile_sums = reinterpret_cast<int32_t*>(p + off[1]);
  w->totals = reinterpret_cast<int32_t*>(p + off[2]);
  w->entries = reinterpret_cast<int32_t*>(p + off[3]);
  w->chunks = reinterpret_cast<int4*>(p + off[4]);
  w->opart = reinterpret_cast<uint16_t*>(p + off[5]);
  w->lpart = reinterpret_cast<float2*>(p + off[6]);
}

// ---------------------------------------------------------------------------
// Inversion of the selection for the query rows [t0, t0 + W) of sequence b: a
// counting sort of the entries e = (t - t0) << 6 | slot by (group, block).
//   1. unit histograms: workgroup (c, g) counts, in LDS, the blocks chosen by
//      group g in rows [c*rq, (c+1)*rq) of the window; hist[(g*NB + blk)*nc + c]
//   2. exclusive scan of hist in that order: the entries of bin (g, blk) are
//      contiguous, and inside a bin ordered by row unit
//   3. scatter: each unit writes its entries from its offsets (LDS cursors)
//   4. chunks: every bin is cut into chunks of at most kChunkQueries; chunk slots
//      are allocated with one atomic per wave
// LDS atomics keep hot blocks (block 0, the local block, needles) from
// serialising on a global counter.
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

struct InvArgs {
  const int32_t* idx;
  int32_t* hist;
  int32_t* entries;
  int64_t T, t0, W;
  int32_t b, G, k, NB, rq, nc;
};

__global__ void __launch_bounds__(256) hist_kernel(InvArgs a) {
  extern __shared__ int32_t sh[];
  const int c = blockIdx.x, g = blockIdx.y;
  for (int i = threadIdx.x; i < a.NB; i += 256) sh[i] = 0;
  __syncthreads();
  const int64_t r_lo = static_cast<int64_t>(c) * a.rq;
  const int64_t r_hi = (r_lo + a.rq) < a.W ? (r_lo + a.rq) : a.W;
  const int32_t* src = a.idx + ((static_cast<int64_t>(a.b) * a.G + g) * a.T + a.t0 + r_lo) * a.k;
  const int64_t n = (r_hi - r_lo) * a.k;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const int32_t blk = src[i];
    if (blk >= 0 && blk < a.NB) atomicAdd(&sh[blk], 1);
  }
  __syncthreads();
  int32_t* dst = a.hist + static_cast<int64_t>(g) * a.NB * a.nc + c;
  for (int i = threadIdx.x; i < a.NB; i += 256) dst[static_cast<int64_t>(i) * a.nc] = sh[i];
}

__global__ void __launch_bounds__(256) scatter_kernel(InvArgs a) {
  extern __shared__ int32_t sh[];
  const int c = blockIdx.x, g = blockIdx.y;
  const int32_t* off = a.hist + static_cast<int64_t>(g) * a.NB * a.nc + c;
  for (int i = threadIdx.x; i < a.NB; i += 256) sh[i] = off[static_cast<int64_t>(i) * a.nc];
  __syncthreads();
  const int64_t r_lo = static_cast<int64_t>(c) * a.rq;
  const int64_t r_hi = (r_lo + a.rq) < a.W ? (r_lo + a.rq) : a.W;
  const int32_t* src = a.idx + ((static_cast<int64_t>(a.b) * a.G + g) * a.T + a.t0 + r_lo) * a.k;
  const int64_t n = (r_hi - r_lo) * a.k;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const int32_t blk = src[i];
    if (blk >= 0 && blk < a.NB) {
      const int32_t pos = atomicAdd(&sh[blk], 1);
      // entry = window row << 6 | slot (k <= 64), decoded with a shift
      a.entries[pos] = static_cast<int32_t>(((r_lo + i / a.k) << 6) | (i % a.k));
    }
  }
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t x = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  const int32_t incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

// Scan phase 1: per-tile sums.
__global__ void __launch_bounds__(256) scan_tiles_kernel(const int32_t* x, int64_t n,
                                                         int32_t* tile_sums) {
  __shared__ int32_t sh[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * 16;
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += (base + j < n) ? x[base + j] : 0;
  int32_t total;
  block_exclusive_scan(s, sh, &total);
  if (threadIdx.x == 0) tile_sums[blockIdx.x] = total;
}

// Scan phase 2: exclusive scan of the tile sums (one workgroup); totals[0] =
// number of entries.
__global__ void __launch_bounds__(256) scan_sums_kernel(int32_t* tile_sums, int64_t ntiles,
                                                        int32_t* totals) {
  __shared__ int32_t sh[256];
  int32_t carry = 0;
  for (int64_t base = 0; base < ntiles; base += 256) {
    const int64_t i = base + threadIdx.x;
    const int32_t v = i < ntiles ? tile_sums[i] : 0;
    int32_t total;
    const int32_t ex = block_exclusive_scan(v, sh, &total);
    if (i < ntiles) tile_sums[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) totals[0] = carry;
}

// Scan phase 3: exclusive offsets in place.
__global__ void __launch_bounds__(256) scan_apply_kernel(int32_t* x, int64_t n,
                                                         const int32_t* tile_sums) {
  __shared__ int32_t sh[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * 16;
  int32_t v[16];
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    v[j] = (base + j < n) ? x[base + j] : 0;
    s += v[j];
  }
  int32_t total;
  int32_t run = tile_sums[blockIdx.x] + block_exclusive_scan(s, sh, &total);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (base + j < n) x[base + j] = run;
    run += v[j];
  }
}

// Stage chunk lists.  Stage (g, s) covers group g and the window rows of
// sub-window s (units [s*U, (s+1)*U)); thread (g, s, blk) cuts the entries of
// bin (g, blk) in those units into chunks of at most kChunkQueries.  A wave
// holds 64 blocks of one stage and takes its chunk slots with one atomic.
__global__ void __launch_bounds__(256) stage_chunk_kernel(const int32_t* off, int32_t* totals,
                                                          int4* chunks, int32_t NB, int64_t nbins,
                                                          int32_t nc, int32_t U, int32_t S,
                                                          int64_t maxc, int32_t bg_base) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_stage = ((NB + 63) / 64) * 64;  // waves never straddle stages
  const int64_t st = tid / per_stage;
  if (st >= nbins / NB * S) return;  // whole waves: st is uniform in a wave
  const int32_t blk = static_cast<int32_t>(tid % per_stage);
  const int lane = threadIdx.x & 63;
  const int32_t g = static_cast<int32_t>(st / S), sub = static_cast<int32_t>(st % S);
  int32_t start = 0, n = 0;
  if (blk < NB) {
    const int64_t bin = static_cast<int64_t>(g) * NB + blk;
    const int32_t u0 = sub * U;
    const int32_t u1 = (sub + 1) * U < nc ? (sub + 1) * U : nc;
    start = off[bin * nc + u0];
    int32_t end;
    if (u1 < nc)
      end = off[bin * nc + u1];
    else  // the flat order continues with the next bin (next group after the last block)
      end = (bin + 1 < nbins) ? off[(bin + 1) * nc] : totals[0];
    n = end - start;
  }
  const int32_t nch = (n + kChunkQueries - 1) / kChunkQueries;
  int32_t incl = nch;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int32_t wsum = __shfl(incl, 63);
  int32_t base = 0;
  if (lane == 63 && wsum > 0) base = atomicAdd(&totals[4 + st], wsum);
  base = __shfl(base, 63);
  int4* out = chunks + st * maxc;
  int32_t cs = base + incl - nch;
  for (int32_t j = 0; j < n; j += kChunkQueries, ++cs) {
    const int32_t m = (n - j) < kChunkQueries ? (n - j) : kChunkQueries;
    out[cs] = make_int4(bg_base + g, start + j, m, blk);
  }
}

// ---------------------------------------------------------------------------
// KV-outer attention.  One workgroup per chunk (b, g, block, <= 128 queries):
// the block's K (row-major) and V (transposed) go to LDS once and every
// gathered (query, head) row is processed against them: S^T = K Q^T with keys
// on the MFMA M side (a lane holds 16 keys of one row, so the row max and sum
// are in-register plus one half-wave exchange), softmax in fp32 with exp2,
// P rounded to bf16, O^T = V^T P^T.  Each row writes its unnormalised partial
// O (bf16) and (log2-domain max, sum) for the combine.
//
// LDS rows (keys of K, dims of V^T) are 272 bytes apart: 16 lanes reading the
// same 16-B column of 16 consecutive rows hit distinct banks, and every
// fragment address is a per-lane base plus a constant.  V^T row d holds the
// 128 keys of the block; inside every 16-key group the keys are stored in the
// order 0-3, 8-11, 4-7, 12-15, which is the order in which one half-wave's P
// values reach the PV MFMA's k slots, so each lane's A operand is one 16-B read.
//
// Partial layout ("MFMA order"): the partial of entry E (a (row, slot) pair,
// hg heads) is 256*hg bytes: piece (j, half, head) at byte
// E*256*hg + j*32*hg + (half*hg + head)*16 holds the 8 values
// d = 32*(j/2) + 16*(j%2) + 4*half + {0,1,2,3, 8,9,10,11}, which is what one
// lane holds after the PV MFMAs (j = 0..7 over its 64 accumulators).  Each
// lane thus stores its registers directly, and each store instruction writes
// runs of 32*hg contiguous bytes.
// ---------------------------------------------------------------------------
constexpr int kPitch = 272;  // LDS row pitch of the K and V^T tiles

struct AttnArgs {
  const u16* q;
  const u16* K;
  const u16* V;
  const int4* chunks;     // this launch's chunk list
  const int32_t* entries;
  const int32_t* count;   // number of chunks in the list
  u16* opart;
  float2* lpart;
  int64_t T, N, r0;       // r0: global row (b*T + t) of window row 0
  int32_t Hq, G, NB, k;
  int32_t rl_base;        // first window row of this launch's partial buffer
  int32_t pgroups;        // groups held by the partial buffer (1 for a stage, G for decode)
  int32_t sink;           // spare partial entry (hg rows) that absorbs rows past a chunk's end
};

__device__ __forceinline__ int vt_pos(int key) {
  const int o = key & 15;
  return (key & ~15) + ((o >> 2) & 1) * 8 + ((o >> 3) & 1) * 4 + (o & 3);
}

// NKT: 32-key tiles per block (Bk = 32 * NKT).
template <int HG, int NKT>
__global__ void __launch_bounds__(256, 2) kv_outer_kernel(AttnArgs a) {
  constexpr int BK = 32 * NKT;
  __shared__ __align__(16) unsigned char ks[128 * kPitch];
  __shared__ __align__(16) unsigned char vt[128 * kPitch];
  // Workgroups are dealt to the 8 XCDs round-robin; give XCD x the x-th
  // contiguous eighth of the chunk list, so that the chunks of one KV block
  // (and the rows of one group) share an L2.
  const int nchunks = *a.count;
  const int per_xcd = (nchunks + 7) >> 3;
  const int xj = static_cast<int>(blockIdx.x >> 3);
  const int ci = static_cast<int>(blockIdx.x & 7) * per_xcd + xj;
  if (xj >= per_xcd || ci >= nchunks) return;
  const int4 ch = a.chunks[ci];
  const int n = ch.z;
  if (n <= 0) return;
  const int64_t blk = ch.w;
  const int64_t bg = ch.x;
  const int g = static_cast<int>(bg) & (a.G - 1);  // G is a power of two
  const int64_t b = bg >> __builtin_ctz(a.G);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int64_t key0 = blk * BK;
  const u16* Kb = a.K + (bg * a.N + key0) * kHeadDim;
  const u16* Vb = a.V + (bg * a.N + key0) * kHeadDim;
  // Issue the K/V block loads first; they are written to LDS after the first
  // pass's query rows are on their way.
  uint4 kr[2 * NKT], v0r[NKT], v1r[NKT];
  // Branch-free loads (keys past N re-read the last key and are zeroed) keep
  // the number of outstanding loads fixed for the compiler's wait counting.
  const int nvalid = static_cast<int>(a.N - key0 < BK ? a.N - key0 : BK);
#pragma unroll
  for (int j = 0; j < 2 * NKT; ++j) {
    const int i = tid + j * 256;
    const int r = i >> 4, c = i & 15;
    const uint4 v = ld16(Kb + (r < nvalid ? r : nvalid - 1) * kHeadDim + c * 8);
    kr[j] = r < nvalid ? v : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    const int i = tid + j * 256;
    const int kp = i % (BK / 2), c = i / (BK / 2);  // key pair, 16-B chunk of d
    const int k0 = 2 * kp;
    const uint4 x0 = ld16(Vb + (k0 < nvalid ? k0 : nvalid - 1) * kHeadDim + c * 8);
    const uint4 x1 = ld16(Vb + (k0 + 1 < nvalid ? k0 + 1 : nvalid - 1) * kHeadDim + c * 8);
    v0r[j] = k0 < nvalid ? x0 : make_uint4(0, 0, 0, 0);
    v1r[j] = k0 + 1 < nvalid ? x1 : make_uint4(0, 0, 0, 0);
  }

  // The chunk's entries live in kChunkQueries / 64 registers per lane; a row
  // fetches its entry with lane shuffles.
  constexpr int kEntRegs = kChunkQueries / 64;
  int ent[kEntRegs];
#pragma unroll
  for (int r = 0; r < kEntRegs; ++r)
    ent[r] = lane + 64 * r < n ? a.entries[ch.y + lane + 64 * r] : 0;
  const int rows = n * HG;
  // Window rows are rows t0 .. t0+W-1 of sequence b (r0 = b*T + t0), so a
  // row's query index is t0 + rl and everything fits 32-bit offsets except
  // the q pointer.
  const int64_t t0 = a.r0 - b * a.T;
  // A row's bookkeeping lives in plain scalars (a struct here ends up in
  // scratch memory, whose accesses share the load/store wait counter).
  auto row_of = [&](int pass, bool& valid, int& hh, int& slot, int& rl, int& p, const u16*& q) {
    const int rr = pass * 128 + wave * 32 + l32;
    valid = rr < rows;
    const int qi = valid ? rr / HG : 0;
    int e = __shfl(ent[0], qi & 63);
#pragma unroll
    for (int r = 1; r < kEntRegs; ++r) {
      const int er = __shfl(ent[r], qi & 63);
      if ((qi >> 6) == r) e = er;
    }
    hh = rr % HG;
    rl = e >> 6;
    slot = e & 63;
    const int64_t t = t0 + rl;
    p = static_cast<int>(a.N - a.T + t);
    q = a.q + ((b * a.T + t) * a.Hq + g * HG + hh) * kHeadDim;
  };
  // Rows past the chunk's end load a real row (entry 0) and are never
  // stored, so the loads need no masking: using the data immediately would
  // force a wait right after the prefetch is issued.
  auto load_q = [&](const u16* q, bf16x8 (&qf)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld16(q + 16 * s + 8 * half));
  };

  bool valid;
  int hh, slot, rl, p;
  const u16* qptr;
  row_of(0, valid, hh, slot, rl, p, qptr);
  bf16x8 qf[8];
  load_q(qptr, qf);

#pragma unroll
  for (int j = 0; j < 2 * NKT; ++j) {
    const int i = tid + j * 256;
    *reinterpret_cast<uint4*>(&ks[(i >> 4) * kPitch + (i & 15) * 16]) = kr[j];
  }
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    const int i = tid + j * 256;
    const int kp = i % (BK / 2), c = i / (BK / 2);
    const int P = vt_pos(2 * kp);  // even; key 2*kp + 1 lands at P + 1
    const uint32_t w0[4] = {v0r[j].x, v0r[j].y, v0r[j].z, v0r[j].w};
    const uint32_t w1[4] = {v1r[j].x, v1r[j].y, v1r[j].z, v1r[j].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t hi = (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const int d = 8 * c + e;
      *reinterpret_cast<uint32_t*>(&vt[d * kPitch + 2 * P]) = lo | (hi << 16);
    }
  }
  // Nothing is left in flight past this point, so the waits inside the pass
  // loop only ever count the loop's own loads and stores.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const unsigned char* kbase = ks + l32 * kPitch + half * 16;
  const unsigned char* vbase = vt + l32 * kPitch + half * 16;
  constexpr float kLog2e = 1.4426950408889634f;
  const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  for (int pass = 0; pass * 128 + wave * 32 < rows; ++pass) {
    // S^T = K Q^T, one 32-key tile at a time
    f32x16 sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kbase + kt * 32 * kPitch + s * 32);
        sacc[kt] = s == 0 ? mfma32(as_bf16x8(ka), qf[0], f32x16{})
                          : mfma32(as_bf16x8(ka), qf[s], sacc[kt]);
      }
    }
    sched_fence();
    // the next pass's query rows load while this pass does softmax and PV
    const bool more = (pass + 1) * 128 + wave * 32 < rows;
    bool n_valid = false;
    int n_hh = 0, n_slot = 0, n_rl = 0, n_p = 0;
    const u16* n_q = qptr;
    bf16x8 qn[8];
    if (more) {
      row_of(pass + 1, n_valid, n_hh, n_slot, n_rl, n_p, n_q);
      load_q(n_q, qn);
    }

    // causal mask: only the local block of a row has keys after the row
    const int lim = p - static_cast<int>(key0);  // >= 0: block <= local(row)
    if (__ballot(lim < BK - 1)) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (off > lim) sacc[kt][i] = -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) m = max16(m, sacc[kt]);
    m = halves_max(m);
    const float mc = m * qscale;

    // P = exp2(s * log2e/sqrt(d) - max) rounded to bf16, O^T += V^T P^T.  The
    // V^T fragments of a key tile are read before its exponentials.
    f32x16 oacc[4];
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      uint4 va[4][2];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          va[dt][hf] = *reinterpret_cast<const uint4*>(vbase + dt * 32 * kPitch + kt * 64 + hf * 32);
      uint4 pb[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = fast_exp2(fmaf(sacc[kt][8 * hf + i], qscale, -mc));
          l += pv[i];
        }
        pb[hf] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                            pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        oacc[dt] = kt == 0 ? mfma32(as_bf16x8(va[dt][0]), as_bf16x8(pb[0]), f32x16{})
                           : mfma32(as_bf16x8(va[dt][0]), as_bf16x8(pb[0]), oacc[dt]);
        oacc[dt] = mfma32(as_bf16x8(va[dt][1]), as_bf16x8(pb[1]), oacc[dt]);
      }
    }
    l = halves_sum(l);
    // Unnormalised partial O (bf16, MFMA order) and its (log2-domain max,
    // sum).  Rows past the chunk's end write to the buffer's sink entry;
    // stores are unconditional so that no branch hides them from the wait
    // counting.
    const int prow =
        (valid ? (((rl - a.rl_base) * a.pgroups + (a.pgroups > 1 ? g : 0)) * a.k + slot) * HG
               : a.sink) + hh;
    a.lpart[prow] = make_float2(mc, l);  // both half-waves hold the same values
    u16* dst = a.opart + static_cast<int64_t>(prow - hh) * kHeadDim + (half * HG + hh) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x16& o = oacc[j >> 1];
      const int i0 = 8 * (j & 1);
      uint4 w;
      w.x = pack_bf16x2(o[i0 + 0], o[i0 + 1]);
      w.y = pack_bf16x2(o[i0 + 2], o[i0 + 3]);
      w.z = pack_bf16x2(o[i0 + 4], o[i0 + 5]);
      w.w = pack_bf16x2(o[i0 + 6], o[i0 + 7]);
      *reinterpret_cast<uint4*>(dst + j * 16 * HG) = w;
    }
    if (more) {
      valid = n_valid;
      hh = n_hh;
      slot = n_slot;
      rl = n_rl;
      p = n_p;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = qn[s];
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: one wave per (row, group).  The valid slots are the leading
// non-negative entries of the row's idx; their partials are merged with
// weights exp(lse_i - max lse) in slot order, so the result does not depend
// on the order in which the chunks ran.
// ---------------------------------------------------------------------------
struct CombArgs {
  const int32_t* idx;
  const u16* opart;
  const float2* lpart;
  u16* O;
  float* lse;
  int64_t T, r0;     // r0: global row of window row 0
  int64_t rows;      // rows combined by this launch (window rows rl_base ..)
  int32_t Hq, G, k;
  int32_t rl_base;
  int32_t group;     // the stage's group, or -1: every group (decode)
  int32_t pgroups;   // groups held by the partial buffer
};

// WIDE: more than 16 slots (k <= 64): the row max first, then the partials
// 16 slots at a time.
template <int HG, bool WIDE>
__global__ void __launch_bounds__(256) combine_kernel(CombArgs a) {
  // A row's partial is 16 pieces of 8 values per head (MFMA order, see the
  // KV-outer kernel); a lane takes PPL consecutive pieces of one head.
  constexpr int LPH = HG >= 4 ? 64 / HG : 16;  // lanes per head
  constexpr int PPL = 16 / LPH;                // pieces per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int gper = a.group >= 0 ? 1 : a.G;
  if (wid >= a.rows * gper) return;
  const int64_t rl = wid / gper;  // row inside this launch's partial buffer
  const int g = a.group >= 0 ? a.group : static_cast<int>(wid % gper);
  const int64_t grow = a.r0 + a.rl_base + rl;
  const int64_t b = grow / a.T, t = grow % a.T;
  const int32_t* ir = a.idx + ((b * a.G + g) * a.T + t) * a.k;
  const bool sv = lane < a.k && ir[lane < a.k ? lane : 0] >= 0;
  const int nval = __popcll(__ballot(sv));
  // lanes past HG * LPH (only when HG < 4) take head 0's pieces and store nothing
  const bool active = lane < HG * LPH;
  const int hh = active ? lane / LPH : 0;
  const int li = lane % LPH;
  const int64_t pbase = (rl * a.pgroups + (a.pgroups > 1 ? g : 0)) * a.k;

  float mx = -INFINITY;
  if constexpr (WIDE) {
    for (int s = 0; s < nval; ++s) mx = fmaxf(mx, a.lpart[(pbase + s) * HG + hh].x);
  }
  float acc[PPL][8];
#pragma unroll
  for (int q = 0; q < PPL; ++q)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[q][u] = 0.f;
  float den = 0.f;
  // One pass over 16 slots (WIDE: as many as the row has), all loaded at
  // once (slots past nval re-read slot 0 and get weight 0) so that every lane
  // has them in flight.
  for (int s0 = 0; s0 < (WIDE ? nval : 1); s0 += 16) {
    // every load is issued before any is used (a use right after a load
    // makes the compiler wait for it there)
    float2 ml[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int ss = s0 + s < nval ? s0 + s : 0;
      ml[s] = a.lpart[(pbase + ss) * HG + hh];
    }
    uint4 raw[16][PPL];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int ss = s0 + s < nval ? s0 + s : 0;
      const u16* src = a.opart + (pbase + ss) * HG * kHeadDim;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int pc = li * PPL + q, j = pc >> 1, hf = pc & 1;
        raw[s][q] = ld16_once(src + j * 16 * HG + (hf * HG + hh) * 8);
      }
    }
    sched_fence();  // keep the uses below the loads
    if constexpr (!WIDE) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < nval) mx = fmaxf(mx, ml[s].x);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float w = s0 + s < nval ? fast_exp2(ml[s].x - mx) : 0.f;
      den += w * ml[s].y;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const uint32_t wv[4] = {raw[s][q].x, raw[s][q].y, raw[s][q].z, raw[s][q].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc[q][2 * u] += w * __uint_as_float(wv[u] << 16);
          acc[q][2 * u + 1] += w * __uint_as_float(wv[u] & 0xffff0000u);
        }
      }
    }
  }
  const float inv = 1.f / den;
  u16* dst = a.O + ((b * a.T + t) * a.Hq + g * HG + hh) * kHeadDim;
  if (active) {
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      // piece (j, hf): values 0-3 at d0, 4-7 at d0 + 8
      const int pc = li * PPL + q, j = pc >> 1, hf = pc & 1;
      const int d0 = 32 * (j >> 1) + 16 * (j & 1) + 4 * hf;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        uint2 w;
        w.x = pack_bf16x2(acc[q][4 * r + 0] * inv, acc[q][4 * r + 1] * inv);
        w.y = pack_bf16x2(acc[q][4 * r + 2] * inv, acc[q][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(dst + d0 + 8 * r) = w;
      }
    }
  }
  // lse in natural log: (max + log2(sum)) * ln 2, the max being log2-domain
  if (a.lse && active && li == 0)
    a.lse[(b * a.Hq + g * HG + hh) * a.T + t] = (mx + __log2f(den)) * 0.6931471805599453f;
}

// ---------------------------------------------------------------------------
template <int HG, int NKT>
static hipError_t launch_kv_combine(const AttnArgs& aa, const CombArgs& ca, int64_t grid_chunks,
                                    hipStream_t st) {
  const int64_t grid = (grid_chunks + 7) & ~static_cast<int64_t>(7);
  {
    TimedLaunch tl(MSA_KERNEL_KV_OUTER, st);
    hipLaunchKernelGGL((kv_outer_kernel<HG, NKT>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, st, aa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = ca.rows * (ca.group >= 0 ? 1 : ca.G);
  TimedLaunch tl(MSA_KERNEL_COMBINE, st);
  if (ca.k > 16)
    hipLaunchKernelGGL((combine_kernel<HG, true>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(256), 0, st, ca);
  else
    hipLaunchKernelGGL((combine_kernel<HG, false>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(256), 0, st, ca);
  return hipGetLastError();
}

template <int NKT>
static hipError_t dispatch_hg_t(int hg, const AttnArgs& aa, const CombArgs& ca, int64_t grid,
                                hipStream_t st) {
  switch (hg) {
    case 8: return launch_kv_combine<8, NKT>(aa, ca, grid, st);
    case 4: return launch_kv_combine<4, NKT>(aa, ca, grid, st);
    case 16: return launch_kv_combine<16, NKT>(aa, ca, grid, st);
    case 2: return launch_kv_combine<2, NKT>(aa, ca, grid, st);
    case 1: return launch_kv_combine<1, NKT>(aa, ca, grid, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch_hg(int hg, int Bk, const AttnArgs& aa, const CombArgs& ca,
                              int64_t grid, hipStream_t st) {
  switch (Bk) {
    case 128: return dispatch_hg_t<4>(hg, aa, ca, grid, st);
    case 64: return dispatch_hg_t<2>(hg, aa, ca, grid, st);
    case 32: return dispatch_hg_t<1>(hg, aa, ca, grid, st);
  }
  return hipErrorInvalidValue;
}

static unsigned blocks_for(int64_t n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

// Inversion of the query rows [t0, t0 + W) of sequence b (unit histograms,
// scan, scatter, stage chunk lists); *nsub receives the number of row stages
// per group.
hipError_t launch_invert_window(const int32_t* idx, int64_t b, int64_t T, int64_t t0, int64_t W,
                                int64_t N, int G, int k, int Bk, const AttnWorkspace& w,
                                int32_t* nsub, hipStream_t st) {
  const int32_t NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  const size_t lds = sizeof(int32_t) * NB;
  InvArgs ia;
  ia.idx = idx;
  ia.hist = w.hist;
  ia.entries = w.entries;
  ia.T = T;
  ia.t0 = t0;
  ia.W = W;
  ia.b = static_cast<int32_t>(b);
  ia.G = G;
  ia.k = k;
  ia.NB = NB;
  ia.rq = w.rq;
  ia.nc = static_cast<int32_t>((W + w.rq - 1) / w.rq);
  const int64_t nhist = static_cast<int64_t>(G) * NB * ia.nc;
  const int64_t ntiles = (nhist + kScanTile - 1) / kScanTile;
  const int32_t S = static_cast<int32_t>((W + w.stage_rows - 1) / w.stage_rows);
  const int32_t U = static_cast<int32_t>(w.stage_rows / w.rq);
  const int64_t nst = static_cast<int64_t>(G) * S;
  const dim3 ugrid(static_cast<unsigned>(ia.nc), static_cast<unsigned>(G));
  TimedLaunch tl(MSA_KERNEL_INVERT, st);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(nst, 256)), dim3(256), 0, st,
                     w.totals + 4, nst, 0);
  hipLaunchKernelGGL(hist_kernel, ugrid, dim3(256), lds, st, ia);
  hipLaunchKernelGGL(scan_tiles_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, st,
                     w.hist, nhist, w.tile_sums);
  hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(256), 0, st, w.tile_sums, ntiles,
                     w.totals);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, st,
                     w.hist, nhist, w.tile_sums);
  hipLaunchKernelGGL(scatter_kernel, ugrid, dim3(256), lds, st, ia);
  const int64_t per_stage = ((NB + 63) / 64) * 64;
  hipLaunchKernelGGL(stage_chunk_kernel, dim3(blocks_for(nst * per_stage, 256)), dim3(256), 0,
                     st, w.hist, w.totals, w.chunks, NB, static_cast<int64_t>(G) * NB, ia.nc,
                     U, S, w.max_chunks, static_cast<int32_t>(b * G));
  *nsub = S;
  return hipGetLastError();
}

// Prefill: for every sequence and every window of its rows, one inversion;
// then the stages in group-major order.  A stage is one group and
// stage_rows consecutive rows: its KV-outer launch writes the stage's
// partials (a buffer small enough to stay in the last-level cache next to
// the group's K/V) and the combine launch right after reads them back.
hipError_t launch_attn_prefill(const void* q, const void* K, const void* V,
                               const int32_t* idx, void* O, float* lse, int64_t B,
                               int64_t T, int64_t N, int Hq, int G, int k, int Bk,
                               const AttnWorkspace& w, hipStream_t st) {
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t0 = 0; t0 < T; t0 += w.window) {
      const int64_t W = (T - t0) < w.window ? (T - t0) : w.window;
      const hipError_t e =
          launch_attn_prefill_rows(q, K, V, idx, O, lse, b, T, t0, W, N, Hq, G, k, Bk, w, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_attn_prefill_rows(const void* q, const void* K, const void* V,
                                    const int32_t* idx, void* O, float* lse, int64_t b,
                                    int64_t T, int64_t t0, int64_t W, int64_t N, int Hq, int G,
                                    int k, int Bk, const AttnWorkspace& w, hipStream_t st) {
  const int hg = Hq / G;
  const int32_t NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  int32_t S = 0;
  hipError_t e = launch_invert_window(idx, b, T, t0, W, N, G, k, Bk, w, &S, st);
  if (e != hipSuccess) return e;
  const int64_t r0 = b * T + t0;
  for (int g = 0; g < G; ++g) {
    for (int32_t sub = 0; sub < S; ++sub) {
      const int64_t si = static_cast<int64_t>(g) * S + sub;
      const int32_t rl_base = sub * static_cast<int32_t>(w.stage_rows);
      const int64_t rows = (W - rl_base) < w.stage_rows ? (W - rl_base) : w.stage_rows;
      AttnArgs aa;
      aa.q = static_cast<const u16*>(q);
      aa.K = static_cast<const u16*>(K);
      aa.V = static_cast<const u16*>(V);
      aa.chunks = w.chunks + si * w.max_chunks;
      aa.entries = w.entries;
      aa.count = w.totals + 4 + si;
      aa.opart = w.opart;
      aa.lpart = w.lpart;
      aa.T = T;
      aa.N = N;
      aa.r0 = r0;
      aa.Hq = Hq;
      aa.G = G;
      aa.NB = NB;
      aa.k = k;
      aa.rl_base = rl_base;
      aa.pgroups = 1;
      aa.sink = static_cast<int32_t>(w.sink);
      CombArgs ca;
      ca.idx = idx;
      ca.opart = w.opart;
      ca.lpart = w.lpart;
      ca.O = static_cast<u16*>(O);
      ca.lse = lse;
      ca.T = T;
      ca.r0 = r0;
      ca.rows = rows;
      ca.Hq = Hq;
      ca.G = G;
      ca.k = k;
      ca.rl_base = rl_base;
      ca.group = g;
      ca.pgroups = 1;
      e = dispatch_hg(hg, Bk, aa, ca, w.max_chunks, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Stages 1-4 of a prefill, one window of query rows after another.  The
// selection of window i runs on st; an event hands its rows to st2, where
// their attention (inversion, KV-outer stages, combines) runs while st goes on
// with the selection of window i + 1.  The selection is MFMA-bound and moves
// little memory; the attention is bound by the memory traffic of its gathers
// and partial results, so the two overlap on the chip.  st2 == st runs the
// same launches in order on one stream.  ev: nwin + 1 events.
// Workgroups (one per CU: 128 KB of LDS, 8 waves of 256 registers) of the
// fused select's own launches while an attention window runs beside them.
#ifndef MSA_PIPE_SELECT_WGS
#define MSA_PIPE_SELECT_WGS 128
#endif
constexpr int kPipeSelectWGs = MSA_PIPE_SELECT_WGS;

// Window boundaries of the pipelined prefill: windows of `win` rows, the
// last one (unless it is the only one) cut in two halves: its attention runs
// alone, after the last selection, so a shorter one costs less.  Returns the
// number of windows.
int prefill_windows(int64_t T, int64_t win, int64_t* bounds, int max_windows) {
  int n = 0;
  bounds[0] = 0;
  for (int64_t t0 = 0; t0 < T && n < max_windows; t0 += win) {
    const int64_t t1 = t0 + win < T ? t0 + win : T;
    if (t1 == T && t0 > 0 && t1 - t0 >= 8192 && n + 2 <= max_windows)
      bounds[++n] = t0 + (t1 - t0) / 2;
    bounds[++n] = t1;
  }
  return n;
}

// Stages 1-4 of a prefill, one window of query rows after another.  The
// selection is MFMA-bound and moves little memory; the attention is bound by
// the memory traffic of its gathers and partial results, so the two are run
// side by side: window i's attention (inversion, KV-outer stages, combines)
// on st2 while st selects the windows after it.  A fused-select workgroup
// fills a CU by itself, so left alone its workgroups would take every CU an
// attention launch frees and the two would merely alternate; instead each
// window's selection is launched twice over one item counter: on st with at
// most kPipeSelectWGs workgroups (the first window: no cap), and on st2 right
// after the attention of the window before, uncapped, to take whatever items
// are left once that attention is done.  Either launch may find the counter
// exhausted.  With Bk < 128 (scores materialised window by window, then
// ranked) and with st2 == st every launch runs in order on one stream.
hipError_t launch_prefill_pipelined(const void* qI, const void* kI, const void* q, const void* K,
                                    const void* V, int32_t* idx, void* O, float* lse, int64_t B,
                                    int64_t T, int64_t N, int Hq, int G, int k, int Bk,
                                    int64_t win, float* S, int64_t srows, int32_t* counters,
                                    const AttnWorkspace& w, hipStream_t st, hipStream_t st2,
                                    hipEvent_t* ev, int nev) {
  int64_t bounds[kMaxPrefillWindows + 1];
  const int maxw = nev - 1 < kMaxPrefillWindows ? nev - 1 : kMaxPrefillWindows;
  const int nwin = prefill_windows(T, win, bounds, maxw);
  if (bounds[nwin] != T) return hipErrorInvalidValue;
  if (nwin == 1) st2 = st;  // nothing to overlap
  hipError_t e = hipSuccess;
  auto attend = [&](int i, hipStream_t s) {
    hipError_t r = hipSuccess;
    for (int64_t b = 0; b < B && r == hipSuccess; ++b)
      r = launch_attn_prefill_rows(q, K, V, idx, O, lse, b, T, bounds[i],
                                   bounds[i + 1] - bounds[i], N, Hq, G, k, Bk, w, s);
    return r;
  };
  if (Bk != 128 || st2 == st) {
    for (int i = 0; i < nwin && e == hipSuccess; ++i) {
      const int64_t t0 = bounds[i], Tw = bounds[i + 1] - bounds[i];
      if (Bk == 128) {
        e = launch_index_tiles(false, false, qI, kI, nullptr, idx, B, T, t0, Tw, N, G, 128, k,
                               st);
      } else {
        for (int64_t s0 = t0; s0 < t0 + Tw && e == hipSuccess; s0 += srows) {
          const int64_t n = (t0 + Tw - s0) < srows ? (t0 + Tw - s0) : srows;
          e = launch_index_tiles(true, false, qI, kI, S, nullptr, B, T, s0, n, N, G, Bk, k, st);
          if (e == hipSuccess) {
            const PagedCache none = {nullptr, nullptr, 0, 0};
            e = launch_topk_rows(S, idx, B, T, s0, n, N, G, Bk, k, none, st);
          }
        }
      }
      if (e == hipSuccess && st2 != st) {
        e = hipEventRecord(ev[i], st);
        if (e == hipSuccess) e = hipStreamWaitEvent(st2, ev[i], 0);
      }
      if (e == hipSuccess) e = attend(i, st2);
    }
  } else {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, counters,
                       static_cast<int64_t>(nwin), 0);
    e = hipGetLastError();
    for (int i = 0; i < nwin && e == hipSuccess; ++i) {
      e = launch_index_tiles(false, false, qI, kI, nullptr, idx, B, T, bounds[i],
                             bounds[i + 1] - bounds[i], N, G, 128, k, st,
                             i == 0 ? 0 : kPipeSelectWGs, counters + i);
      if (e == hipSuccess) e = hipEventRecord(ev[i], st);
    }
    for (int i = 0; i < nwin && e == hipSuccess; ++i) {
      e = hipStreamWaitEvent(st2, ev[i], 0);
      if (e == hipSuccess) e = attend(i, st2);
      if (e == hipSuccess && i + 1 < nwin)
        e = launch_index_tiles(false, false, qI, kI, nullptr, idx, B, T, bounds[i + 1],
                               bounds[i + 2] - bounds[i + 1], N, G, 128, k, st2, 0,
                               counters + i + 1);
    }
  }
  if (e == hipSuccess && st2 != st) {
    e = hipEventRecord(ev[nwin], st2);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, ev[nwin], 0);
  }
  return e;
}

// ---------------------------------------------------------------------------
// Decode attention: one wave per (sequence, group, slot).  With one query per
// sequence there is nothing to gather, so K is read straight from HBM as the
// A operand of 16x16x32 MFMAs (16 keys x the hg heads of the group, padded to
// 16 columns); V goes through 32 KB of LDS, transposed, for O^T = V^T P^T.
// Inside each 32-key k-step the keys sit in the order the P fragments reach
// the MFMA's k slots (lane quarter qd holds keys 4qd..4qd+3 of both 16-key
// tiles), so every A fragment is one 16-B LDS read.  Writes the slot's
// unnormalised partial O and (log2-domain max, sum) for the combine.
// ---------------------------------------------------------------------------
struct DecArgs {
  const u16* q;        // [B, Hq, 128]
  const u16* K;        // [B, G, N, 128], or the page pool [pages, G, 128, 128] when paged
  const u16* V;
  const int32_t* idx;  // [B, G, 1, k]
  u16* opart;          // [B, G, k, hg, 128]
  float2* lpart;       // [B, G, k, hg]
  int64_t N;           // cache capacity (tokens)
  int32_t Hq, G, k, Bk;
  PagedCache pc;
};

// Key offset 0..31 within a wave's quarter -> its column in that wave's V^T
// rows, matching the k order of the P^T operand (lane quarter qd holds keys
// 4qd..4qd+3 of both 16-key score tiles).
__device__ __forceinline__ int dec_pos(int key) {
  return 8 * ((key & 15) >> 2) + 4 * (key >> 4) + (key & 3);
}

// V^T byte offset of (d, 16-byte chunk c) in a wave's 8 KB region: 64-byte
// rows, chunk index xor-ed with (d >> 2) so that the 8 lanes of one LDS read
// phase (consecutive d) hit distinct banks.
__device__ __forceinline__ int dec_vt(int d, int c) { return d * 64 + ((c ^ (d >> 2)) & 3) * 16; }

// One workgroup of four waves per (sequence, group, selected block); wave w
// takes keys 32w..32w+31 of the block.  Each wave: K rows straight from HBM as
// the A operand of 16x16x32 MFMAs (keys on M, the group's heads on N), its own
// max / sum, V^T of its 32 keys through 8 KB of LDS, and a PV product over its
// keys.  The four (max, sum, O) meet in LDS (log-sum-exp merge) and the
// workgroup writes one unnormalised partial per head, like a prefill slot.
template <int HG>
__global__ void __launch_bounds__(256) decode_attn_kernel(DecArgs a) {
  __shared__ __align__(16) unsigned char lds[32768];  // V^T, then the O merge
  __shared__ float wm[4][16], wl[4][16];
  const int64_t item = blockIdx.x;  // (b * G + g) * k + slot
  const int slot = static_cast<int>(item % a.k);
  const int64_t bg = item / a.k;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int blk = a.idx[bg * a.k + slot];
  const int64_t len = paged_len(a.pc, b, a.N);  // this sequence's cache length
  if (blk < 0 || static_cast<int64_t>(blk) * a.Bk >= len) return;  // unused slot
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int64_t kblk = static_cast<int64_t>(blk) * a.Bk;
  // keys of the block inside the sequence (>= 1); loads clamp to the last of
  // them, and this wave's quarter holds nvalid of them (<= 0: none)
  const int nblk = static_cast<int>(len - kblk < a.Bk ? len - kblk : a.Bk);
  const int nvalid = nblk - 32 * wave < 32 ? nblk - 32 * wave : 32;
  const int64_t row0 = a.pc.table ? (paged_page(a.pc, b, blk) * a.G + g) * kBlock
                                  : bg * a.N + kblk;  // first key row of the block
  const u16* Kb = a.K + row0 * kHeadDim;
  const u16* Vb = a.V + row0 * kHeadDim;
  auto krow = [&](int kk) { return (32 * wave + kk < nblk ? 32 * wave + kk : nblk - 1) * kHeadDim; };
  unsigned char* vt = lds + wave * 8192;

  // issue every load: V (4 tasks of a key pair x 8 d), K (2 tiles x 4 k-steps), q
  uint4 v0[4], v1[4], kf[2][4], qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tsk = lane + 64 * j;  // 0..255
    const int kp = tsk & 15, c = tsk >> 4;
    const int k0 = 2 * kp;
    v0[j] = ld16(Vb + krow(k0) + c * 8);
    v1[j] = ld16(Vb + krow(k0 + 1) + c * 8);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 16 * t + col;
    const u16* kr = Kb + krow(key) + 8 * qd;
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[t][s] = ld16(kr + 32 * s);
  }
  const u16* qr = a.q + (b * a.Hq + g * HG + (col < HG ? col : 0)) * kHeadDim + 8 * qd;
#pragma unroll
  for (int s = 0; s < 4; ++s) qv[s] = ld16(qr + 32 * s);

  // V -> V^T: key pair (k0, k0 + 1) x d = 8c..8c+7, one 32-bit word per d
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tsk = lane + 64 * j;
    const int kp = tsk & 15, c = tsk >> 4;
    const int k0 = 2 * kp;
    const int P = dec_pos(k0);  // even; key k0 + 1 lands at P + 1
    const uint32_t w0[4] = {v0[j].x, v0[j].y, v0[j].z, v0[j].w};
    const uint32_t w1[4] = {v1[j].x, v1[j].y, v1[j].z, v1[j].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = k0 < nvalid ? (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu : 0u;
      const uint32_t hi = k0 + 1 < nvalid ? (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu : 0u;
      const int d = 8 * c + e;
      *reinterpret_cast<uint32_t*>(&vt[dec_vt(d, P >> 3) + 2 * (P & 7)]) = lo | (hi << 16);
    }
  }

  // S^T tiles: lane holds head `col`, keys 16t + 4qd + r
  f32x4 sc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sc[t] = f32x4{};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sc[t] = mfma16(as_bf16x8(kf[t][s]), as_bf16x8(col < HG ? qv[s] : make_uint4(0, 0, 0, 0)),
                     sc[t]);
  }
  constexpr float qscale = 1.4426950408889634f * 0.08838834764831845f;
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (16 * t + 4 * qd + r >= nvalid) sc[t][r] = -INFINITY;
      m = fmaxf(m, sc[t][r]);
    }
  m = quads_max(m);
  const float mc = m == -INFINITY ? 0.f : m * qscale;  // all-masked quarter: p = 0
  float pv[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = fast_exp2(fmaf(sc[0][r], qscale, -mc));
    pv[4 + r] = fast_exp2(fmaf(sc[1][r], qscale, -mc));
  }
  float l = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) l += pv[e];
  l = quads_sum(l);
  const uint4 pf = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                              pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // O^T tiles: lane holds head `col`, d = 16dt + 4qd + r
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint4 av = *reinterpret_cast<const uint4*>(&vt[dec_vt(16 * dt + col, qd)]);
    o[dt] = mfma16(as_bf16x8(av), as_bf16x8(pf), f32x4{});
  }
  if (qd == 0) {
    wm[wave][col] = m == -INFINITY ? -INFINITY : mc;
    wl[wave][col] = l;
  }
  __syncthreads();  // every wave is done with its V^T; the merge reuses the LDS
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][col]);
  const float sw = fast_exp2(wm[wave][col] - M);  // 0 for an all-masked quarter
  float* red = reinterpret_cast<float*>(lds);  // [4][HG][128]
  if (col < HG) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&red[(wave * HG + col) * kHeadDim + 16 * dt + 4 * qd]) =
          o[dt] * sw;
  }
  __syncthreads();
  // the partial in MFMA order (the layout the KV-outer kernel writes): d0's
  // four values sit in piece (j, half) at value offset t0
  const int64_t prow0 = (bg * a.k + slot) * HG;
  for (int e = threadIdx.x; e < HG * 32; e += 256) {
    const int h = e >> 5, d0 = 4 * (e & 31);
    f32x4 acc = *reinterpret_cast<const f32x4*>(&red[h * kHeadDim + d0]);
#pragma unroll
    for (int w = 1; w < 4; ++w)
      acc += *reinterpret_cast<const f32x4*>(&red[(w * HG + h) * kHeadDim + d0]);
    uint2 st;
    st.x = pack_bf16x2(acc[0], acc[1]);
    st.y = pack_bf16x2(acc[2], acc[3]);
    const int dw = d0 & 31;
    const int j = 2 * (d0 >> 5) + (dw >> 4), hf = (dw >> 2) & 1, t0 = 4 * ((dw >> 3) & 1);
    *reinterpret_cast<uint2*>(a.opart + prow0 * kHeadDim + j * 16 * HG + (hf * HG + h) * 8 + t0) = st;
  }
  if (threadIdx.x < HG) {
    const int h = threadIdx.x;
    float Mh = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, wm[w][h]);
#pragma unroll
    for (int w = 0; w < 4; ++w) L += wl[w][h] * fast_exp2(wm[w][h] - Mh);
    a.lpart[prow0 + h] = make_float2(Mh, L);
  }
}

// Decode combine: one wave per (sequence, group, head), so that the batch's
// few rows still spread over many waves.  Lane l takes piece l % 16 of the
// head's partial (8 values, MFMA order as written by decode_attn_kernel) in
// the slots s = l / 16 + 4i, i = 0..NSL-1; the four slot groups are then
// summed across the wave.  O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// over the row's valid slots, M = max m_s.
template <int HG, int NSL>
__global__ void __launch_bounds__(256) decode_combine_kernel(CombArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wid >= a.rows * a.G * HG) return;
  const int h = static_cast<int>(wid % HG);
  const int64_t bg = wid / HG;  // b * G + g
  const int64_t b = bg / a.G;
  const int g = static_cast<int>(bg % a.G);
  const int32_t* ir = a.idx + bg * a.k;
  const int nval = __popcll(__ballot(lane < a.k && ir[lane < a.k ? lane : 0] >= 0));
  const int pc = lane & 15, sg = lane >> 4;
  const int j = pc >> 1, hf = pc & 1;
  float2 ml[NSL];
  uint4 raw[NSL];
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int sl = sg + 4 * i;
    const int64_t e = bg * a.k + (sl < nval ? sl : 0);  // entry (b, g, slot)
    ml[i] = a.lpart[e * HG + h];
    raw[i] = ld16_once(a.opart + e * HG * kHeadDim + j * 16 * HG + (hf * HG + h) * 8);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    if (sg + 4 * i < nval) mx = fmaxf(mx, ml[i].x);
  mx = quads_max(mx);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const float w = sg + 4 * i < nval ? fast_exp2(ml[i].x - mx) : 0.f;
    den += w * ml[i].y;
    const uint32_t wv[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] += w * __uint_as_float(wv[u] << 16);
      acc[2 * u + 1] += w * __uint_as_float(wv[u] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    acc[u] = quads_sum(acc[u]);
  }
  den = quads_sum(den);
  const int hq = g * HG + h;
  if (sg == 0) {
    const float inv = 1.f / den;
    // piece (j, hf): values 0-3 at d0, 4-7 at d0 + 8
    const int d0 = 32 * (j >> 1) + 16 * (j & 1) + 4 * hf;
    u16* dst = a.O + (b * a.Hq + hq) * kHeadDim + d0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint2 w;
      w.x = pack_bf16x2(acc[4 * r + 0] * inv, acc[4 * r + 1] * inv);
      w.y = pack_bf16x2(acc[4 * r + 2] * inv, acc[4 * r + 3] * inv);
      *reinterpret_cast<uint2*>(dst + 8 * r) = w;
    }
  }
  // lse in natural log: (max + log2(sum)) * ln 2, the max being log2-domain
  if (a.lse && lane == 0) a.lse[b * a.Hq + hq] = (mx + __log2f(den)) * 0.6931471805599453f;
}

// ---------------------------------------------------------------------------
// One-call decode step, after the index-key scan.  Each (sequence, group) row
// is split over SPLIT workgroups of eight waves (SPLIT = 2 while the batch has
// fewer than 256 rows, so that every CU streams K / V).  In each workgroup,
// waves 0-3 select the row's blocks from its block scores (the four-wave
// top-k of the decode selection; the first workgroup of the row writes idx).
// Then wave w takes the slots h + SPLIT (w + 8i) of the row (h: the
// workgroup's part) and each of their 32-key quarters in turn: K rows
// straight from HBM as the A operand of 16x16x32 MFMAs (keys x the group's
// heads), V^T of the quarter through the wave's 8 KB of LDS (the layout of
// decode_attn_kernel), and an online softmax per head: a running log2-domain
// max and sum, the O accumulators rescaled before each PV product.  The next
// quarter's K and V load while the current one is computed.  The waves'
// (max, sum, O) meet in LDS; with SPLIT = 1 the workgroup writes O and lse,
// with SPLIT = 2 each part writes its fp32 (max, sum, O) and a small combine
// merges the two.  No bf16 partials leave the chip.
// ---------------------------------------------------------------------------
struct StepArgs {
  const float* S;  // [B, G, NB] block scores
  const u16* q;    // [B, Hq, 128]
  const u16* K;    // [B, G, N, 128], or the page pool [pages, G, 128, 128] when paged
  const u16* V;
  int32_t* idx;    // [B, G, 1, k], written
  u16* O;          // [B, Hq, 128]
  float* lse;      // [B, Hq], natural log, or null
  float* part;     // SPLIT > 1: [B * G, SPLIT, hg, 128] fp32 unnormalised O of each part
  float2* ml;      // SPLIT > 1: [B * G, SPLIT, hg] (log2-domain max, sum)
  int64_t N;       // cache capacity (tokens)
  int32_t Hq, G, k, Bk, NB;
  PagedCache pc;
};

// One quarter's operands: K as MFMA A fragments (2 tiles of 16 keys x 4
// k-steps) and V as key pairs x 8 dims (4 tasks per lane).
struct StepQuarter {
  uint4 kf[2][4];
  uint4 v0[4], v1[4];
};

// Waves per workgroup of the step kernel; a part's (slot, quarter) items are
// dealt to them round-robin (four per wave for 16 slots in two parts).
// Measured per decode step at 256K x 16: 8 waves 216.8 us, 16 waves (two
// items each, 128 VGPRs) 218.1 us; 4 parts of 8 or 16 waves 227.0 / 230.1 us;
// one workgroup per row 223.7 us.
#ifndef MSA_STEP_WAVES
#define MSA_STEP_WAVES 8
#endif
constexpr int kStepWaves = MSA_STEP_WAVES;
// Parts per row below kStepSplitRows rows.
#ifndef MSA_STEP_PARTS
#define MSA_STEP_PARTS 2
#endif
constexpr int kStepParts = MSA_STEP_PARTS;

template <int HG, int SPLIT>
__global__ void __launch_bounds__(64 * kStepWaves) decode_step_kernel(StepArgs a) {
  constexpr int NW = kStepWaves;
  __shared__ WideTopkLds tk;
  __shared__ int sel[64];
  __shared__ __align__(16) unsigned char lds[NW * 8192];  // V^T per wave, then the O merge
  __shared__ __align__(16) uint4 qs[4][64];                // the heads' q fragments
  __shared__ float wm[NW][16], wl[NW][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int64_t bg = blockIdx.x / SPLIT;
  const int h = static_cast<int>(blockIdx.x % SPLIT);
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t len = paged_len(a.pc, b, a.N);  // this sequence's cache length (>= 1)
  const int L = static_cast<int>((len - 1) / a.Bk);  // the local block
  const int m = L < a.k - 1 ? L : a.k - 1;          // blocks chosen besides it

  // selection: the best m of blocks 0..L-1, then L, then -1 padding; waves
  // 4-7 fetch the q fragments meanwhile
  if (m == 0) {
    if (threadIdx.x < a.k) sel[threadIdx.x] = threadIdx.x == 0 ? L : -1;
  } else if (wave < 4) {
    wide_topk_part1(a.S + bg * a.NB, L, m, lane, wave, tk);
  }
  if (wave >= 4 && wave < 8) {
    const int s = wave - 4;
    const u16* qr = a.q + (b * a.Hq + g * HG + (col < HG ? col : 0)) * kHeadDim + 8 * qd;
    qs[s][lane] = col < HG ? ld16(qr + 32 * s) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  if (m > 0 && wave == 0) {
    const int v = wide_topk_part2(L, m, lane, tk);
    if (lane < a.k) sel[lane] = v;
  }
  __syncthreads();
  if (h == 0 && threadIdx.x < a.k) a.idx[bg * a.k + threadIdx.x] = sel[threadIdx.x];

  // this part's items: its valid slots h, h + SPLIT, ... <= m times Bk / 32
  // quarters; wave w takes items w, w + NW, ...
  const int nq = a.Bk >> 5;
  const int ns = h <= m ? (m - h) / SPLIT + 1 : 0;
  const int nitems = ns * nq;
  const int mine = wave < nitems ? (nitems - wave + NW - 1) / NW : 0;
  unsigned char* vt = lds + wave * 8192;
  // V^T store bases of this lane (see the store loop)
  const int Pv = dec_pos(2 * col);
  const int vb0 = 8 * qd * 64 + (((Pv >> 3) ^ (2 * qd)) & 3) * 16 + 2 * (Pv & 7);
  const int vb1 = 8 * qd * 64 + (((Pv >> 3) ^ (2 * qd + 1)) & 3) * 16 + 2 * (Pv & 7);
  // geometry of this wave's j-th item: its quarter's first K / V rows and its
  // valid keys (keys past the block's end re-read its last key, masked below)
  auto item = [&](int j, const u16*& Kq, const u16*& Vq, int& nv) {
    const int it = wave + NW * j;
    const int s = h + SPLIT * (it / nq);
    const int qq = it % nq;
    const int blk = sel[s];
    const int64_t kblk = static_cast<int64_t>(blk) * a.Bk;
    const int nblk = static_cast<int>(len - kblk < a.Bk ? len - kblk : a.Bk);
    const int64_t row0 = a.pc.table ? (paged_page(a.pc, b, blk) * a.G + g) * kBlock
                                    : bg * a.N + kblk;
    nv = nblk - 32 * qq < 32 ? nblk - 32 * qq : 32;
    const int first = 32 * qq < nblk ? 32 * qq : nblk - 1;
    Kq = a.K + (row0 + first) * kHeadDim;
    Vq = a.V + (row0 + first) * kHeadDim;
  };
  auto load_k = [&](StepQuarter& x, const u16* Kq, int nv) {
    const int lim = nv > 0 ? nv - 1 : 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = 16 * t + col;
      const u16* kr = Kq + (key < lim ? key : lim) * kHeadDim + 8 * qd;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) x.kf[t][s4] = ld16(kr + 32 * s4);
    }
  };
  auto load_v = [&](StepQuarter& x, const u16* Vq, int nv) {
    const int lim = nv > 0 ? nv - 1 : 0;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int k0 = 2 * col, c = qd + 4 * j4;
      x.v0[j4] = ld16(Vq + (k0 < lim ? k0 : lim) * kHeadDim + c * 8);
      x.v1[j4] = ld16(Vq + (k0 + 1 < lim ? k0 + 1 : lim) * kHeadDim + c * 8);
    }
  };

  constexpr float qscale = 1.4426950408889634f * 0.08838834764831845f;
  float M = -INFINITY, Ls = 0.f;  // running log2-domain max and sum of this lane's head
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
  // One buffer: item j's V goes to LDS and its K into the S product, then
  // item j + 1's V loads go out (landing during item j's softmax and PV) and
  // its K loads after them.  Loads past the last item re-read it.  (Two
  // buffers, item j + 2 in flight beside j + 1, measured slower: 220.6
  // against 217.4 us per decode step.)
  StepQuarter cur;
  int nvalid = 0;
  if (mine > 0) {
    const u16 *Kq, *Vq;
    item(0, Kq, Vq, nvalid);
    load_k(cur, Kq, nvalid);
    load_v(cur, Vq, nvalid);
  }
  for (int j = 0; j < mine; ++j) {
    const int nv = nvalid;
    f32x4 sc[2] = {f32x4{}, f32x4{}};
    if (nv > 0) {
      // V -> V^T: task j4 of a lane holds keys 2 col, 2 col + 1 and d = 8 qd +
      // 32 j4 + e; dec_vt's swizzle depends on e >> 2 only, so two base
      // addresses plus immediate offsets cover all 32 stores
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int k0 = 2 * col;
        const uint32_t w0[4] = {cur.v0[j4].x, cur.v0[j4].y, cur.v0[j4].z, cur.v0[j4].w};
        const uint32_t w1[4] = {cur.v1[j4].x, cur.v1[j4].y, cur.v1[j4].z, cur.v1[j4].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = k0 < nv ? (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu : 0u;
          const uint32_t hi = k0 + 1 < nv ? (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu : 0u;
          *reinterpret_cast<uint32_t*>(&vt[(e < 4 ? vb0 : vb1) + (32 * j4 + e) * 64]) =
              lo | (hi << 16);
        }
      }
      // S^T tiles: lane holds head col, keys 16t + 4qd + r
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          sc[t] = mfma16(as_bf16x8(cur.kf[t][s4]), as_bf16x8(qs[s4][lane]), sc[t]);
    }
    const u16 *Kq, *Vq;
    item(j + 1 < mine ? j + 1 : j, Kq, Vq, nvalid);
    load_v(cur, Vq, nvalid);
    if (nv > 0) {
      float mq = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (16 * t + 4 * qd + r >= nv) sc[t][r] = -INFINITY;
          mq = fmaxf(mq, sc[t][r]);
        }
      mq = quads_max(mq);
      const float Mn = fmaxf(M, mq * qscale);  // finite: the quarter has a valid key
      const float alpha = fast_exp2(M - Mn);    // 0 while M is -inf
      float pv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = fast_exp2(fmaf(sc[0][r], qscale, -Mn));
        pv[4 + r] = fast_exp2(fmaf(sc[1][r], qscale, -Mn));
      }
      float l = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) l += pv[e];
      l = quads_sum(l);
      Ls = Ls * alpha + l;
      M = Mn;
      const uint4 pf = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O^T tiles: lane holds head col, d = 16dt + 4qd + r
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 av = *reinterpret_cast<const uint4*>(&vt[dec_vt(16 * dt + col, qd)]);
        o[dt] = mfma16(as_bf16x8(av), as_bf16x8(pf), o[dt] * alpha);
      }
    }
    load_k(cur, Kq, nvalid);
  }

  // the waves' (max, sum, O) meet in LDS
  if (qd == 0) {
    wm[wave][col] = M;
    wl[wave][col] = Ls;
  }
  __syncthreads();  // every wave is done with its V^T; the merge reuses the LDS
  float* red = reinterpret_cast<float*>(lds);  // [NW][HG][128]
  if (col < HG) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&red[(wave * HG + col) * kHeadDim + 16 * dt + 4 * qd]) = o[dt];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < HG * 32; e += 64 * NW) {
    const int hh = e >> 5, d0 = 4 * (e & 31);
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mh = fmaxf(Mh, wm[w][hh]);
    f32x4 acc = f32x4{};
    float den = 0.f;
    if (Mh > -INFINITY) {  // a part without items keeps zeros and -inf
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sw = fast_exp2(wm[w][hh] - Mh);  // 0 for a wave without items
        acc += *reinterpret_cast<const f32x4*>(&red[(w * HG + hh) * kHeadDim + d0]) * sw;
        den += wl[w][hh] * sw;
      }
    }
    if constexpr (SPLIT == 1) {
      const float inv = 1.f / den;
      uint2 st;
      st.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      st.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<uint2*>(a.O + (b * a.Hq + g * HG + hh) * kHeadDim + d0) = st;
      if (a.lse && d0 == 0)
        a.lse[b * a.Hq + g * HG + hh] = (Mh + __log2f(den)) * 0.6931471805599453f;
    } else {
      const int64_t pr = (bg * SPLIT + h) * HG + hh;
      *reinterpret_cast<f32x4*>(a.part + pr * kHeadDim + d0) = acc;
      if (d0 == 0) a.ml[pr] = make_float2(Mh, den);
    }
  }
}

// Merge of the SPLIT parts of each (sequence, head): one wave per (sequence,
// head), two values per lane.
template <int SPLIT>
__global__ void __launch_bounds__(256) decode_step_merge_kernel(StepArgs a, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wid >= rows) return;  // rows = B * Hq
  const int hg = a.Hq / a.G;
  const int64_t b = wid / a.Hq;
  const int hq = static_cast<int>(wid % a.Hq);
  const int64_t bg = b * a.G + hq / hg;
  const int hh = hq % hg;
  float2 ml[SPLIT];
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < SPLIT; ++p) {
    ml[p] = a.ml[(bg * SPLIT + p) * hg + hh];
    M = fmaxf(M, ml[p].x);
  }
  float o0 = 0.f, o1 = 0.f, den = 0.f;
#pragma unroll
  for (int p = 0; p < SPLIT; ++p) {
    const float sw = ml[p].x > -INFINITY ? fast_exp2(ml[p].x - M) : 0.f;
    const float2 v =
        *reinterpret_cast<const float2*>(a.part + ((bg * SPLIT + p) * hg + hh) * kHeadDim + 2 * lane);
    o0 += v.x * sw;
    o1 += v.y * sw;
    den += ml[p].y * sw;
  }
  const float inv = 1.f / den;
  *reinterpret_cast<uint32_t*>(a.O + wid * kHeadDim + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
  if (a.lse && lane == 0) a.lse[wid] = (M + __log2f(den)) * 0.6931471805599453f;
}

// Rows below which the step splits each row over two workgroups.
#ifndef MSA_STEP_SPLIT_ROWS
#define MSA_STEP_SPLIT_ROWS 256
#endif
constexpr int64_t kStepSplitRows = MSA_STEP_SPLIT_ROWS;

size_t decode_step_scratch_bytes(int64_t B, int G, int Hq) {
  if (B * G >= kStepSplitRows) return 0;
  const int64_t pr = B * G * kStepParts * (Hq / G);
  return static_cast<size_t>(pr) * (kHeadDim * sizeof(float) + sizeof(float2));
}

template <int HG>
static hipError_t launch_step_t(const StepArgs& sa, int64_t rows, hipStream_t st) {
  if (rows >= kStepSplitRows) {
    hipLaunchKernelGGL((decode_step_kernel<HG, 1>), dim3(static_cast<unsigned>(rows)),
                       dim3(64 * kStepWaves), 0, st, sa);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_step_kernel<HG, kStepParts>),
                     dim3(static_cast<unsigned>(kStepParts * rows)), dim3(64 * kStepWaves), 0, st,
                     sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t heads = rows * HG;
  hipLaunchKernelGGL((decode_step_merge_kernel<kStepParts>),
                     dim3(static_cast<unsigned>((heads + 3) / 4)),
                     dim3(256), 0, st, sa, heads);
  return hipGetLastError();
}

hipError_t launch_decode_step(const float* S, const void* q, const void* K, const void* V,
                              int32_t* idx, void* O, float* lse, void* scratch, int64_t B,
                              int64_t N, int Hq, int G, int k, int Bk, const PagedCache& pc,
                              hipStream_t st) {
  StepArgs sa;
  sa.S = S;
  sa.q = static_cast<const u16*>(q);
  sa.K = static_cast<const u16*>(K);
  sa.V = static_cast<const u16*>(V);
  sa.idx = idx;
  sa.O = static_cast<u16*>(O);
  sa.lse = lse;
  const int64_t rows = B * G;
  sa.part = static_cast<float*>(scratch);
  sa.ml = reinterpret_cast<float2*>(static_cast<float*>(scratch) +
                                    rows * kStepParts * (Hq / G) * kHeadDim);
  sa.N = N;
  sa.Hq = Hq;
  sa.G = G;
  sa.k = k;
  sa.Bk = Bk;
  sa.NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  sa.pc = pc;
  TimedLaunch tl(MSA_KERNEL_DECODE_STEP, st);
  switch (Hq / G) {
    case 8: return launch_step_t<8>(sa, rows, st);
    case 4: return launch_step_t<4>(sa, rows, st);
    case 16: return launch_step_t<16>(sa, rows, st);
    case 2: return launch_step_t<2>(sa, rows, st);
    case 1: return launch_step_t<1>(sa, rows, st);
  }
  return hipErrorInvalidValue;
}

template <int HG>
static hipError_t launch_decode_t(const DecArgs& da, const CombArgs& ca, int64_t n,
                                  hipStream_t st) {
  {
    TimedLaunch tl(MSA_KERNEL_DECODE_ATTN, st);
    hipLaunchKernelGGL((decode_attn_kernel<HG>), dim3(static_cast<unsigned>(n)), dim3(256), 0,
                       st, da);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = ca.rows * ca.G * HG;
  TimedLaunch tl(MSA_KERNEL_DECODE_COMBINE, st);
  if (ca.k > 16)
    hipLaunchKernelGGL((decode_combine_kernel<HG, 16>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(256), 0, st, ca);
  else
    hipLaunchKernelGGL((decode_combine_kernel<HG, 4>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(256), 0, st, ca);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse, int64_t B, int64_t N,
                              int Hq, int G, int k, int Bk, const PagedCache& pc,
                              const AttnWorkspace& w, hipStream_t st) {
  const int hg = Hq / G;
  DecArgs da;
  da.pc = pc;
  da.q = static_cast<const u16*>(q);
  da.K = static_cast<const u16*>(K);
  da.V = static_cast<const u16*>(V);
  da.idx = idx;
  da.opart = w.opart;
  da.lpart = w.lpart;
  da.N = N;
  da.Hq = Hq;
  da.G = G;
  da.k = k;
  da.Bk = Bk;
  CombArgs ca;
  ca.idx = idx;
  ca.opart = w.opart;
  ca.lpart = w.lpart;
  ca.O = static_cast<u16*>(O);
  ca.lse = lse;
  ca.T = 1;
  ca.r0 = 0;
  ca.rows = B;
  ca.Hq = Hq;
  ca.G = G;
  ca.k = k;
  ca.rl_base = 0;
  ca.group = -1;
  ca.pgroups = G;
  const int64_t n = B * G * k;
  switch (hg) {
    case 8: return launch_decode_t<8>(da, ca, n, st);
    case 4: return launch_decode_t<4>(da, ca, n, st);
    case 16: return launch_decode_t<16>(da, ca, n, st);
    case 2: return launch_decode_t<2>(da, ca, n, st);
    case 1: return launch_decode_t<1>(da, ca, n, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
