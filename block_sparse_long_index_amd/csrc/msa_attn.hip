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

#include <math.h>

namespace msa {

constexpr int kChunkQueries = 64;  // queries per work chunk (rows = 64 * hg)

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static int64_t max_chunks_for(int64_t window, int64_t nbins, int G, int k, bool decode) {
  const int64_t entries = window * G * k;
  if (decode) return entries;  // one chunk per (sequence, group, slot)
  return entries / kChunkQueries + (nbins < entries ? nbins : entries) + 1;
}

size_t attn_workspace_bytes(int64_t window, int64_t B, int64_t N, int G, int hg, int k,
                            bool decode) {
  const int64_t NB = (N + kBlock - 1) / kBlock;
  const int64_t nbins = B * G * NB;
  const int64_t entries = window * G * k;
  size_t s = 0;
  s += 4 * align256(sizeof(int32_t) * nbins);                  // counts, cursor, offsets, chunk_start
  s += align256(sizeof(int32_t) * 4);                          // totals
  s += align256(sizeof(int32_t) * entries);                    // entries
  s += align256(sizeof(int4) * max_chunks_for(window, nbins, G, k, decode));
  s += align256(sizeof(uint16_t) * entries * hg * kHeadDim);   // partial O
  s += align256(sizeof(float) * entries * hg);                 // partial lse
  return s;
}

void attn_workspace_carve(void* ws, int64_t window, int64_t B, int64_t N, int G,
                          int hg, int k, bool decode, AttnWorkspace* w) {
  const int64_t NB = (N + kBlock - 1) / kBlock;
  const int64_t nbins = B * G * NB;
  const int64_t entries = window * G * k;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += align256(bytes);
    return r;
  };
  w->counts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nbins));
  w->cursor = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nbins));
  w->offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nbins));
  w->chunk_start = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nbins));
  w->totals = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 4));
  w->entries = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * entries));
  w->max_chunks = max_chunks_for(window, nbins, G, k, decode);
  w->chunks = reinterpret_cast<int4*>(take(sizeof(int4) * w->max_chunks));
  w->opart = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * entries * hg * kHeadDim));
  w->lpart = reinterpret_cast<float*>(take(sizeof(float) * entries * hg));
  w->window = window;
  w->nbins = nbins;
}

// ---------------------------------------------------------------------------
// Inversion of the selection for the query rows [r0, r0 + W) (row r is query
// t = r % T of sequence b = r / T): histogram per (b, g, block), exclusive
// scan, scatter of the entries e = (r - r0) * k + slot, and the chunk list.
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

struct InvArgs {
  const int32_t* idx;
  int32_t* counts;
  int32_t* cursor;
  const int32_t* offsets;
  int32_t* entries;
  int64_t T, r0, W;
  int32_t G, k, NB;
};

__device__ __forceinline__ void entry_bin(const InvArgs& a, int64_t i, int64_t& bin,
                                          int32_t& e) {
  // i enumerates (row in window, group, slot)
  const int32_t s = static_cast<int32_t>(i % a.k);
  const int64_t rg = i / a.k;
  const int32_t g = static_cast<int32_t>(rg % a.G);
  const int64_t rl = rg / a.G;
  const int64_t r = a.r0 + rl;
  const int64_t b = r / a.T, t = r % a.T;
  const int32_t blk = a.idx[((b * a.G + g) * a.T + t) * a.k + s];
  bin = blk < 0 ? -1 : (b * a.G + g) * a.NB + blk;
  e = static_cast<int32_t>(rl * a.k + s);
}

__global__ void count_kernel(InvArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= a.W * a.G * a.k) return;
  int64_t bin;
  int32_t e;
  entry_bin(a, i, bin, e);
  if (bin >= 0) atomicAdd(&a.counts[bin], 1);
}

__global__ void scatter_kernel(InvArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= a.W * a.G * a.k) return;
  int64_t bin;
  int32_t e;
  entry_bin(a, i, bin, e);
  if (bin < 0) return;
  const int32_t pos = a.offsets[bin] + atomicAdd(&a.cursor[bin], 1);
  a.entries[pos] = e;
}

// Single-workgroup exclusive scan of the bin counts and of their chunk
// counts; totals[0] = entries, totals[1] = chunks.
__global__ void __launch_bounds__(1024) scan_kernel(const int32_t* counts, int32_t* offsets,
                                                    int32_t* chunk_start, int32_t* totals,
                                                    int64_t nbins) {
  __shared__ int32_t s_e[1024], s_c[1024];
  __shared__ int32_t carry_e, carry_c;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_e = 0;
    carry_c = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < nbins; base += 1024) {
    const int64_t i = base + tid;
    const int32_t c = i < nbins ? counts[i] : 0;
    const int32_t ch = (c + kChunkQueries - 1) / kChunkQueries;
    s_e[tid] = c;
    s_c[tid] = ch;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t ve = tid >= off ? s_e[tid - off] : 0;
      const int32_t vc = tid >= off ? s_c[tid - off] : 0;
      __syncthreads();
      s_e[tid] += ve;
      s_c[tid] += vc;
      __syncthreads();
    }
    if (i < nbins) {
      offsets[i] = carry_e + s_e[tid] - c;
      chunk_start[i] = carry_c + s_c[tid] - ch;
    }
    __syncthreads();
    if (tid == 1023) {
      carry_e += s_e[1023];
      carry_c += s_c[1023];
    }
    __syncthreads();
  }
  if (tid == 0) {
    totals[0] = carry_e;
    totals[1] = carry_c;
  }
}

__global__ void chunk_kernel(const int32_t* counts, const int32_t* offsets,
                             const int32_t* chunk_start, int4* chunks, int64_t nbins) {
  const int64_t bin = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (bin >= nbins) return;
  const int32_t c = counts[bin];
  const int32_t off = offsets[bin];
  int32_t cs = chunk_start[bin];
  for (int32_t j = 0; j < c; j += kChunkQueries, ++cs) {
    const int32_t n = (c - j) < kChunkQueries ? (c - j) : kChunkQueries;
    chunks[cs] = make_int4(static_cast<int32_t>(bin), off + j, n, 0);
  }
}

// Decode needs no inversion: every (sequence, group, slot) is its own chunk
// with one entry.  The window is the B decode rows.
__global__ void decode_work_kernel(const int32_t* idx, int4* chunks, int32_t* entries,
                                   int32_t* totals, int64_t B, int32_t G, int32_t k,
                                   int32_t NB) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = B * G * k;
  if (i == 0) {
    totals[0] = static_cast<int32_t>(n);
    totals[1] = static_cast<int32_t>(n);
  }
  if (i >= n) return;
  const int32_t s = static_cast<int32_t>(i % k);
  const int64_t bg = i / k;
  const int64_t b = bg / G;
  const int32_t blk = idx[bg * k + s];
  entries[i] = static_cast<int32_t>(b * k + s);
  chunks[i] = make_int4(static_cast<int32_t>(bg * NB + (blk < 0 ? 0 : blk)),
                        static_cast<int32_t>(i), blk < 0 ? 0 : 1, 0);
}

// ---------------------------------------------------------------------------
// KV-outer attention.  One workgroup per chunk (b, g, block, <= 64 queries):
// the block's K (row-major) and V (transposed) go to LDS once and every
// gathered (query, head) row is processed against them: S^T = K Q^T with keys
// on the MFMA M side (a lane holds 16 keys of one row, so the row max and sum
// are in-register plus one half-wave exchange), softmax in fp32 with exp2,
// P rounded to bf16, O^T = V^T P^T.  Each row writes its normalised partial O
// (bf16) and lse (fp32, natural log) for the combine.
//
// V^T layout: row d holds the 128 keys of the block; inside every 16-key group
// the keys are stored in the order 0-3, 8-11, 4-7, 12-15, which is the order
// in which one half-wave's P values reach the PV MFMA's k slots, so each
// lane's A operand is one 16-B read.  Rows are chunk-swizzled like K.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const u16* q;
  const u16* K;
  const u16* V;
  const int4* chunks;
  const int32_t* entries;
  const int32_t* totals;
  u16* opart;
  float* lpart;
  int64_t T, N, r0;
  int32_t Hq, G, NB, k;
};

__device__ __forceinline__ int vt_pos(int key) {
  const int o = key & 15;
  return (key & ~15) + ((o >> 2) & 1) * 8 + ((o >> 3) & 1) * 4 + (o & 3);
}

template <int HG>
__global__ void __launch_bounds__(512) kv_outer_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char ks[32768];
  __shared__ __align__(16) unsigned char vt[32768];
  if (static_cast<int>(blockIdx.x) >= a.totals[1]) return;
  const int4 ch = a.chunks[blockIdx.x];
  const int n = ch.z;
  if (n <= 0) return;
  const int64_t bin = ch.x;
  const int64_t blk = bin % a.NB;
  const int64_t bg = bin / a.NB;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const int64_t key0 = blk * kBlock;
  const u16* Kb = a.K + (bg * a.N + key0) * kHeadDim;
  const u16* Vb = a.V + (bg * a.N + key0) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * 512;
    const int r = i >> 4, c = i & 15;
    const uint4 v = key0 + r < a.N ? ld16(Kb + r * kHeadDim + c * 8) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&ks[swz(r, c)]) = v;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + j * 512;
    const int kp = i & 63, c = i >> 6;
    const int k0 = 2 * kp;
    const uint4 v0 = key0 + k0 < a.N ? ld16(Vb + k0 * kHeadDim + c * 8) : make_uint4(0, 0, 0, 0);
    const uint4 v1 = key0 + k0 + 1 < a.N ? ld16(Vb + (k0 + 1) * kHeadDim + c * 8)
                                          : make_uint4(0, 0, 0, 0);
    const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
    const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
    const int P = vt_pos(k0);  // even; k0 + 1 lands at P + 1
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t hi = (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const int d = 8 * c + e;
      *reinterpret_cast<uint32_t*>(&vt[swz(d, P >> 3) + ((2 * P) & 15)]) = lo | (hi << 16);
    }
  }
  __syncthreads();

  const int rows = n * HG;
  constexpr float kLog2e = 1.4426950408889634f;
  const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  for (int pass = 0; pass * 256 + wave * 32 < rows; ++pass) {
    const int rr = pass * 256 + wave * 32 + l32;
    const bool valid = rr < rows;
    const int e = valid ? a.entries[ch.y + rr / HG] : 0;
    const int hh = rr % HG;
    const int64_t rl = e / a.k;
    const int slot = e % a.k;
    const int64_t grow = a.r0 + rl;
    const int64_t t = grow % a.T;
    const int64_t p = a.N - a.T + t;
    const u16* qrow = a.q + ((b * a.T + t) * a.Hq + g * HG + hh) * kHeadDim;
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = as_bf16x8(valid ? ld16(qrow + 16 * s + 8 * half) : make_uint4(0, 0, 0, 0));

    // S^T = K Q^T, one 32-key tile at a time
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x16{};
      const int r = kt * 32 + l32;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&ks[swz(r, 2 * s + half)]));
        sacc[kt] = mfma32(av, qf[s], sacc[kt]);
      }
      sched_fence();
    }
    // causal mask: only the local block of a row has keys after the row
    const int lim = static_cast<int>(p - key0);  // >= 0: block <= local(row)
    if (__ballot(lim < kBlock - 1)) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (off > lim) sacc[kt][i] = -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) m = max3(m, sacc[kt][i], sacc[kt][i + 1]);
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mc = m * qscale;

    // P = exp2(s * log2e/sqrt(d) - max), rounded to bf16, then O^T += V^T P^T
    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
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
        const int d = dt * 32 + l32;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bf16x8 av = as_bf16x8(
              *reinterpret_cast<const uint4*>(&vt[swz(d, kt * 4 + hf * 2 + half)]));
          oacc[dt] = mfma32(av, as_bf16x8(pb[hf]), oacc[dt]);
        }
      }
      sched_fence();
    }
    l += __shfl_xor(l, 32);
    if (valid) {
      const float inv = 1.f / l;
      const int64_t prow = ((rl * a.G + g) * a.k + slot) * HG + hh;
      u16* dst = a.opart + prow * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = dt * 32 + 8 * q4 + 4 * half;
          uint2 w;
          w.x = pack_bf16x2(oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv);
          w.y = pack_bf16x2(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(dst + d0) = w;
        }
      }
      if (half == 0) a.lpart[prow] = (mc + __log2f(l)) * 0.6931471805599453f;
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
  const float* lpart;
  u16* O;
  float* lse;
  int64_t T, r0, W;
  int32_t Hq, G, k;
};

template <int HG>
__global__ void __launch_bounds__(256) combine_kernel(CombArgs a) {
  constexpr int LPH = 64 / HG;          // lanes per head
  constexpr int VPL = kHeadDim / LPH;   // values per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rg = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (rg >= a.W * a.G) return;
  const int64_t rl = rg / a.G;
  const int g = static_cast<int>(rg % a.G);
  const int64_t grow = a.r0 + rl;
  const int64_t b = grow / a.T, t = grow % a.T;
  const int32_t* ir = a.idx + ((b * a.G + g) * a.T + t) * a.k;
  const bool sv = lane < a.k && ir[lane < a.k ? lane : 0] >= 0;
  const int nval = __popcll(__ballot(sv));
  const int hh = lane / LPH;
  const int d0 = (lane % LPH) * VPL;
  const int64_t pbase = (rl * a.G + g) * a.k;

  float ls[16];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    ls[s] = s < nval ? a.lpart[(pbase + s) * HG + hh] : -INFINITY;
    mx = fmaxf(mx, ls[s]);
  }
  float acc[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < nval) {
      const float w = __expf(ls[s] - mx);
      den += w;
      const u16* src = a.opart + ((pbase + s) * HG + hh) * kHeadDim + d0;
      if constexpr (VPL >= 8) {
#pragma unroll
        for (int j = 0; j < VPL; j += 8) {
          const uint4 v = ld16(src + j);
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            acc[j + 2 * u] += w * __uint_as_float(wv[u] << 16);
            acc[j + 2 * u + 1] += w * __uint_as_float(wv[u] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) acc[j] += w * bf16_to_f32(src[j]);
      }
    }
  }
  const float inv = 1.f / den;
  u16* dst = a.O + ((b * a.T + t) * a.Hq + g * HG + hh) * kHeadDim + d0;
  if constexpr (VPL >= 8) {
#pragma unroll
    for (int j = 0; j < VPL; j += 8) {
      uint4 w;
      w.x = pack_bf16x2(acc[j + 0] * inv, acc[j + 1] * inv);
      w.y = pack_bf16x2(acc[j + 2] * inv, acc[j + 3] * inv);
      w.z = pack_bf16x2(acc[j + 4] * inv, acc[j + 5] * inv);
      w.w = pack_bf16x2(acc[j + 6] * inv, acc[j + 7] * inv);
      *reinterpret_cast<uint4*>(dst + j) = w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) dst[j] = f32_to_bf16(acc[j] * inv);
  }
  if (a.lse && (lane % LPH) == 0)
    a.lse[(b * a.Hq + g * HG + hh) * a.T + t] = mx + logf(den);
}

// ---------------------------------------------------------------------------
template <int HG>
static hipError_t launch_kv_combine(const AttnArgs& aa, const CombArgs& ca, int64_t grid_chunks,
                                    hipStream_t st) {
  hipLaunchKernelGGL((kv_outer_kernel<HG>), dim3(static_cast<unsigned>(grid_chunks)), dim3(512),
                     0, st, aa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cgrid = (ca.W * ca.G + 3) / 4;
  hipLaunchKernelGGL((combine_kernel<HG>), dim3(static_cast<unsigned>(cgrid)), dim3(256), 0, st,
                     ca);
  return hipGetLastError();
}

static hipError_t dispatch_hg(int hg, const AttnArgs& aa, const CombArgs& ca, int64_t grid,
                              hipStream_t st) {
  switch (hg) {
    case 8: return launch_kv_combine<8>(aa, ca, grid, st);
    case 4: return launch_kv_combine<4>(aa, ca, grid, st);
    case 16: return launch_kv_combine<16>(aa, ca, grid, st);
    case 2: return launch_kv_combine<2>(aa, ca, grid, st);
    case 1: return launch_kv_combine<1>(aa, ca, grid, st);
  }
  return hipErrorInvalidValue;
}

static unsigned blocks_for(int64_t n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

hipError_t launch_attn_prefill(const void* q, const void* K, const void* V,
                               const int32_t* idx, void* O, float* lse, int64_t B,
                               int64_t T, int64_t N, int Hq, int G, int k,
                               const AttnWorkspace& w, hipStream_t st) {
  const int hg = Hq / G;
  const int32_t NB = static_cast<int32_t>((N + kBlock - 1) / kBlock);
  const int64_t rows = B * T;
  for (int64_t r0 = 0; r0 < rows; r0 += w.window) {
    const int64_t W = (rows - r0) < w.window ? (rows - r0) : w.window;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(w.nbins, 256)), dim3(256), 0, st,
                       w.counts, w.nbins, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(w.nbins, 256)), dim3(256), 0, st,
                       w.cursor, w.nbins, 0);
    InvArgs ia;
    ia.idx = idx;
    ia.counts = w.counts;
    ia.cursor = w.cursor;
    ia.offsets = w.offsets;
    ia.entries = w.entries;
    ia.T = T;
    ia.r0 = r0;
    ia.W = W;
    ia.G = G;
    ia.k = k;
    ia.NB = NB;
    const int64_t n_ent = W * G * k;
    hipLaunchKernelGGL(count_kernel, dim3(blocks_for(n_ent, 256)), dim3(256), 0, st, ia);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, w.counts, w.offsets,
                       w.chunk_start, w.totals, w.nbins);
    hipLaunchKernelGGL(scatter_kernel, dim3(blocks_for(n_ent, 256)), dim3(256), 0, st, ia);
    hipLaunchKernelGGL(chunk_kernel, dim3(blocks_for(w.nbins, 256)), dim3(256), 0, st, w.counts,
                       w.offsets, w.chunk_start, w.chunks, w.nbins);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    AttnArgs aa;
    aa.q = static_cast<const u16*>(q);
    aa.K = static_cast<const u16*>(K);
    aa.V = static_cast<const u16*>(V);
    aa.chunks = w.chunks;
    aa.entries = w.entries;
    aa.totals = w.totals;
    aa.opart = w.opart;
    aa.lpart = w.lpart;
    aa.T = T;
    aa.N = N;
    aa.r0 = r0;
    aa.Hq = Hq;
    aa.G = G;
    aa.NB = NB;
    aa.k = k;
    CombArgs ca;
    ca.idx = idx;
    ca.opart = w.opart;
    ca.lpart = w.lpart;
    ca.O = static_cast<u16*>(O);
    ca.lse = lse;
    ca.T = T;
    ca.r0 = r0;
    ca.W = W;
    ca.Hq = Hq;
    ca.G = G;
    ca.k = k;
    const int64_t grid = max_chunks_for(W, w.nbins, G, k, false);
    e = dispatch_hg(hg, aa, ca, grid, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_decode(const void* q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse, int64_t B, int64_t N,
                              int Hq, int G, int k, const AttnWorkspace& w, hipStream_t st) {
  const int hg = Hq / G;
  const int32_t NB = static_cast<int32_t>((N + kBlock - 1) / kBlock);
  const int64_t n = B * G * k;
  hipLaunchKernelGGL(decode_work_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, idx,
                     w.chunks, w.entries, w.totals, B, G, k, NB);
  AttnArgs aa;
  aa.q = static_cast<const u16*>(q);
  aa.K = static_cast<const u16*>(K);
  aa.V = static_cast<const u16*>(V);
  aa.chunks = w.chunks;
  aa.entries = w.entries;
  aa.totals = w.totals;
  aa.opart = w.opart;
  aa.lpart = w.lpart;
  aa.T = 1;
  aa.N = N;
  aa.r0 = 0;
  aa.Hq = Hq;
  aa.G = G;
  aa.NB = NB;
  aa.k = k;
  CombArgs ca;
  ca.idx = idx;
  ca.opart = w.opart;
  ca.lpart = w.lpart;
  ca.O = static_cast<u16*>(O);
  ca.lse = lse;
  ca.T = 1;
  ca.r0 = 0;
  ca.W = B;
  ca.Hq = Hq;
  ca.G = G;
  ca.k = k;
  return dispatch_hg(hg, aa, ca, n, st);
}

}  // namespace msa
