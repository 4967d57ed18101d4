// msa_index_kl.hip -- backward of the index branch's KL alignment on gfx950:
// dq^I, dk^I (and the loss) of sum over rows and groups of KL(teacher ||
// proxy), each row's selection held fixed, scheduled KV-outer from the
// forward's inversion.
//
// Method: the study notes (sections 4-2 and 4-3) train the index branch by a
// KL loss against the mean of the group's main-branch head weights, that
// teacher detached; the Flash-MSA training blog (hackernews.jp, "KL
// divergence loss") shows that the loss's gradient on the proxy logits is
// the proxy weight minus the main weight, and recomputes the proxy lse over
// the selected sparse activations.  Per (row, group), over the row's support
// J (visible keys of its selected blocks), with c_I = 1/sqrt(128):
//   s_j = c_I q^I . k^I_j,      p_x = softmax_J(s)          (proxy)
//   p_t(j) = mean over the group's heads h of exp(q_h . K_j / sqrt(128) - lse_h)
//   KL = sum_j p_t (log p_t - log p_x),  dz_j = p_x(j) - p_t(j),
//   dq^I = c_I sum_j dz_j k^I_j,         dk^I_j += c_I dz_j q^I.
// KV-outer passes per stage: the teacher p_t per (row, slot, key) (written by
// teacher_kernel, or by the main backward's stage in the fused training
// backward); index_px_kernel writes (max, sum) of the proxy exponentials per
// (row, slot) and px_combine_kernel makes the proxy lse per row;
// index_kl_teach_kernel then forms p_x and dz per (row, key), adds dk^I (fp32
// atomics: the index keys are shared by all groups) and writes per-(row,
// slot) partials of dq^I and of the loss, summed in slot order.
#include "msa_common.h"
#include "msa_internal.h"

#include <math.h>

namespace msa {

namespace {

constexpr int kP = 272;   // LDS row pitch of a 128-column bf16 tile
constexpr int kTq = 80;   // LDS row pitch of the transposed 32-query q^I tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScale = 0.08838834764831845f;  // 1/sqrt(128)

// Column of pass query r (0..31) in the transposed q^I tile: the k-slot order
// of the dk^I product's A operand (see the backward kernel's transposed tiles).
__device__ __forceinline__ int tcol(int r) {
  const int o = r & 15;
  return (r & 16) + 8 * ((o >> 2) & 1) + 4 * (o >> 3) + (o & 3);
}

struct IkArgs {
  const u16* qI;          // [B, T, G, 128]
  const u16* kI;          // [B, N, 128]
  const u16* q;           // [B, T, Hq, 128]
  const u16* K;           // [B, G, N, 128]
  const float* lse;       // main lse [B, Hq, T], natural log
  const float* lpx;       // proxy lse [B, G, T], log2 domain (gradient pass)
  const float* teach;     // [stage rows, k, Bk] teacher per (row, slot, key) (teach kernel)
  const int4* chunks;
  const int32_t* entries;
  const int32_t* count;
  float2* part;           // per (row, slot): (max, sum) or (loss, -)
  u16* dqpart;            // per (row, slot): 128 bf16
  float* dkI;             // [B, N, 128]
  int64_t T, N, r0;
  int32_t Hq, G, k, Bk, rl_base, sink;
};

// Proxy lse partials.  One workgroup per chunk; wave w takes queries
// 32w..32w+31 of the chunk against the block's 128 index keys: s^T = k^I q^I^T
// with keys on M, so a lane holds 16 keys of its query per 32-key tile and the
// row max / sum stay in-register plus one half-wave exchange.
static_assert(kChunkQueries == 128, "index_px_kernel: four waves of 32 queries cover a chunk");
__global__ void __launch_bounds__(256) index_px_kernel(IkArgs a) {
  __shared__ __align__(16) unsigned char kis[128 * kP];
  const int nchunks = *a.count;
  const int per_xcd = (nchunks + 7) >> 3;
  const int xj = static_cast<int>(blockIdx.x >> 3);
  const int ci = static_cast<int>(blockIdx.x & 7) * per_xcd + xj;
  if (xj >= per_xcd || ci >= nchunks) return;
  const int4 ch = a.chunks[ci];
  const int n = ch.z;
  if (n <= 0) return;
  const int64_t blk = ch.w, bg = ch.x;
  const int g = static_cast<int>(bg) & (a.G - 1);
  const int64_t b = bg >> __builtin_ctz(a.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t key0 = blk * a.Bk;
  // the block's keys (>= 1); LDS rows past them are zero and masked
  const int nvalid = static_cast<int>(a.N - key0 < a.Bk ? a.N - key0 : a.Bk);
  const u16* kb = a.kI + (b * a.N + key0) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + 256 * j;
    const int r = i >> 4, c = i & 15;
    const uint4 y = ld16(kb + (r < nvalid ? r : nvalid - 1) * kHeadDim + 8 * c);
    *reinterpret_cast<uint4*>(&kis[r * kP + 16 * c]) = r < nvalid ? y : make_uint4(0, 0, 0, 0);
  }
  // this lane's query
  const int qi = 32 * wave + l32;
  const bool valid = qi < n;
  const int e = a.entries[ch.y + (valid ? qi : 0)];
  const int64_t t = (a.r0 - b * a.T) + (e >> 6);
  const int lim =
      valid ? static_cast<int>(min(a.N - a.T + t - key0, static_cast<int64_t>(nvalid - 1))) : -1;
  const u16* qr = a.qI + ((b * a.T + t) * a.G + g) * kHeadDim + 8 * half;
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld16(qr + 16 * s));
  __syncthreads();
  const float c2 = kScale * kLog2e;
  float v[4][16];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x16 acc = f32x16{};
    const unsigned char* ka = kis + (32 * kt + l32) * kP + half * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(ka + 32 * s)), qf[s], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
      v[kt][i] = key <= lim ? acc[i] * c2 : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, v[kt][i]);
  m = halves_max(m);
  float l = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) l += fast_exp2(v[kt][i] - m);
  }
  l = halves_sum(l);
  if (valid && half == 0) {
    const int prow = ((e >> 6) - a.rl_base) * a.k + (e & 63);
    a.part[prow] = make_float2(m, l);
  }
}

struct PxArgs {
  const int32_t* idx;
  const float2* part;
  float* lpx;  // [B, G, T], log2 domain
  int64_t T, r0, rows;
  int32_t G, k, rl_base, group;
};

// proxy lse of a row = log2 of the sum over its valid slots of l 2^m
__global__ void __launch_bounds__(256) px_combine_kernel(PxArgs a) {
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (wid >= a.rows) return;
  const int64_t grow = a.r0 + a.rl_base + wid;
  const int64_t b = grow / a.T, t = grow % a.T;
  const int32_t* ir = a.idx + ((b * a.G + a.group) * a.T + t) * a.k;
  float M = -INFINITY;
  int nval = 0;
  for (int s = 0; s < a.k && ir[s] >= 0; ++s) {
    M = fmaxf(M, a.part[wid * a.k + s].x);
    nval = s + 1;
  }
  float L = 0.f;
  for (int s = 0; s < nval; ++s) {
    const float2 p = a.part[wid * a.k + s];
    L += p.y * fast_exp2(p.x - M);
  }
  a.lpx[(b * a.G + a.group) * a.T + t] = M + __log2f(L);
}

// The gradient pass with the teacher given: p_t per (row, slot, key) has
// been written (by teacher_kernel or the fused training backward's main
// stage), so no main-branch operand is loaded and the kernel needs only k^I and the passes' q^I in LDS (64 KB:
// two workgroups per CU hide each other's load latency).  Per pass of 32
// queries: s from q^I k^I^T, dz = p_x - p_t, the loss terms (one reduce-
// scatter over the half-wave's keys), dk^I += dz^T q^I in registers, and
// dq^I^T = k^I^T dz^T with this wave's k^I^T fragments (dims 32w..32w+31,
// every key) held in registers for the whole chunk.
__global__ void __launch_bounds__(256, 2) index_kl_teach_kernel(IkArgs a) {
  __shared__ __align__(16) unsigned char kis[128 * kP];   // k^I [key][d]
  __shared__ __align__(16) unsigned char qis[32 * kP];    // the pass's q^I [query][d]
  __shared__ __align__(16) unsigned char qit[128 * kTq];  // q^I^T [d][tcol(query)]
  __shared__ __align__(16) unsigned char dzs[32 * kP];    // c_I dz [query][key], bf16
  __shared__ float r_px[32], r_kl[4][32];  // r_kl: per wave, summed in order
  __shared__ int r_lim[32], r_prow[32];
  __shared__ int ents[kChunkQueries];

  const int nchunks = *a.count;
  const int per_xcd = (nchunks + 7) >> 3;
  const int xj = static_cast<int>(blockIdx.x >> 3);
  const int ci = static_cast<int>(blockIdx.x & 7) * per_xcd + xj;
  if (xj >= per_xcd || ci >= nchunks) return;
  const int4 ch = a.chunks[ci];
  const int n = ch.z;
  if (n <= 0) return;
  const int64_t blk = ch.w, bg = ch.x;
  const int g = static_cast<int>(bg) & (a.G - 1);
  const int64_t b = bg >> __builtin_ctz(a.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t key0 = blk * a.Bk;
  // the block's keys (>= 1); LDS rows past them are zero and masked
  const int nvalid = static_cast<int>(a.N - key0 < a.Bk ? a.N - key0 : a.Bk);
  const u16* kib = a.kI + (b * a.N + key0) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + 256 * j;
    const int r = i >> 4, c = i & 15;
    const uint4 y = ld16(kib + (r < nvalid ? r : nvalid - 1) * kHeadDim + 8 * c);
    *reinterpret_cast<uint4*>(&kis[r * kP + 16 * c]) = r < nvalid ? y : make_uint4(0, 0, 0, 0);
  }
  if (tid < n) ents[tid] = a.entries[ch.y + tid];
  __syncthreads();

  const int64_t t0 = a.r0 - b * a.T;
  const int key_w = 32 * wave + l32;
  f32x16 dk[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dk[dt] = f32x16{};
  // k^I^T fragments of the dq^I product: lane = dim 32 wave + l32, k-step s
  // holds keys 16s + 8 half + 0..7
  uint4 kA[8];
  {
    const unsigned char* col = kis + 2 * (32 * wave + l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 16 * s + 8 * half + 2 * e;
        const uint32_t lo = *reinterpret_cast<const u16*>(col + kk * kP);
        const uint32_t hi = *reinterpret_cast<const u16*>(col + (kk + 1) * kP);
        w[e] = lo | (hi << 16);
      }
      kA[s] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  const int npass = (n + 31) / 32;
  // A pass's gather, one thread's share: q^I of queries 2rp, 2rp + 1 (dims
  // 8cc..8cc+7) and their row data; per lane, the teacher of the pass's rows
  // m(i) = 8(i/4) + 4 half + i%4 at its key (clamped into the block: keys
  // past Bk are masked at use).  fetch(p) only issues loads (every lane, valid
  // addresses) and runs during the previous pass; stash() masks and writes
  // to LDS at the pass's start.
  const int rp = tid & 15, cc = tid >> 4;
  const int tkey = key_w < a.Bk ? key_w : a.Bk - 1;
  uint4 xq[2];
  float fpx[2], tv[16];
  int flim[2], fprow[2];
  bool fval[2];
  auto fetch = [&](int p) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qq = p * 32 + 2 * rp + u;
      const bool valid = qq < n;
      const int e = ents[valid ? qq : 0];
      const int64_t t = t0 + (e >> 6);
      xq[u] = ld16(a.qI + ((b * a.T + t) * a.G + g) * kHeadDim + 8 * cc);
      fpx[u] = a.lpx[(b * a.G + g) * a.T + t];
      fval[u] = valid;
      flim[u] = valid ? static_cast<int>(min(a.N - a.T + t - key0, static_cast<int64_t>(nvalid - 1)))
                       : -1;  // last key of the block the row sees
      fprow[u] = valid ? ((e >> 6) - a.rl_base) * a.k + (e & 63) : a.sink;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qq = p * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      const int e = ents[qq < n ? qq : 0];
      const int64_t tp = ((e >> 6) - a.rl_base) * a.k + (e & 63);
      tv[i] = __builtin_nontemporal_load(a.teach + tp * a.Bk + tkey);
    }
  };
  auto stash = [&]() {
    const uint4 x0 = fval[0] ? xq[0] : make_uint4(0, 0, 0, 0);
    const uint4 x1 = fval[1] ? xq[1] : make_uint4(0, 0, 0, 0);
    const int r0 = 2 * rp;
    *reinterpret_cast<uint4*>(&qis[r0 * kP + 16 * cc]) = x0;
    *reinterpret_cast<uint4*>(&qis[(r0 + 1) * kP + 16 * cc]) = x1;
    const int P = tcol(r0);
    const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w};
    const uint32_t w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 16 * (e & 1);
      *reinterpret_cast<uint32_t*>(&qit[(8 * cc + e) * kTq + 2 * P]) =
          ((w0[e >> 1] >> sh) & 0xffffu) | (((w1[e >> 1] >> sh) & 0xffffu) << 16);
    }
    if (cc == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        r_lim[r0 + u] = flim[u];
        r_px[r0 + u] = fval[u] ? fpx[u] : INFINITY;
        r_prow[r0 + u] = fprow[u];
      }
    }
  };
  fetch(0);
  for (int pass = 0; pass < npass; ++pass) {
    const bool more = pass + 1 < npass;
    stash();
    float pt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pt[i] = tv[i];
    __syncthreads();
    fetch(more ? pass + 1 : pass);  // lands during this pass

    // index scores s: queries on M (A = q^I rows), this wave's keys on N
    f32x16 sacc = f32x16{};
    {
      const unsigned char* qa = qis + l32 * kP + half * 16;
      const unsigned char* kb = kis + key_w * kP + half * 16;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        sacc = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(qa + 32 * s)),
                      as_bf16x8(*reinterpret_cast<const uint4*>(kb + 32 * s)), sacc);
    }
    // dz = p_x - p_t and the loss terms p_t (log p_t - log p_x); c_I dz to LDS
    const float c2 = kScale * kLog2e;
    float dz[16], term[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 8 * (i >> 2) + 4 * half + (i & 3);
      const bool vis = key_w <= r_lim[m];
      const float lx2 = fmaf(sacc[i], c2, -r_px[m]);  // log2 p_x
      const float px = vis ? fast_exp2(lx2) : 0.f;
      const float t = vis ? pt[i] : 0.f;
      dz[i] = px - t;
      term[i] = t > 0.f ? t * (__log2f(t) - lx2) * kLn2 : 0.f;
      *reinterpret_cast<u16*>(&dzs[m * kP + 2 * key_w]) = f32_to_bf16(dz[i] * kScale);
    }
    // the terms' sums over the half-wave's 32 keys, reduce-scatter: after the
    // steps over lane bits 4, 3, 2, 1 and a final add over bit 0, lane l32
    // holds the sum of term i = 8 b4 + 4 b3 + 2 b2 + b1 (b = bits of l32)
    {
      float v8[8], v4[4], v2[2];
      const bool b4 = l32 & 16, b3 = l32 & 8, b2 = l32 & 4, b1 = l32 & 2;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v8[j] = (b4 ? term[j + 8] : term[j]) + __shfl_xor(b4 ? term[j] : term[j + 8], 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v4[j] = (b3 ? v8[j + 4] : v8[j]) + __shfl_xor(b3 ? v8[j] : v8[j + 4], 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        v2[j] = (b2 ? v4[j + 2] : v4[j]) + __shfl_xor(b2 ? v4[j] : v4[j + 2], 4);
      float v1 = (b1 ? v2[1] : v2[0]) + __shfl_xor(b1 ? v2[0] : v2[1], 2);
      v1 += __shfl_xor(v1, 1);
      const int i = 8 * b4 + 4 * b3 + 2 * b2 + b1;
      if ((l32 & 1) == 0) r_kl[wave][8 * (i >> 2) + 4 * half + (i & 3)] = v1;
    }
    // dk^I += c_I dz^T q^I (keys on M, dims on N; B from the transposed tile)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 da = make_uint4(pack_bf16x2(dz[8 * s + 0] * kScale, dz[8 * s + 1] * kScale),
                                  pack_bf16x2(dz[8 * s + 2] * kScale, dz[8 * s + 3] * kScale),
                                  pack_bf16x2(dz[8 * s + 4] * kScale, dz[8 * s + 5] * kScale),
                                  pack_bf16x2(dz[8 * s + 6] * kScale, dz[8 * s + 7] * kScale));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int o = (32 * dt + l32) * kTq + 2 * (16 * s + 8 * half);
        dk[dt] = mfma32(as_bf16x8(da), as_bf16x8(*reinterpret_cast<const uint4*>(&qit[o])), dk[dt]);
      }
    }
    __syncthreads();  // dzs and r_kl complete

    // dq^I^T of this wave's 32 dims x the pass's queries = k^I^T (c_I dz)^T
    {
      const unsigned char* db = dzs + l32 * kP + half * 16;
      f32x16 q0 = f32x16{}, q1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; s += 2) {
        q0 = mfma32(as_bf16x8(kA[s]), as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s)), q0);
        q1 = mfma32(as_bf16x8(kA[s + 1]),
                    as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s + 32)), q1);
      }
      const f32x16 qacc = q0 + q1;
      // lane = query l32: its 16 values at element 32 wave + 16 half of the
      // partial row (the layout the dq combine reads)
      u16* dst = a.dqpart + static_cast<int64_t>(r_prow[l32]) * kHeadDim + 32 * wave + 16 * half;
      uint4 w0, w1;
      w0.x = pack_bf16x2(qacc[0], qacc[1]);
      w0.y = pack_bf16x2(qacc[2], qacc[3]);
      w0.z = pack_bf16x2(qacc[4], qacc[5]);
      w0.w = pack_bf16x2(qacc[6], qacc[7]);
      w1.x = pack_bf16x2(qacc[8], qacc[9]);
      w1.y = pack_bf16x2(qacc[10], qacc[11]);
      w1.z = pack_bf16x2(qacc[12], qacc[13]);
      w1.w = pack_bf16x2(qacc[14], qacc[15]);
      *reinterpret_cast<uint4*>(dst) = w0;
      *reinterpret_cast<uint4*>(dst + 8) = w1;
    }
    if (tid < 32)
      a.part[r_prow[tid]] =
          make_float2(((r_kl[0][tid] + r_kl[1][tid]) + r_kl[2][tid]) + r_kl[3][tid], 0.f);
    __syncthreads();  // before the next pass's gather overwrites the tiles
  }

  // dk^I of this wave's keys (shared by every group): lane = dim 32 dt + l32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t key = key0 + 32 * wave + 8 * (i >> 2) + 4 * half + (i & 3);
    if (key < key0 + nvalid) {
      float* pk = a.dkI + (b * a.N + key) * kHeadDim + l32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) unsafeAtomicAdd(pk + 32 * dt, dk[dt][i]);
    }
  }
}

struct KlArgs {
  const int32_t* idx;
  const float2* part;
  float* kl;  // [B, G, T]
  int64_t T, r0, rows;
  int32_t G, k, rl_base, group;
};

// loss of a row = the sum of its valid slots' partials, in slot order
__global__ void __launch_bounds__(256) kl_combine_kernel(KlArgs a) {
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (wid >= a.rows) return;
  const int64_t grow = a.r0 + a.rl_base + wid;
  const int64_t b = grow / a.T, t = grow % a.T;
  const int32_t* ir = a.idx + ((b * a.G + a.group) * a.T + t) * a.k;
  float sum = 0.f;
  for (int s = 0; s < a.k && ir[s] >= 0; ++s) sum += a.part[wid * a.k + s].x;
  a.kl[(b * a.G + a.group) * a.T + t] = sum;
}

__global__ void __launch_bounds__(256) ik_zero_kernel(float4* p, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

unsigned nblk_of(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

// The teacher of the KL alignment for the standalone index-branch backward
// (the fused training backward's main stage writes it as a side product): per
// (row, slot, key) of a stage, the mean over the group's heads of the main
// branch's weight exp(q_h . K_j / sqrt(128) - lse_h), masked past the row's
// causal limit.  One workgroup per chunk; the chunk's (query, head) rows (a
// query's heads consecutive) stream through in passes of 32 against the
// block's K rows of wave w's keys (32w..32w+31), held in registers.  The rows
// of pass p + 1 are stored to the second q tile while pass p is scored, so a
// pass has one barrier; the kernel is small (17 KB of LDS), so several
// workgroups share a CU and hide each other's gathers.
template <int HG>
__global__ void __launch_bounds__(256, 2) teacher_kernel(IkArgs a, float* teach) {
  __shared__ __align__(16) unsigned char qs[2][32 * kP];  // the pass's q rows, by parity
  __shared__ float r_l2[2][32];
  __shared__ int r_lim[2][32], r_prow[2][32];
  __shared__ int ents[kChunkQueries];

  const int nchunks = *a.count;
  const int per_xcd = (nchunks + 7) >> 3;
  const int xj = static_cast<int>(blockIdx.x >> 3);
  const int ci = static_cast<int>(blockIdx.x & 7) * per_xcd + xj;
  if (xj >= per_xcd || ci >= nchunks) return;
  const int4 ch = a.chunks[ci];
  const int n = ch.z;
  if (n <= 0) return;
  const int64_t blk = ch.w, bg = ch.x;
  const int g = static_cast<int>(bg) & (a.G - 1);
  const int64_t b = bg >> __builtin_ctz(a.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t key0 = blk * a.Bk;
  // the block's keys (>= 1); rows past them repeat its last key and are masked
  const int nvalid = static_cast<int>(a.N - key0 < a.Bk ? a.N - key0 : a.Bk);
  const int key_w = 32 * wave + l32;
  uint4 kf[8];  // B operand of S: key key_w, dims 16s + 8 half .. + 7
  {
    const int kr = key_w < nvalid ? key_w : nvalid - 1;
    const u16* kp = a.K + (bg * a.N + key0 + kr) * kHeadDim + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = ld16(kp + 16 * s);
  }
  if (tid < n) ents[tid] = a.entries[ch.y + tid];
  __syncthreads();

  const int rows = n * HG;
  const int npass = (rows + 31) / 32;
  const int64_t t0 = a.r0 - b * a.T;
  // A pass's gather, one thread's share: rows 2 rp, 2 rp + 1, dims 8 cc ..
  // 8 cc + 7, plus (cc == 0) the rows' lse, causal limit and (row, slot)
  // index times HG.  Rows past the chunk's end repeat the chunk's first row
  // with lse = +inf and an empty causal range: their weights are 0 and they
  // write nothing.  fetch only issues loads; they are used a pass later.
  const int rp = tid & 15, cc = tid >> 4, r0 = 2 * rp;
  uint4 fq[2];
  float fl[2];
  int flim[2], fprow[2];
  bool fvalid[2];
  auto fetch = [&](int pass) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rr = pass * 32 + r0 + u;
      const bool valid = rr < rows;
      const int qi = valid ? rr / HG : 0;
      const int hh = rr % HG;
      const int e = ents[qi];
      const int64_t t = t0 + (e >> 6);
      const int64_t hq = static_cast<int64_t>(g) * HG + hh;
      fq[u] = ld16(a.q + ((b * a.T + t) * a.Hq + hq) * kHeadDim + 8 * cc);
      fl[u] = a.lse[(b * a.Hq + hq) * a.T + t];
      fvalid[u] = valid;
      flim[u] = valid ? static_cast<int>(min(a.N - a.T + t - key0, static_cast<int64_t>(nvalid - 1)))
                      : -1;  // last key of the block the row sees
      fprow[u] = valid ? (((e >> 6) - a.rl_base) * a.k + (e & 63)) * HG + hh : a.sink + hh;
    }
  };
  auto stash = [&](int pass) {
    const int pb = pass & 1;
    *reinterpret_cast<uint4*>(&qs[pb][r0 * kP + 16 * cc]) = fq[0];
    *reinterpret_cast<uint4*>(&qs[pb][(r0 + 1) * kP + 16 * cc]) = fq[1];
    if (cc == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        r_l2[pb][r0 + u] = fvalid[u] ? fl[u] * kLog2e : INFINITY;
        r_lim[pb][r0 + u] = flim[u];
        r_prow[pb][r0 + u] = fprow[u];
      }
    }
  };
  // the lane's weights are rows m(i) = 8(i/4) + 4 half + i%4; a query's HG
  // head rows are consecutive, so the head sum is in-lane (HG <= 4) or
  // in-lane plus the other half-wave (HG = 8, 16).  Keys past Bk belong to
  // no block (wave-uniform test).
  auto put = [&](const int* rpw, int m, float sum) {
    const int pw = rpw[m];  // (row, slot) index * HG of the query's first head
    if (pw < a.sink)  // read once, by the gradient pass: kept out of the caches
      __builtin_nontemporal_store(sum * (1.f / HG),
                                  teach + static_cast<int64_t>(pw / HG) * a.Bk + key_w);
  };
  const float qscale = kLog2e * kScale;
  fetch(0);
  stash(0);
  fetch(npass > 1 ? 1 : 0);
  __syncthreads();
  for (int pass = 0; pass < npass; ++pass) {
    const int pb = pass & 1;
    if (pass + 1 < npass) {  // qs[pb ^ 1] was last read by pass - 1
      stash(pass + 1);
      fetch(pass + 2 < npass ? pass + 2 : pass + 1);
    }
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    const unsigned char* qa = qs[pb] + l32 * kP + half * 16;
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      s0 = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(qa + 32 * s)), as_bf16x8(kf[s]), s0);
      s1 = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(qa + 32 * s + 32)),
                  as_bf16x8(kf[s + 1]), s1);
    }
    const f32x16 sc = s0 + s1;
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 8 * (i >> 2) + 4 * half + (i & 3);
      const float ex = fast_exp2(fmaf(sc[i], qscale, -r_l2[pb][m]));
      pr[i] = key_w <= r_lim[pb][m] ? ex : 0.f;
    }
    if (32 * wave < a.Bk) {
      const int* rpw = r_prow[pb];
      if constexpr (HG <= 4) {
#pragma unroll
        for (int i = 0; i < 16; i += HG) {
          float sum = 0.f;
#pragma unroll
          for (int j = 0; j < HG; ++j) sum += pr[i + j];
          put(rpw, 8 * (i >> 2) + 4 * half + (i & 3), sum);
        }
      } else if constexpr (HG == 8) {
        float sum[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sum[j] = (pr[4 * j] + pr[4 * j + 1]) + (pr[4 * j + 2] + pr[4 * j + 3]);
        }
        // half h writes queries 2h and 2h + 1 (rows 16h and 16h + 8), each
        // summed over both half-waves
        put(rpw, 16 * half, halves_sum2(sum[0], sum[2]));
        put(rpw, 16 * half + 8, halves_sum2(sum[1], sum[3]));
      } else {
        static_assert(HG == 16, "heads per group");
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a0 += pr[j];
          a1 += pr[8 + j];
        }
        put(rpw, 16 * half, halves_sum2(a0, a1));  // half h writes query h
      }
    }
    __syncthreads();  // pass's tile and row data may be replaced
  }
}

hipError_t launch_kl(const IkArgs& ia, int64_t grid, hipStream_t st) {
  TimedLaunch tl(MSA_KERNEL_INDEX_KL, st);
  hipLaunchKernelGGL(index_kl_teach_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     ia);
  return hipGetLastError();
}

hipError_t launch_teacher(int hg, const IkArgs& ia, float* teach, int64_t grid, hipStream_t st) {
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
  switch (hg) {
    case 8: hipLaunchKernelGGL((teacher_kernel<8>), gd, bd, 0, st, ia, teach); break;
    case 4: hipLaunchKernelGGL((teacher_kernel<4>), gd, bd, 0, st, ia, teach); break;
    case 16: hipLaunchKernelGGL((teacher_kernel<16>), gd, bd, 0, st, ia, teach); break;
    case 2: hipLaunchKernelGGL((teacher_kernel<2>), gd, bd, 0, st, ia, teach); break;
    case 1: hipLaunchKernelGGL((teacher_kernel<1>), gd, bd, 0, st, ia, teach); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t index_kl_prepare(float* dkI, int64_t B, int64_t N, hipStream_t st) {
  const int64_t n4 = B * N * kHeadDim / 4;
  hipLaunchKernelGGL(ik_zero_kernel, dim3(nblk_of(n4, 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(dkI), n4);
  return hipGetLastError();
}

// One stage (group g, row stage sub) of a window inverted by
// launch_invert_window: the teacher (when make_teacher is set; otherwise the
// main backward's stage has written it to teach), the proxy lse pass and its
// combine, the gradient pass, then the slot-ordered sums of the dq^I and loss
// partials.
hipError_t index_kl_stage(const void* qI, const void* kI, const void* q, const void* K,
                          const int32_t* idx, const float* lse, float* teach, bool make_teacher,
                          float* dqI,
                          float* dkI, float* kl, float* lpx, int64_t T, int64_t N, int Hq, int G,
                          int k, int Bk, const AttnWorkspace& w, int64_t r0, int64_t W, int32_t S,
                          int g, int32_t sub, hipStream_t st) {
  const int64_t si = static_cast<int64_t>(g) * S + sub;
  const int32_t rl_base = sub * static_cast<int32_t>(w.stage_rows);
  const int64_t rows = (W - rl_base) < w.stage_rows ? (W - rl_base) : w.stage_rows;
  IkArgs ia;
  ia.qI = static_cast<const u16*>(qI);
  ia.kI = static_cast<const u16*>(kI);
  ia.q = static_cast<const u16*>(q);
  ia.K = static_cast<const u16*>(K);
  ia.lse = lse;
  ia.lpx = lpx;
  ia.teach = teach;
  ia.chunks = w.chunks + si * w.max_chunks;
  ia.entries = w.entries;
  ia.count = w.totals + 4 + si;
  ia.part = w.lpart;
  ia.dqpart = w.opart;
  ia.dkI = dkI;
  ia.T = T;
  ia.N = N;
  ia.r0 = r0;
  ia.Hq = Hq;
  ia.G = G;
  ia.k = k;
  ia.Bk = Bk;
  ia.rl_base = rl_base;
  ia.sink = static_cast<int32_t>(w.sink);
  const int64_t grid = (w.max_chunks + 7) & ~static_cast<int64_t>(7);
  if (make_teacher) {
    const hipError_t et = launch_teacher(Hq / G, ia, teach, grid, st);
    if (et != hipSuccess) return et;
  }
  hipLaunchKernelGGL(index_px_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, ia);
  PxArgs pa;
  pa.idx = idx;
  pa.part = w.lpart;
  pa.lpx = lpx;
  pa.T = T;
  pa.r0 = r0;
  pa.rows = rows;
  pa.G = G;
  pa.k = k;
  pa.rl_base = rl_base;
  pa.group = g;
  hipLaunchKernelGGL(px_combine_kernel, dim3(nblk_of(rows, 256)), dim3(256), 0, st, pa);
  hipError_t e = launch_kl(ia, grid, st);
  if (e != hipSuccess) return e;
  e = launch_dq_combine(idx, w.opart, dqI, T, r0, rows, G, G, k, rl_base, g, st);
  if (e != hipSuccess) return e;
  if (kl) {
    KlArgs ka;
    ka.idx = idx;
    ka.part = w.lpart;
    ka.kl = kl;
    ka.T = T;
    ka.r0 = r0;
    ka.rows = rows;
    ka.G = G;
    ka.k = k;
    ka.rl_base = rl_base;
    ka.group = g;
    hipLaunchKernelGGL(kl_combine_kernel, dim3(nblk_of(rows, 256)), dim3(256), 0, st, ka);
  }
  return hipGetLastError();
}

hipError_t launch_index_kl_backward(const void* qI, const void* kI, const void* q, const void* K,
                                    const int32_t* idx, const float* lse, float* dqI, float* dkI,
                                    float* kl, float* lpx, float* teach, int64_t B, int64_t T,
                                    int64_t N, int Hq, int G, int k, int Bk,
                                    const AttnWorkspace& w, hipStream_t st) {
  hipError_t e = index_kl_prepare(dkI, B, N, st);
  if (e != hipSuccess) return e;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t0 = 0; t0 < T; t0 += w.window) {
      const int64_t W = (T - t0) < w.window ? (T - t0) : w.window;
      int32_t S = 0;
      e = launch_invert_window(idx, b, T, t0, W, N, G, k, Bk, w, &S, st);
      if (e != hipSuccess) return e;
      for (int g = 0; g < G; ++g) {
        for (int32_t sub = 0; sub < S; ++sub) {
          e = index_kl_stage(qI, kI, q, K, idx, lse, teach, true, dqI, dkI, kl, lpx, T, N, Hq,
                             G, k, Bk, w, b * T + t0, W, S, g, sub, st);
          if (e != hipSuccess) return e;
        }
      }
    }
  }
  return hipSuccess;
}

// The fused training backward: both branches per stage from one inversion;
// the main backward's stage writes the teacher of its rows, which the KL
// stage right after reads instead of recomputing the main scores.
hipError_t launch_train_backward(const void* q, const void* K, const void* V, const void* qI,
                                 const void* kI, const int32_t* idx, const void* O,
                                 const float* lse, const void* dO, float* dq, float* dK,
                                 float* dV, float* dqI, float* dkI, float* kl, float* Dr,
                                 float* lpx, float* teach, int64_t B, int64_t T, int64_t N,
                                 int Hq, int G, int k, int Bk, const AttnWorkspace& w,
                                 hipStream_t st) {
  hipError_t e = attn_bwd_prepare(O, dO, dK, dV, Dr, B, T, N, Hq, G, st);
  if (e != hipSuccess) return e;
  e = index_kl_prepare(dkI, B, N, st);
  if (e != hipSuccess) return e;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t0 = 0; t0 < T; t0 += w.window) {
      const int64_t W = (T - t0) < w.window ? (T - t0) : w.window;
      int32_t S = 0;
      e = launch_invert_window(idx, b, T, t0, W, N, G, k, Bk, w, &S, st);
      if (e != hipSuccess) return e;
      const int64_t r0 = b * T + t0;
      for (int g = 0; g < G; ++g) {
        for (int32_t sub = 0; sub < S; ++sub) {
          e = attn_bwd_stage(q, K, V, idx, lse, dO, Dr, dq, dK, dV, teach, T, N, Hq, G, k, Bk, w,
                             r0, W, S, g, sub, st);
          if (e != hipSuccess) return e;
          e = index_kl_stage(qI, kI, q, K, idx, lse, teach, false, dqI, dkI, kl, lpx, T, N, Hq,
                             G, k, Bk, w, r0, W, S, g, sub, st);
          if (e != hipSuccess) return e;
        }
      }
    }
  }
  return hipSuccess;
}

}  // namespace msa
