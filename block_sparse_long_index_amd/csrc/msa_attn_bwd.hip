// msa_attn_bwd.hip -- backward of the main branch of MSA (stage 4) on gfx950:
// dq, dK and dV of exact softmax attention over each row's selected blocks,
// scheduled KV-outer like the forward.
//
// Method: the selection is fixed by the forward (the top-k has no gradient);
// the Flash-MSA training blog (hackernews.jp, "Backward pass") keeps the
// forward's block indices and the main branch's lse for the backward, inverts
// the [batch, group, query, slot] -> block map into block -> queries and
// schedules the sparse KV blocks shared by many queries from that inverse.
// Per (row, head), over the row's support keys j (scale c = 1/sqrt(128)):
//   P_j = exp(c q.K_j - lse),  dP_j = dO.V_j,  D = dO.O = sum_j P_j dP_j,
//   dS_j = P_j (dP_j - D),  dq = c sum_j dS_j K_j,
//   dK_j += c dS_j q,  dV_j += P_j dO.
//
// One workgroup per chunk (b, g, block, <= 128 queries, all heads of the
// group): the block's K, V and K^T stay in registers while the chunk's
// (query, head) rows stream through in passes of 32.  Score waves 0-3 own keys 32w..32w+31 for S, dP and dS and dims
// 32w..32w+31 of the pass's dq; key-gradient waves 4-7 hold the dK / dV
// accumulators of the same keys for the whole chunk and gather the rows.  The
// dq of a (row, slot) pair is written as a bf16 partial and the partials of a
// row are summed in slot order by dq_combine_kernel; dK and dV of a chunk are
// added to the fp32 outputs with one atomic add per element (a block's queries
// may span several chunks and stages).
#include "msa_common.h"
#include "msa_internal.h"

#include <math.h>

namespace msa {

constexpr int kBP = 272;  // LDS row pitch (bytes) of every 128-column bf16 tile
constexpr int kTP = 80;   // LDS row pitch of the transposed 32-row q and dO tiles
// One pass's P and dS operands for the dK / dV products: [score wave][j][lane]
// 16-byte slots, j = 0, 1: P of k-steps 0, 1; j = 2, 3: dS of k-steps 0, 1.
constexpr int kPdBytes = 4 * 4 * 64 * 16;

// Column of pass row r (0..31) in the transposed q / dO tiles.  The dK / dV
// products take a lane's P (or dS) values of k-step s in the order
// rows 16s + 8(j/4) + 4 half + j%4, j = 0..7; storing row 16s + o at column
// 16s + 8 ((o >> 2) & 1) + 4 (o >> 3) + o % 4 puts exactly those rows side by
// side, so each B operand is one 16-byte LDS read.  Rows 2i and 2i + 1 stay
// adjacent.
__device__ __forceinline__ int tpos(int r) {
  const int o = r & 15;
  return (r & 16) + 8 * ((o >> 2) & 1) + 4 * (o >> 3) + (o & 3);
}

struct BwdArgs {
  const u16* q;
  const u16* K;
  const u16* V;
  const u16* dO;
  const float* lse;       // [B, Hq, T], natural log
  const float* Dr;        // [B, T, Hq]: dO . O
  const int4* chunks;     // this stage's chunk list
  const int32_t* entries;
  const int32_t* count;
  u16* dqpart;            // [stage rows, k, hg, 128] bf16
  float* dK;              // [B, G, N, 128]
  float* dV;
  float* teach;           // [stage rows, k, Bk] fp32: the teacher of each (row, slot), or null
  int64_t T, N, r0;       // r0: global row (b*T + t) of window row 0
  int32_t Hq, G, k, Bk;
  int32_t rl_base;        // first window row of this stage
  int32_t sink;           // spare partial row (hg rows) for rows past a chunk's end
};

// TW: also write the teacher of the index branch's KL alignment, the mean over
// the group's heads of P, per (row, slot, key).
//
// Eight waves, two per SIMD, in two roles that run side by side:
//  * score waves 0-3: wave w keeps the K and V rows of keys 32w..32w+31 and
//    the K^T rows of dims 32w..32w+31 in registers; per pass it forms S and
//    dP (rows x its keys), P and dS, and the dq of the previous pass for its
//    dims (from the dS tile of all keys in LDS);
//  * key-gradient waves 4-7: wave 4 + w holds the dK and dV accumulators of
//    the same 32 keys and adds pass p - 1's P^T dO and dS^T q while the score
//    waves work on pass p; they also store pass p + 1's q / dO rows (loaded a
//    pass earlier) and issue the loads of pass p + 2.
// The score waves hand P and dS over through LDS in their own register order
// (a 16-byte slot per lane and k-step), which is exactly the A operand layout
// of the key-gradient products, so neither side rearranges them.  Every
// buffer a pass writes is distinct from those the other role reads in the
// same pass (two row tiles, three transposed tiles, two P / dS and dS tiles,
// three partial-row lists), so a pass ends with a single workgroup barrier,
// reached by both roles the same number of times.
template <int HG, bool TW>
__global__ void __launch_bounds__(512, 1) kv_outer_bwd_kernel(BwdArgs a) {
  constexpr int kRowTile = 32 * kBP;   // 32 rows x 128 dims, row-major
  constexpr int kTTile = 128 * kTP;    // 128 dims x 32 rows, transposed
  __shared__ __align__(16) unsigned char qs[2][kRowTile];    // the pass's q rows, by parity
  __shared__ __align__(16) unsigned char gs[2][kRowTile];    // the pass's dO rows
  // q^T and dO^T tiles [d][tpos(row)] of passes p mod 3; before the first
  // pass the same bytes stage the block's K^T [d][key]
  __shared__ __align__(16) unsigned char tt[6 * kTTile];
  __shared__ __align__(16) unsigned char dss[2][kRowTile];   // dS [row][key], bf16, scaled by c
  __shared__ __align__(16) unsigned char pd[2][kPdBytes];    // P, dS operands [wave][j][lane]
  __shared__ float r_l2[2][32], r_D[2][32];
  __shared__ int r_lim[2][32], r_prow[3][32];
  __shared__ int ents[kChunkQueries];  // the chunk's (row << 6 | slot) entries
  static_assert(6 * kTTile >= 128 * kBP, "K^T staging fits the transposed tiles");

  // the chunk list is dealt to the 8 XCDs in contiguous eighths (as forward)
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

  const int64_t key0 = blk * a.Bk;
  // the block's keys (>= 1); K^T columns past them are zero
  const int nvalid = static_cast<int>(a.N - key0 < a.Bk ? a.N - key0 : a.Bk);
  const u16* Kb = a.K + (bg * a.N + key0) * kHeadDim;
  const u16* Vb = a.V + (bg * a.N + key0) * kHeadDim;

  // K^T: 64 key pairs x 16 chunks of 8 dims, staged as 32-bit (key, key + 1)
  // words.  Keys past N are zero.
  unsigned char* kt = tt;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 512 * j;
    const int kp = i & 63, c = i >> 6;
    const int k0 = 2 * kp;
    const uint4 y0 = ld16(Kb + (k0 < nvalid ? k0 : nvalid - 1) * kHeadDim + 8 * c);
    const uint4 y1 = ld16(Kb + (k0 + 1 < nvalid ? k0 + 1 : nvalid - 1) * kHeadDim + 8 * c);
    const uint4 x0 = k0 < nvalid ? y0 : make_uint4(0, 0, 0, 0);
    const uint4 x1 = k0 + 1 < nvalid ? y1 : make_uint4(0, 0, 0, 0);
    const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w};
    const uint32_t w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t hi = (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      *reinterpret_cast<uint32_t*>(&kt[(8 * c + e) * kBP + 2 * k0]) = lo | (hi << 16);
    }
  }
  for (int i = tid; i < n; i += 512) ents[i] = a.entries[ch.y + i];
  __syncthreads();
  const int rows = n * HG;
  const int npass = (rows + 31) / 32;
  const int64_t t0 = a.r0 - b * a.T;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kScale = 0.08838834764831845f;  // 1/sqrt(128)

  if (wave >= 4) {
    // ---- key-gradient waves ----
    const int gw = wave - 4;
    // A pass's gather, one thread's share: rows 2 rp and 2 rp + 1, dims
    // 8 cc .. 8 cc + 7 of q and dO, plus (for cc == 0) the rows' lse, D,
    // causal limit and partial row.  Rows past the chunk's end repeat the
    // chunk's first row with lse = +inf and an empty causal range, so their P
    // and dS are 0 and they add nothing to dK and dV; their dq goes to the
    // sink row.  (rp varies fastest across lanes: one wave's stores to a
    // transposed tile row then hit 16 consecutive words instead of one bank 16
    // times.)
    const int t = tid - 256;
    const int rp = t & 15, cc = t >> 4;
    const int r0 = 2 * rp;
    uint4 fq[2], fg[2];
    float fl[2], fD[2];
    int flim[2], fprow[2];
    bool fvalid[2];
    // fetch only issues loads (every lane, valid addresses); they are used a
    // pass later, by stash
    auto fetch = [&](int pass) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = pass * 32 + r0 + u;
        const bool valid = rr < rows;
        const int qi = valid ? rr / HG : 0;
        const int hh = rr % HG;
        const int e = ents[qi];
        const int64_t tt_ = t0 + (e >> 6);
        const int64_t hq = static_cast<int64_t>(g) * HG + hh;
        const int64_t off = ((b * a.T + tt_) * a.Hq + hq) * kHeadDim + 8 * cc;
        fq[u] = ld16(a.q + off);
        fg[u] = ld16(a.dO + off);
        fl[u] = a.lse[(b * a.Hq + hq) * a.T + tt_];
        fD[u] = a.Dr[(b * a.T + tt_) * a.Hq + hq];
        fvalid[u] = valid;
        flim[u] = valid ? static_cast<int>(min(a.N - a.T + tt_ - key0,
                                               static_cast<int64_t>(nvalid - 1)))
                        : -1;  // last key of the block the row sees
        fprow[u] = valid ? (((e >> 6) - a.rl_base) * a.k + (e & 63)) * HG + hh : a.sink + hh;
      }
    };
    // the row-major tiles and the rows' scalars (read by the score waves) and
    // the transposed tiles (read by this role), all for pass `pass`
    auto stash = [&](int pass) {
      const int pb = pass & 1;
      *reinterpret_cast<uint4*>(&qs[pb][r0 * kBP + 16 * cc]) = fq[0];
      *reinterpret_cast<uint4*>(&qs[pb][(r0 + 1) * kBP + 16 * cc]) = fq[1];
      *reinterpret_cast<uint4*>(&gs[pb][r0 * kBP + 16 * cc]) = fg[0];
      *reinterpret_cast<uint4*>(&gs[pb][(r0 + 1) * kBP + 16 * cc]) = fg[1];
      if (cc == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          r_l2[pb][r0 + u] = fvalid[u] ? fl[u] * kLog2e : INFINITY;
          r_D[pb][r0 + u] = fvalid[u] ? fD[u] : 0.f;
          r_lim[pb][r0 + u] = flim[u];
          r_prow[pass % 3][r0 + u] = fprow[u];
        }
      }
      const int P = tpos(r0);  // even; row r0 + 1 sits at P + 1
      const uint32_t q0[4] = {fq[0].x, fq[0].y, fq[0].z, fq[0].w};
      const uint32_t q1[4] = {fq[1].x, fq[1].y, fq[1].z, fq[1].w};
      const uint32_t g0[4] = {fg[0].x, fg[0].y, fg[0].z, fg[0].w};
      const uint32_t g1[4] = {fg[1].x, fg[1].y, fg[1].z, fg[1].w};
      unsigned char* qTw = tt + (2 * (pass % 3)) * kTTile;
      unsigned char* gTw = qTw + kTTile;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const int o = (8 * cc + e) * kTP + 2 * P;
        *reinterpret_cast<uint32_t*>(&qTw[o]) =
            ((q0[e >> 1] >> sh) & 0xffffu) | (((q1[e >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint32_t*>(&gTw[o]) =
            ((g0[e >> 1] >> sh) & 0xffffu) | (((g1[e >> 1] >> sh) & 0xffffu) << 16);
      }
    };
    // dV += P^T dO and dK += dS^T q over pass p's rows: keys on M, dims on N;
    // A = the score wave's P / dS slots, B = the transposed tiles (see tpos).
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      dk[dt] = f32x16{};
      dv[dt] = f32x16{};
    }
    auto key_grads = [&](int p) {
      const unsigned char* pdr = pd[p & 1] + (gw * 256 + lane) * 16;
      const unsigned char* qTr = tt + (2 * (p % 3)) * kTTile;
      const unsigned char* gTr = qTr + kTTile;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 pa = *reinterpret_cast<const uint4*>(pdr + 1024 * s);
        const uint4 da = *reinterpret_cast<const uint4*>(pdr + 1024 * (2 + s));
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int o = (32 * dt + l32) * kTP + 2 * (16 * s + 8 * half);
          dv[dt] = mfma32(as_bf16x8(pa), as_bf16x8(*reinterpret_cast<const uint4*>(&gTr[o])),
                          dv[dt]);
          dk[dt] = mfma32(as_bf16x8(da), as_bf16x8(*reinterpret_cast<const uint4*>(&qTr[o])),
                          dk[dt]);
        }
      }
    };
    fetch(0);
    __syncthreads();  // the score waves have their K^T rows: the staging may be replaced
    stash(0);
    fetch(npass > 1 ? 1 : 0);
    __syncthreads();  // pass 0's rows are in LDS
    for (int pass = 0; pass < npass; ++pass) {
      if (pass > 0) key_grads(pass - 1);
      if (pass + 1 < npass) {
        stash(pass + 1);
        fetch(pass + 2 < npass ? pass + 2 : pass + 1);
      }
      __syncthreads();
    }
    key_grads(npass - 1);

    // dK, dV of this wave's keys: lane = dim 32 dt + l32, keys m(i)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = key0 + 32 * gw + 8 * (i >> 2) + 4 * half + (i & 3);
      if (key < key0 + nvalid) {
        float* pk = a.dK + (bg * a.N + key) * kHeadDim + l32;
        float* pv = a.dV + (bg * a.N + key) * kHeadDim + l32;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          unsafeAtomicAdd(pk + 32 * dt, dk[dt][i]);
          unsafeAtomicAdd(pv + 32 * dt, dv[dt][i]);
        }
      }
    }
  } else {
    // ---- score waves ----
    const int key_w = 32 * wave + l32;  // this lane's key in S, dP, dS
    const float qscale = kLog2e * kScale;
    // this wave's operands that stay fixed for the whole chunk, kept in
    // registers: its keys' K and V rows (B of S and dP) and its dims' K^T
    // rows (A of dq), 8 k-steps each.  K / V rows past the block's end repeat
    // its last key (their P is masked to 0).
    uint4 kf[8], vf[8], tf[8];
    {
      const int kr = key_w < nvalid ? key_w : nvalid - 1;
      const u16* kp = Kb + static_cast<int64_t>(kr) * kHeadDim + 8 * half;
      const u16* vp = Vb + static_cast<int64_t>(kr) * kHeadDim + 8 * half;
      const unsigned char* ka = kt + (32 * wave + l32) * kBP + half * 16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        kf[s] = ld16(kp + 16 * s);
        vf[s] = ld16(vp + 16 * s);
        tf[s] = *reinterpret_cast<const uint4*>(ka + 32 * s);
      }
    }
    // dq^T of this wave's 32 dims x pass p's 32 rows = K^T dS^T over the 128
    // keys, from dss[p & 1]; stored as the (row, slot) partial, lane = row
    // l32: the lane's 16 values (dims 32 wave + 8(i/4) + 4 half + i%4) go
    // contiguously to element 32 wave + 16 half of the partial row (see
    // dq_combine_kernel).
    auto store_dq = [&](int p, const f32x16& qacc) {
      const int prow = r_prow[p % 3][l32];
      u16* dst = a.dqpart + static_cast<int64_t>(prow) * kHeadDim + 32 * wave + 16 * half;
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
    };

    // The teacher of the pass's queries at this lane's key: the lane's P
    // values are rows m(i) = 8(i/4) + 4 half + i%4, a query's HG head rows are
    // consecutive, so the head sum is in-lane (HG <= 4), in-lane plus the
    // other half-wave (HG = 8, HG = 16).  Rows past the chunk's end (partial
    // row >= sink) write nothing; keys past Bk belong to no block
    // (wave-uniform test).
    auto write_teacher = [&](int pass, const float* pr) {
      if (32 * wave >= a.Bk) return;
      const int* rpw = r_prow[pass % 3];
      auto put = [&](int m, float sum) {
        const int pw = rpw[m];  // (row, slot) entry * HG for the query's first head
        if (pw < a.sink)  // read once, by the KL pass: kept out of the caches
          __builtin_nontemporal_store(sum * (1.f / HG),
                                      a.teach + static_cast<int64_t>(pw / HG) * a.Bk + key_w);
      };
      if constexpr (HG <= 4) {
#pragma unroll
        for (int i = 0; i < 16; i += HG) {
          float sum = 0.f;
#pragma unroll
          for (int j = 0; j < HG; ++j) sum += pr[i + j];
          put(8 * (i >> 2) + 4 * half + (i & 3), sum);
        }
      } else if constexpr (HG == 8) {
        float sum[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sum[j] = (pr[4 * j] + pr[4 * j + 1]) + (pr[4 * j + 2] + pr[4 * j + 3]);
        }
        // half h writes queries 2h and 2h + 1 (rows 16h and 16h + 8), each
        // summed over both half-waves
        put(16 * half, halves_sum2(sum[0], sum[2]));
        put(16 * half + 8, halves_sum2(sum[1], sum[3]));
      } else {
        static_assert(HG == 16, "heads per group");
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s0 += pr[j];
          s1 += pr[8 + j];
        }
        put(16 * half, halves_sum2(s0, s1));  // half h writes query h
      }
    };

    __syncthreads();  // this role's K^T rows are read: the staging may be replaced
    __syncthreads();  // pass 0's rows are in LDS
    // Pass p: the S / dP products of pass p run beside the dq product of pass
    // p - 1 (two independent MFMA streams), then P and dS: into dss[p & 1]
    // (row-major, for the next pass's dq) and into pd[p & 1] (the key-gradient
    // waves' operands).
    for (int pass = 0; pass < npass; ++pass) {
      const int pb = pass & 1;
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      f32x16 q0 = f32x16{}, q1 = f32x16{};
      // raised priority while issuing the MFMAs: the key-gradient waves
      // wait on the P / dS this wave writes next
      __builtin_amdgcn_s_setprio(1);
      {
        const unsigned char* qa = qs[pb] + l32 * kBP + half * 16;
        const unsigned char* ga = gs[pb] + l32 * kBP + half * 16;
        // dS of pass p - 1 (for pass 0 this reads the other buffer's stale
        // contents, and the result is not stored)
        const unsigned char* db = dss[pb ^ 1] + l32 * kBP + half * 16;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          sacc = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(qa + 32 * s)), as_bf16x8(kf[s]),
                        sacc);
          pacc = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(ga + 32 * s)), as_bf16x8(vf[s]),
                        pacc);
          if (s & 1)
            q1 = mfma32(as_bf16x8(tf[s]), as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s)),
                        q1);
          else
            q0 = mfma32(as_bf16x8(tf[s]), as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s)),
                        q0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // P and c*dS; lane: key key_w, rows m(i) = 8(i/4) + 4 half + i%4
      unsigned char* dsw = dss[pb];
      float pr[16], dsr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * half + (i & 3);
        const float ex = fast_exp2(fmaf(sacc[i], qscale, -r_l2[pb][m]));
        const float p = key_w <= r_lim[pb][m] ? ex : 0.f;
        pr[i] = p;
        dsr[i] = p * (pacc[i] - r_D[pb][m]) * kScale;
        *reinterpret_cast<u16*>(&dsw[m * kBP + 2 * key_w]) = f32_to_bf16(dsr[i]);
      }
      if (pass > 0) store_dq(pass - 1, q0 + q1);
      unsigned char* pdw = pd[pb] + (wave * 256 + lane) * 16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *reinterpret_cast<uint4*>(pdw + 1024 * s) =
            make_uint4(pack_bf16x2(pr[8 * s + 0], pr[8 * s + 1]),
                       pack_bf16x2(pr[8 * s + 2], pr[8 * s + 3]),
                       pack_bf16x2(pr[8 * s + 4], pr[8 * s + 5]),
                       pack_bf16x2(pr[8 * s + 6], pr[8 * s + 7]));
        *reinterpret_cast<uint4*>(pdw + 1024 * (2 + s)) =
            make_uint4(pack_bf16x2(dsr[8 * s + 0], dsr[8 * s + 1]),
                       pack_bf16x2(dsr[8 * s + 2], dsr[8 * s + 3]),
                       pack_bf16x2(dsr[8 * s + 4], dsr[8 * s + 5]),
                       pack_bf16x2(dsr[8 * s + 6], dsr[8 * s + 7]));
      }
      if constexpr (TW) write_teacher(pass, pr);
      __syncthreads();
    }
    {  // dq of the last pass
      const unsigned char* db = dss[(npass - 1) & 1] + l32 * kBP + half * 16;
      f32x16 q0 = f32x16{}, q1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; s += 2) {
        q0 = mfma32(as_bf16x8(tf[s]), as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s)), q0);
        q1 = mfma32(as_bf16x8(tf[s + 1]),
                    as_bf16x8(*reinterpret_cast<const uint4*>(db + 32 * s + 32)), q1);
      }
      store_dq(npass - 1, q0 + q1);
    }
  }
}

// D = dO . O per (row, head): 16 lanes per row, fp32.
__global__ void __launch_bounds__(256) bwd_rowdot_kernel(const u16* O, const u16* dO, float* Dr,
                                                         int64_t nrows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = i >> 4;
  const int part = static_cast<int>(i & 15);
  float s = 0.f;
  if (row < nrows) {
    const uint4 o = ld16(O + row * kHeadDim + 8 * part);
    const uint4 d = ld16(dO + row * kHeadDim + 8 * part);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s = fmaf(__uint_as_float(ow[u] << 16), __uint_as_float(dw[u] << 16), s);
      s = fmaf(__uint_as_float(ow[u] & 0xffff0000u), __uint_as_float(dw[u] & 0xffff0000u), s);
    }
  }
  s += __shfl_xor(s, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  if (row < nrows && part == 0) Dr[row] = s;
}

__global__ void __launch_bounds__(256) bwd_zero_kernel(float4* p, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

struct DqArgs {
  const int32_t* idx;
  const u16* dqpart;
  float* dq;
  int64_t T, r0, rows;  // rows: window rows rl_base .. rl_base + rows - 1
  int32_t Hq, G, k, rl_base, group;
};

// dq of a row = the sum of its valid slots' partials, in slot order.  One wave
// per (row, stage group); 16 lanes per head, one 8-value piece per lane.  A
// partial row holds its 128 dims in the KV-outer kernel's register order:
// piece p (elements 8p .. 8p + 7) is wave w = p / 4, half h = (p / 2) % 2,
// groups a = 2 (p % 2) + {0, 1}, i.e. dims 32 w + 8 a + 4 h + {0, 1, 2, 3}.
template <int HG>
__global__ void __launch_bounds__(256) dq_combine_kernel(DqArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wid >= a.rows) return;  // uniform per wave
  const int64_t grow = a.r0 + a.rl_base + wid;  // b * T + t
  const int64_t b = grow / a.T, t = grow % a.T;
  const int32_t* ir = a.idx + ((b * a.G + a.group) * a.T + t) * a.k;
  const int nval = __popcll(__ballot(lane < a.k && ir[lane < a.k ? lane : 0] >= 0));
  const int piece = lane & 15;
#pragma unroll
  for (int h0 = 0; h0 < HG; h0 += 4) {
    const int h = h0 + (lane >> 4);
    if (h < HG) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < nval; ++s) {
        const int64_t prow = (wid * a.k + s) * HG + h;
        const uint4 v = ld16_once(a.dqpart + prow * kHeadDim + 8 * piece);
        const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc[2 * u] += __uint_as_float(vw[u] << 16);
          acc[2 * u + 1] += __uint_as_float(vw[u] & 0xffff0000u);
        }
      }
      const int d0 = 32 * (piece >> 2) + 16 * (piece & 1) + 4 * ((piece >> 1) & 1);
      float* dst =
          a.dq + (grow * a.Hq + static_cast<int64_t>(a.group) * HG + h) * kHeadDim + d0;
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(dst + 8) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

template <int HG>
static hipError_t launch_bwd_stage(const BwdArgs& ba, const DqArgs& da, int64_t grid_chunks,
                                   hipStream_t st) {
  const int64_t grid = (grid_chunks + 7) & ~static_cast<int64_t>(7);
  {
    TimedLaunch tl(MSA_KERNEL_ATTN_BACKWARD, st);
    if (ba.teach)
      hipLaunchKernelGGL((kv_outer_bwd_kernel<HG, true>), dim3(static_cast<unsigned>(grid)),
                         dim3(512), 0, st, ba);
    else
      hipLaunchKernelGGL((kv_outer_bwd_kernel<HG, false>), dim3(static_cast<unsigned>(grid)),
                         dim3(512), 0, st, ba);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_combine_kernel<HG>), dim3(static_cast<unsigned>((da.rows + 3) / 4)),
                     dim3(256), 0, st, da);
  return hipGetLastError();
}

static hipError_t dispatch_bwd(int hg, const BwdArgs& ba, const DqArgs& da, int64_t grid,
                               hipStream_t st) {
  switch (hg) {
    case 8: return launch_bwd_stage<8>(ba, da, grid, st);
    case 4: return launch_bwd_stage<4>(ba, da, grid, st);
    case 16: return launch_bwd_stage<16>(ba, da, grid, st);
    case 2: return launch_bwd_stage<2>(ba, da, grid, st);
    case 1: return launch_bwd_stage<1>(ba, da, grid, st);
  }
  return hipErrorInvalidValue;
}

// The slot-ordered partial sum on its own (one value set per (row, group):
// hg = 1, out [rows, outer, 128] with outer = groups).
hipError_t launch_dq_combine(const int32_t* idx, const uint16_t* part, float* out, int64_t T,
                             int64_t r0, int64_t rows, int outer, int G, int k, int rl_base,
                             int group, hipStream_t st) {
  DqArgs da;
  da.idx = idx;
  da.dqpart = part;
  da.dq = out;
  da.T = T;
  da.r0 = r0;
  da.rows = rows;
  da.Hq = outer;
  da.G = G;
  da.k = k;
  da.rl_base = rl_base;
  da.group = group;
  hipLaunchKernelGGL((dq_combine_kernel<1>), dim3(static_cast<unsigned>((rows + 3) / 4)),
                     dim3(256), 0, st, da);
  return hipGetLastError();
}

static unsigned nblocks_of(int64_t n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

// Zero dK and dV; D = dO . O for every (row, head).
hipError_t attn_bwd_prepare(const void* O, const void* dO, float* dK, float* dV, float* Dr,
                            int64_t B, int64_t T, int64_t N, int Hq, int G, hipStream_t st) {
  const int64_t n4 = B * G * N * kHeadDim / 4;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(nblocks_of(n4, 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(dK), n4);
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(nblocks_of(n4, 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(dV), n4);
  const int64_t nrows = B * T * Hq;
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3(nblocks_of(nrows * 16, 256)), dim3(256), 0, st,
                     static_cast<const u16*>(O), static_cast<const u16*>(dO), Dr, nrows);
  return hipGetLastError();
}

// One stage (group g, row stage sub) of a window inverted by
// launch_invert_window: the KV-outer launch writes the stage's dq partials
// (and the teacher when teach is set) and adds its chunks' dK / dV; the dq
// combine right after sums the partials.
hipError_t attn_bwd_stage(const void* q, const void* K, const void* V, const int32_t* idx,
                          const float* lse, const void* dO, const float* Dr, float* dq,
                          float* dK, float* dV, float* teach, int64_t T, int64_t N, int Hq,
                          int G, int k, int Bk, const AttnWorkspace& w, int64_t r0, int64_t W,
                          int32_t S, int g, int32_t sub, hipStream_t st) {
  const int64_t si = static_cast<int64_t>(g) * S + sub;
  const int32_t rl_base = sub * static_cast<int32_t>(w.stage_rows);
  BwdArgs ba;
  ba.q = static_cast<const u16*>(q);
  ba.K = static_cast<const u16*>(K);
  ba.V = static_cast<const u16*>(V);
  ba.dO = static_cast<const u16*>(dO);
  ba.lse = lse;
  ba.Dr = Dr;
  ba.chunks = w.chunks + si * w.max_chunks;
  ba.entries = w.entries;
  ba.count = w.totals + 4 + si;
  ba.dqpart = w.opart;
  ba.dK = dK;
  ba.dV = dV;
  ba.teach = teach;
  ba.T = T;
  ba.N = N;
  ba.r0 = r0;
  ba.Hq = Hq;
  ba.G = G;
  ba.k = k;
  ba.Bk = Bk;
  ba.rl_base = rl_base;
  ba.sink = static_cast<int32_t>(w.sink);
  DqArgs da;
  da.idx = idx;
  da.dqpart = w.opart;
  da.dq = dq;
  da.T = T;
  da.r0 = r0;
  da.rows = (W - rl_base) < w.stage_rows ? (W - rl_base) : w.stage_rows;
  da.Hq = Hq;
  da.G = G;
  da.k = k;
  da.rl_base = rl_base;
  da.group = g;
  return dispatch_bwd(Hq / G, ba, da, w.max_chunks, st);
}

// Per sequence and window of rows: the inversion, then the stages in
// group-major order.
hipError_t launch_attn_backward(const void* q, const void* K, const void* V,
                                const int32_t* idx, const void* O, const float* lse,
                                const void* dO, float* dq, float* dK, float* dV, float* Dr,
                                int64_t B, int64_t T, int64_t N, int Hq, int G, int k, int Bk,
                                const AttnWorkspace& w, hipStream_t st) {
  hipError_t e = attn_bwd_prepare(O, dO, dK, dV, Dr, B, T, N, Hq, G, st);
  if (e != hipSuccess) return e;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t0 = 0; t0 < T; t0 += w.window) {
      const int64_t W = (T - t0) < w.window ? (T - t0) : w.window;
      int32_t S = 0;
      e = launch_invert_window(idx, b, T, t0, W, N, G, k, Bk, w, &S, st);
      if (e != hipSuccess) return e;
      for (int g = 0; g < G; ++g) {
        for (int32_t sub = 0; sub < S; ++sub) {
          e = attn_bwd_stage(q, K, V, idx, lse, dO, Dr, dq, dK, dV, nullptr, T, N, Hq, G, k, Bk,
                             w, b * T + t0, W, S, g, sub, st);
          if (e != hipSuccess) return e;
        }
      }
    }
  }
  return hipSuccess;
}

}  // namespace msa
