// msa_select.hip -- index branch of MSA on gfx950: token scores, causal block
// max pooling and the exp-free top-k with the forced local block.
//
// Method: MSA study notes (dimensionstp.github.io/study-concept/msa), section
// 2-3, the displayed equations for s, S and the block set; section 3-2 (max
// pooling over causally visible token scores); section 3-4 (forced local
// block); section 3-5 "Exp-free Top-k" (ranking raw scores needs no
// max/exp/sum).  The fused kernel keeps each row's running top-k in registers
// while key blocks stream by, as the Flash-MSA blog (hackernews.jp) describes
// for its proxy attention; the blog sets the local block's score to +inf, we
// leave the local block out of the candidates and append it, which is the
// same selection.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_topk.h"

#include <limits.h>
#include <math.h>

namespace msa {

// ---------------------------------------------------------------------------
// Tile kernel: one workgroup per (sequence, tile of QT consecutive positions).
// QT divides Bk = 128, so every query of a tile has the same local block L and
// the candidate blocks 0..L-1 are fully visible: no causal masking is needed
// except in the local block itself (scored only when S is written).
//
// Columns of the score tile are (query, group) pairs c = q * G + g; keys are
// on the MFMA M side, so each lane's accumulator holds 16 keys of one column
// and the 128-key block max is an in-register max plus one exchange between
// the two half-waves.  Each wave owns 64 columns (two 32-column MFMA tiles);
// its q^I fragments stay in registers for the whole kernel.  k^I blocks
// (32 KB) stream through double-buffered LDS, shared by all waves.
// ---------------------------------------------------------------------------
#ifndef MSA_TILE_COLS
#define MSA_TILE_COLS 512
#endif
template <int G>
struct TileShape {
  static constexpr int QT = (MSA_TILE_COLS / G) < 128 ? (MSA_TILE_COLS / G) : 128;
  static constexpr int NCOL = QT * G;
  static constexpr int NW = NCOL / 64;
  static constexpr int NT = NW * 64;
};

struct TileArgs {
  const u16* qI;
  const u16* kI;
  float* S;         // scores of the window's rows: [B, G, Tw, NB]
  int32_t* idx;     // [B, G, T, k]
  int64_t T, N;
  int64_t t0, Tw;   // this launch's query rows: t0 .. t0 + Tw - 1
  int64_t tile_hi;  // last position tile; workgroups run heaviest first
  int64_t nitems;   // (sequence, position tile) work items
  int32_t* counter; // non-null: workgroups take items from this counter
  int32_t NB, k, B;
  int32_t wgs;      // workgroups to launch (0: one per item)
};

// Insert (x, xi) into a list sorted by score descending, equal scores kept in
// arrival order (an entry already in the list stays ahead of an equal x; x
// below the last entry leaves the list unchanged).  The new score at position
// i is the median of (ts[i], ts[i-1], x), one v_med3 per entry; an index moves
// with its score: position i takes x's index where x beats ts[i] but not
// ts[i-1], and ts[i-1]'s where it beats both.
template <int CAP>
__device__ __forceinline__ void topk_insert(float (&ts)[CAP], int (&ti)[CAP],
                                            float x, int xi) {
  bool c[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) c[i] = x > ts[i];
#pragma unroll
  for (int i = CAP - 1; i > 0; --i) {
    ti[i] = c[i] ? (c[i - 1] ? ti[i - 1] : xi) : ti[i];
    ts[i] = __builtin_amdgcn_fmed3f(ts[i], ts[i - 1], x);
  }
  ti[0] = c[0] ? xi : ti[0];
  ts[0] = fmaxf(ts[0], x);
}

template <int CAP>
__device__ __forceinline__ void sort_ascending(int (&v)[CAP]) {
#pragma unroll
  for (int round = 0; round < CAP; ++round) {
#pragma unroll
    for (int i = round & 1; i + 1 < CAP; i += 2) {
      const int lo = min(v[i], v[i + 1]);
      const int hi = max(v[i], v[i + 1]);
      v[i] = lo;
      v[i + 1] = hi;
    }
  }
}

// F8: q^I and k^I are OCP e4m3 bytes instead of bf16.  A k^I row is then
// 128 B; in LDS the rows sit 144 B apart (16 consecutive rows read at the
// same column hit distinct banks) instead of the bf16 tile's chunk swizzle.
// BK: the block size of the scores written (WRITE_S): each 128-key chunk
// holds 128 / BK blocks, one per BK / 32 key tiles.  The fused selection
// (!WRITE_S) takes BK = 128.
template <int G, bool F8>
struct TileRing {
  // The LDS ring of k^I blocks of the tile body (described there).
  static constexpr int D = TileShape<G>::NT < 512 ? 1 : (F8 ? 4 : 2);
  static constexpr int R = 2 * D;
  static constexpr int PITCH = F8 ? 128 : 256;  // bytes per key row in LDS
};

// One work item (sequence b = item % B, position tile tile_hi - item / B).
template <int G, int CAP, bool WRITE_S, bool F8, int BK>
__device__ __forceinline__ void index_tile(
    const TileArgs& a, int64_t item,
    unsigned char (*kbuf)[128 * TileRing<G, F8>::PITCH]) {
  static_assert(BK == 32 || BK == 64 || BK == 128, "block of 32, 64 or 128 keys");
  static_assert(WRITE_S || BK == 128, "the fused selection takes 128-key blocks");
  constexpr int TPB = BK / 32;   // key tiles per block
  constexpr int BPC = 128 / BK;  // blocks per 128-key chunk
  using TS = TileShape<G>;
  constexpr int QT = TS::QT, NT = TS::NT;
  constexpr int ROWB = F8 ? 128 : 256;      // bytes per k^I / q^I row
  constexpr int CPR = ROWB / 16;            // 16-B chunks per row
  constexpr int PITCH = F8 ? 128 : 256;     // bytes per key row in LDS
  constexpr int PF = 128 * CPR / NT;        // 16-B chunks per thread per block
  static_assert(PF * NT == 128 * CPR, "block chunks must split evenly over the threads");
  // A ring of R = 2D block buffers with a prefetch distance of D: block kb+D
  // is loaded into buffer (kb+D) % R while block kb is scored; that buffer
  // was last read for block kb-D.  The workgroup then needs a barrier only
  // after every D-th block (and after the last): any D consecutive blocks
  // contain one barrier, which both publishes each loaded block before its
  // use (loaded D blocks ahead) and is passed by every wave after it read the
  // block D back before that buffer is reused.  D = 2 for bf16 (4 x 32 KB of
  // LDS), 4 for fp8 (8 x 16 KB); workgroups of fewer than 8 waves (G < 4)
  // keep D = 1 so that several fit on a CU.
  constexpr int D = TileRing<G, F8>::D;
  constexpr int R = TileRing<G, F8>::R;
  static_assert(PITCH == TileRing<G, F8>::PITCH, "LDS pitch");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int b = static_cast<int>(item % a.B);
  const int64_t tile = a.tile_hi - item / a.B;
  const int64_t P0 = tile * QT;
  const int64_t L = P0 / kBlock;
  const int64_t row0 = a.N - a.T;

  // Column data for the two MFMA column tiles of this lane.
  int64_t colp[2];
  bf16x8 qf[2][8];   // bf16: k-step s holds d = 16s + 8*half .. +7
  i32x8 qf8[2][2];   // e4m3: k-step s holds d = 64s + 32*half .. +31
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wave * 64 + j * 32 + l32;
    const int qq = c / G, g = c % G;
    const int64_t p = P0 + qq;
    const int64_t t = p - row0;
    colp[j] = p;
    const bool ok = (t >= a.t0) && (t < a.t0 + a.Tw);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.qI) +
                               ((static_cast<int64_t>(b) * a.T + (ok ? t : 0)) * G + g) * ROWB;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if constexpr (F8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 lo = ld16(src + 64 * s + 32 * half);  // src is a valid row
        const uint4 hi = ld16(src + 64 * s + 32 * half + 16);
        qf8[j][s] = as_i32x8(ok ? lo : z, ok ? hi : z);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 v = ld16(src + 32 * s + 16 * half);  // src is a valid row
        qf[j][s] = as_bf16x8(ok ? v : z);
      }
    }
  }

  // The lane's own column (after the half-wave exchange).
  const int own = wave * 64 + lane;
  const int own_q = own / G, own_g = own % G;
  const int64_t own_t = P0 + own_q - row0;
  const bool own_ok = (own_t >= a.t0) && (own_t < a.t0 + a.Tw);

  const int64_t nkb = WRITE_S ? (L + 1) : L;
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(a.kI) + static_cast<int64_t>(b) * a.N * ROWB;

  float ts[CAP];
  int ti[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    ts[i] = -INFINITY;
    ti[i] = -1;
  }
  float st[4] = {0.f, 0.f, 0.f, 0.f};
  float* srow = nullptr;
  if (WRITE_S && own_ok)
    srow = a.S + ((static_cast<int64_t>(b) * G + own_g) * a.Tw + (own_t - a.t0)) * a.NB;
  const bool s_vec = (a.NB & 3) == 0;
  const int64_t nblocks = WRITE_S ? (L + 1) * BPC : 0;  // blocks this workgroup scores
  // Score of block gb (the BK-key blocks in order): held in st[gb % 4] and
  // stored four at a time, or at the last block.
  auto emit = [&](int64_t gb, float v) {
    const float sv = static_cast<float>(static_cast<double>(v) * kInvSqrt128);
    const int slot = static_cast<int>(gb & 3);
    st[0] = slot == 0 ? sv : st[0];
    st[1] = slot == 1 ? sv : st[1];
    st[2] = slot == 2 ? sv : st[2];
    st[3] = slot == 3 ? sv : st[3];
    if (srow && (slot == 3 || gb + 1 == nblocks)) {
      const int64_t base = gb & ~static_cast<int64_t>(3);
      if (slot == 3 && s_vec && base + 3 < a.NB) {
        *reinterpret_cast<float4*>(srow + base) = make_float4(st[0], st[1], st[2], st[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e <= slot && base + e < a.NB) srow[base + e] = st[e];
      }
    }
  };

  // Blocks go straight from memory into LDS (global_load_lds: lane l of an
  // instruction fills 16 B at the instruction's base + 16 l), no registers
  // hold a block in between.  The LDS block is 256-B lines in the swizzled
  // layout swz (a line is one bf16 key row, or two fp8 rows, which are also
  // contiguous in memory), so wave w's instruction j fills the 1 KB segment
  // j * NW + w of the buffer and its lanes read the chunks that the layout
  // puts there.  Only the local block can hold keys past N (the
  // scores-writing tiles score it): their rows re-read key N - 1, and the
  // causal mask of the local block drops them.
  constexpr int NW = NT / 64;
  static_assert(PF * NW * 1024 == 128 * ROWB, "1 KB segments cover the block");
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // the LDS base is scalar (M0)
  auto direct_block = [&](int buf, int64_t kb) {
    const unsigned char* src = kbase + kb * (kBlock * ROWB);
    const int64_t last = a.N - 1 - kb * kBlock;  // last row of the block inside N
    // (the selection reads only blocks before the local one: no clamp)
    const int lr = WRITE_S && last < kBlock - 1 ? static_cast<int>(last) : kBlock - 1;
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int seg = j * NW + wave_s;
      const int ln = seg * 4 + (lane >> 4);       // (seg * 1024 + lane * 16) >> 8
      const int c = (lane & 15) ^ (ln & 15);      // swz(ln, c) = seg * 1024 + lane * 16
      // the chunk's key row and its offset in that row
      const int r = F8 ? 2 * ln + (c >> 3) : ln;
      const int co = F8 ? (c & 7) * 16 : c * 16;
      __builtin_amdgcn_global_load_lds(
          src + static_cast<uint32_t>((WRITE_S ? min(r, lr) : r) * ROWB + co),
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(kbuf[buf] + seg * 1024)),
          16, 0, 0);
    }
  };

#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < nkb) {
      direct_block(j, j);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // q^I fragments and blocks 0 .. D-1 have landed
  __syncthreads();

  for (int64_t kb = 0; kb < nkb; ++kb) {
    const bool more = kb + D < nkb;
    // the buffer of block kb + D held block kb - D, which every wave has
    // left: a barrier followed the iteration of block kb - D
    if (more) direct_block((kb + D) & (R - 1), kb + D);
    const unsigned char* buf = kbuf[kb & (R - 1)];
    float m0 = -INFINITY, m1 = -INFINITY;
    const bool masked = WRITE_S && (kb == L);
    // One 32-key tile: its K fragments from LDS (8 for bf16: one per
    // 16-dim step; 2 x 32 B for fp8), then 16 (bf16) or 4 (fp8) MFMAs into
    // two column tiles.
    typedef uint4 KFrag[8];
    auto frags = [&](int kt, KFrag& av) {
      if constexpr (F8) {
        // key row r = kt * 32 + l32 is half of line r / 2 (chunks 8 (r & 1) ..
        // +7); k-step s reads its 16-B chunks 4 (s >> 1) + 2 half + (s & 1)
        const int r = kt * 32 + l32;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          av[s] = *reinterpret_cast<const uint4*>(
              &buf[swz(r >> 1, ((r & 1) << 3) | (4 * (s >> 1) + 2 * half + (s & 1)))]);
      } else {
        // rows kt * 32 + l32 share l32's swizzle (32 is a multiple of 16):
        // the lane's offsets plus kt * 32 rows
#pragma unroll
        for (int s = 0; s < 8; ++s)
          av[s] = *reinterpret_cast<const uint4*>(&buf[kt * 32 * 256 + swz(l32, 2 * s + half)]);
      }
    };
    auto tile = [&](const KFrag& av, f32x16& c0, f32x16& c1) {
      if constexpr (F8) {
        // two 32x32x64 steps cover the 128 dims
        const i32x8 a0 = as_i32x8(av[0], av[1]), a1 = as_i32x8(av[2], av[3]);
        c0 = mfma32_f8(a0, qf8[0][0], f32x16{});
        c1 = mfma32_f8(a0, qf8[1][0], f32x16{});
        c0 = mfma32_f8(a1, qf8[0][1], c0);
        c1 = mfma32_f8(a1, qf8[1][1], c1);
      } else {
        c0 = mfma32(as_bf16x8(av[0]), qf[0][0], f32x16{});
        c1 = mfma32(as_bf16x8(av[0]), qf[1][0], f32x16{});
#pragma unroll
        for (int s = 1; s < 8; ++s) {
          c0 = mfma32(as_bf16x8(av[s]), qf[0][s], c0);
          c1 = mfma32(as_bf16x8(av[s]), qf[1][s], c1);
        }
      }
    };
    // Block max over a finished tile (with the causal mask in the local block).
    auto reduce = [&](int kt, f32x16& c0, f32x16& c1) {
      if (masked) {
        // offsets inside the local block past each column's position
        const int lim0 = static_cast<int>(colp[0] - kb * kBlock);
        const int lim1 = static_cast<int>(colp[1] - kb * kBlock);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kt * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
          if (off > lim0) c0[e] = -INFINITY;
          if (off > lim1) c1[e] = -INFINITY;
        }
      }
      m0 = max16(m0, c0);
      m1 = max16(m1, c1);
      if constexpr (WRITE_S && BK < 128) {
        // the last tile of a block: its score, then start the next block
        if ((kt + 1) % TPB == 0) {
          emit(kb * BPC + kt / TPB, halves_max2(m0, m1));
          m0 = -INFINITY;
          m1 = -INFINITY;
        }
      }
    };
    // Software pipeline: the MFMAs of tile kt run while tile kt-1 is reduced
    // and (when S is not written: the score stores need those registers) the
    // K fragments of tile kt+1 are read from LDS.  A wave issuing the block's
    // MFMAs runs at a raised priority, so that the other wave of its SIMD,
    // busy with the vector work of its block's tail (last block max, top-k
    // insertion, the barrier), does not take the issue slots from it
    // (128K select: 10.10-10.12 against 10.27-10.33 ms).
    f32x16 ta0, ta1, tb0, tb1;
    KFrag fa, fb;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!WRITE_S) {
      frags(0, fa);
      sched_fence();
      frags(1, fb);
      tile(fa, ta0, ta1);
      sched_fence();
      frags(2, fa);
      tile(fb, tb0, tb1);
      reduce(0, ta0, ta1);
      sched_fence();
      frags(3, fb);
      tile(fa, ta0, ta1);
      reduce(1, tb0, tb1);
      sched_fence();
      tile(fb, tb0, tb1);
      reduce(2, ta0, ta1);
      sched_fence();
      __builtin_amdgcn_s_setprio(0);
      reduce(3, tb0, tb1);
    } else {
      frags(0, fa);
      tile(fa, ta0, ta1);
      sched_fence();
      frags(1, fb);
      tile(fb, tb0, tb1);
      reduce(0, ta0, ta1);
      sched_fence();
      frags(2, fa);
      tile(fa, ta0, ta1);
      reduce(1, tb0, tb1);
      sched_fence();
      frags(3, fb);
      tile(fb, tb0, tb1);
      reduce(2, ta0, ta1);
      sched_fence();
      __builtin_amdgcn_s_setprio(0);
      reduce(3, tb0, tb1);
    }
    // the block max of the lane's own column (lanes 0-31: tile 0's columns)
    const float v = halves_max2(m0, m1);

    if (WRITE_S) {
      if constexpr (BK == 128) emit(kb, v);
    } else {
      const bool need = v > ts[CAP - 1];
      if (__ballot(need)) {
        if (need) topk_insert<CAP>(ts, ti, v, static_cast<int>(kb));
      }
    }

    if ((kb & (D - 1)) == D - 1 || kb + 1 == nkb) {
      // the loads land in LDS asynchronously: this wave's must be done
      // before the barrier publishes their blocks
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  if (WRITE_S) {
    // Blocks after the local block are invisible: -inf.  The workgroup fills
    // each row's tail together so that consecutive threads write consecutive
    // addresses.
    const int64_t tail0 = nblocks;
    const int64_t len = a.NB - tail0;
    if (len > 0) {
      for (int c = 0; c < TS::NCOL; ++c) {
        const int q = c / G, g = c % G;
        const int64_t t = P0 + q - row0;
        if (t < a.t0 || t >= a.t0 + a.Tw) continue;
        float* row = a.S + ((static_cast<int64_t>(b) * G + g) * a.Tw + (t - a.t0)) * a.NB + tail0;
        for (int64_t e = tid; e < len; e += NT) row[e] = -INFINITY;
      }
    }
    return;
  }

  if (!own_ok) return;
  const int want = static_cast<int>(L < a.k - 1 ? L : a.k - 1);
  int sel[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) sel[i] = i < want ? ti[i] : INT_MAX;
  sort_ascending<CAP>(sel);
  int32_t* out = a.idx + ((static_cast<int64_t>(b) * G + own_g) * a.T + own_t) * a.k;
#pragma unroll
  for (int s = 0; s < CAP + 1; ++s) {
    if (s < a.k) {
      const int val = s < want ? sel[s < CAP ? s : 0] : (s == want ? static_cast<int>(L) : -1);
      out[s] = val;
    }
  }
}

// Workgroups take work items (sequence, position tile) heaviest first; with
// fewer workgroups than items (a.wgs > 0) each loops over every wgs-th item,
// so that the selection keeps to that many CUs and leaves the others to work
// on another stream.
template <int G, int CAP, bool WRITE_S, bool F8, int BK = 128>
__global__ void __launch_bounds__(TileShape<G>::NT)
index_tile_kernel(TileArgs a) {
  __shared__ __align__(16) unsigned char kbuf[TileRing<G, F8>::R][128 * TileRing<G, F8>::PITCH];
  if (a.counter) {
    // items are taken from a counter shared with other launches of the same
    // rows (see launch_index_tiles)
    __shared__ int item_s;
    for (;;) {
      if (threadIdx.x == 0) item_s = atomicAdd(a.counter, 1);
      __syncthreads();
      // the same value in every lane: keep it (and all that derives from it) scalar
      const int64_t item = __builtin_amdgcn_readfirstlane(item_s);
      if (item >= a.nitems) break;  // uniform: every thread read the same value
      index_tile<G, CAP, WRITE_S, F8, BK>(a, item, kbuf);
      __syncthreads();  // item_s is read; the next item refills the ring buffers
    }
    return;
  }
  for (int64_t item = blockIdx.x; item < a.nitems; item += gridDim.x) {
    index_tile<G, CAP, WRITE_S, F8, BK>(a, item, kbuf);
    __syncthreads();  // the next item refills the ring buffers
  }
}

template <int G, bool WS, bool F8, int BK>
static hipError_t launch_tiles_cap(const TileArgs& a, int64_t ntiles, hipStream_t st) {
  using TS = TileShape<G>;
  const int64_t grid = a.wgs > 0 && a.wgs < a.nitems ? a.wgs : a.nitems;
  const dim3 gd(static_cast<unsigned>(grid)), bd(TS::NT);
  TimedLaunch tl(MSA_KERNEL_SELECT, st);
  if (WS || a.k <= 4) {
    hipLaunchKernelGGL((index_tile_kernel<G, 3, WS, F8, BK>), gd, bd, 0, st, a);
  } else if constexpr (BK == 128) {
    if (a.k <= 8)
      hipLaunchKernelGGL((index_tile_kernel<G, 7, WS, F8>), gd, bd, 0, st, a);
    else
      hipLaunchKernelGGL((index_tile_kernel<G, 15, WS, F8>), gd, bd, 0, st, a);
  } else {
    return hipErrorInvalidValue;  // the fused selection takes 128-key blocks
  }
  return hipGetLastError();
}

template <bool WS, bool F8, int BK>
static hipError_t launch_tiles_g(const TileArgs& a, int G, int64_t ntiles, hipStream_t st) {
  switch (G) {
    case 1: return launch_tiles_cap<1, WS, F8, BK>(a, ntiles, st);
    case 2: return launch_tiles_cap<2, WS, F8, BK>(a, ntiles, st);
    case 4: return launch_tiles_cap<4, WS, F8, BK>(a, ntiles, st);
    case 8: return launch_tiles_cap<8, WS, F8, BK>(a, ntiles, st);
    case 16: return launch_tiles_cap<16, WS, F8, BK>(a, ntiles, st);
  }
  return hipErrorInvalidValue;
}

static int tile_queries(int G) { return (MSA_TILE_COLS / G) < 128 ? (MSA_TILE_COLS / G) : 128; }

hipError_t launch_index_tiles(bool write_scores, bool fp8, const void* qI, const void* kI,
                              float* S, int32_t* idx, int64_t B, int64_t T, int64_t t0,
                              int64_t Tw, int64_t N, int G, int Bk, int k, hipStream_t st,
                              int wgs, int32_t* counter) {
  const int QT = tile_queries(G);
  TileArgs a;
  a.qI = static_cast<const u16*>(qI);
  a.kI = static_cast<const u16*>(kI);
  a.S = S;
  a.idx = idx;
  a.T = T;
  a.N = N;
  a.t0 = t0;
  a.Tw = Tw;
  a.NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  a.k = k;
  a.B = static_cast<int32_t>(B);
  const int64_t tile_lo = (N - T + t0) / QT;
  a.tile_hi = (N - T + t0 + Tw - 1) / QT;
  const int64_t ntiles = a.tile_hi - tile_lo + 1;
  a.nitems = ntiles * B;
  a.wgs = wgs;
  a.counter = counter;
  if (Bk != 128 && (fp8 || !write_scores)) return hipErrorInvalidValue;
  if (fp8) {
    if (write_scores) return launch_tiles_g<true, true, 128>(a, G, ntiles, st);
    return launch_tiles_g<false, true, 128>(a, G, ntiles, st);
  }
  if (!write_scores) return launch_tiles_g<false, false, 128>(a, G, ntiles, st);
  switch (Bk) {
    case 128: return launch_tiles_g<true, false, 128>(a, G, ntiles, st);
    case 64: return launch_tiles_g<true, false, 64>(a, G, ntiles, st);
    case 32: return launch_tiles_g<true, false, 32>(a, G, ntiles, st);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Decode scan (T == 1): stream the index-key cache once.  A workgroup takes 4
// consecutive blocks of one sequence, one per wave (many short waves keep
// more loads in flight across the chip than fewer long ones).  16x16x32 MFMA with
// 16 keys on M and the G index queries on N (unused columns are zero).  The
// 32 16-B loads of a block are all issued before its MFMAs so that each wave
// keeps 32 KB in flight.  k-step s covers d = 32*s .. 32*s+31 with lane
// quarter qd holding d = 32*s + 8*qd .. +7, so one load instruction reads 64
// contiguous bytes of each of 16 key rows.
// ---------------------------------------------------------------------------
struct ScanArgs {
  const u16* qI;
  const u16* kI;  // [B, N, 128], or the page pool [pages, 128, 128] when paged
  float* S;       // [B, G, NB]
  int64_t N;      // cache capacity (tokens)
  int32_t NB, G;  // NB: blocks of BK keys
  int32_t NCH;    // 128-key chunks, one per wave
  PagedCache pc;
};

// F8: e4m3 inputs; one 16x16x128 MFMA covers 16 keys x all 128 dims (lane
// quarter qd holds d = 32*qd .. +31), and a block is 16 KB.
// BK: block size of the scores; a wave's 128-key chunk holds 128 / BK blocks.
template <bool F8, int BK>
__global__ void __launch_bounds__(256) decode_scan_kernel(ScanArgs a) {
  constexpr int BPC = 128 / BK;  // blocks per chunk
  constexpr int GPB = BK / 16;   // 16-key groups per block
  constexpr int ROWB = F8 ? 128 : 256;  // bytes per k^I / q^I row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int col = lane & 15, qd = lane >> 4;
  const uint4 z = make_uint4(0, 0, 0, 0);
  const unsigned char* qsrc = reinterpret_cast<const unsigned char*>(a.qI) +
                              (static_cast<int64_t>(b) * a.G + (col < a.G ? col : 0)) * ROWB;
  bf16x8 qf[4];
  i32x8 qf8;
  if constexpr (F8) {
    const uint4 lo = col < a.G ? ld16(qsrc + 32 * qd) : z;
    const uint4 hi = col < a.G ? ld16(qsrc + 32 * qd + 16) : z;
    qf8 = as_i32x8(lo, hi);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(col < a.G ? ld16(qsrc + 64 * s + 16 * qd) : z);
  }
  {
    const int64_t kb = static_cast<int64_t>(blockIdx.x) * 4 + wave;  // the wave's chunk
    if (kb >= a.NCH) return;
    // this sequence's length (paged: its own) and the chunk's keys inside it
    const int64_t len = paged_len(a.pc, b, a.N);
    float* srow = a.S + static_cast<int64_t>(b) * a.G * a.NB + kb * BPC;
    if (kb * kBlock >= len) {  // past the end of this sequence: invisible
      if (lane < a.G) {
#pragma unroll
        for (int j = 0; j < BPC; ++j)
          if (kb * BPC + j < a.NB) srow[static_cast<int64_t>(lane) * a.NB + j] = -INFINITY;
      }
      return;
    }
    const int nvalid = static_cast<int>(len - kb * kBlock < kBlock ? len - kb * kBlock : kBlock);
    const unsigned char* kblk = reinterpret_cast<const unsigned char*>(a.kI) +
                                (a.pc.table ? paged_page(a.pc, b, kb) * kBlock
                                            : static_cast<int64_t>(b) * a.N + kb * kBlock) *
                                    ROWB;
    constexpr int LPK = F8 ? 2 : 4;  // 16-B loads per key row and lane
    uint4 d[8][LPK];
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      const int kk = kg * 16 + col;
      const unsigned char* src = kblk + (kk < nvalid ? kk : nvalid - 1) * ROWB;
#pragma unroll
      for (int s = 0; s < LPK; ++s)  // tail keys masked below
        d[kg][s] = F8 ? ld16(src + 32 * qd + 16 * s) : ld16(src + 64 * s + 16 * qd);
    }
    float m[BPC];
#pragma unroll
    for (int j = 0; j < BPC; ++j) m[j] = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      f32x4 acc = {};
      if constexpr (F8) {
        acc = mfma16_f8(as_i32x8(d[kg][0], d[kg][1]), qf8, acc);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(as_bf16x8(d[kg][s]), qf[s], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kg * 16 + 4 * qd + r;
        m[kg / GPB] = fmaxf(m[kg / GPB], kk < nvalid ? acc[r] : -INFINITY);
      }
    }
#pragma unroll
    for (int j = 0; j < BPC; ++j) {
      m[j] = quads_max(m[j]);
    }
    if (lane < a.G) {
#pragma unroll
      for (int j = 0; j < BPC; ++j)
        if (kb * BPC + j < a.NB)
          srow[static_cast<int64_t>(lane) * a.NB + j] =
              static_cast<float>(static_cast<double>(m[j]) * kInvSqrt128);
    }
  }
}

hipError_t launch_decode_scan(bool fp8, const void* qI, const void* kI, float* S,
                              int64_t B, int64_t N, int G, int Bk, const PagedCache& pc,
                              hipStream_t st) {
  ScanArgs a;
  a.pc = pc;
  a.qI = static_cast<const u16*>(qI);
  a.kI = static_cast<const u16*>(kI);
  a.S = S;
  a.N = N;
  a.NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  a.NCH = static_cast<int32_t>((N + kBlock - 1) / kBlock);
  a.G = G;
  const dim3 grid(static_cast<unsigned>((a.NCH + 3) / 4), static_cast<unsigned>(B));
  TimedLaunch tl(MSA_KERNEL_DECODE_SCAN, st);
  if (fp8 && Bk == 128)
    hipLaunchKernelGGL((decode_scan_kernel<true, 128>), grid, dim3(256), 0, st, a);
  else if (fp8)
    return hipErrorInvalidValue;
  else if (Bk == 128)
    hipLaunchKernelGGL((decode_scan_kernel<false, 128>), grid, dim3(256), 0, st, a);
  else if (Bk == 64)
    hipLaunchKernelGGL((decode_scan_kernel<false, 64>), grid, dim3(256), 0, st, a);
  else if (Bk == 32)
    hipLaunchKernelGGL((decode_scan_kernel<false, 32>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k from materialised scores: one wave per (sequence, group, row).
//   1. each lane takes the strided candidates e = lane + 64 i and keeps their
//      max; the m-th largest lane max (m = min(k-1, L)) is a lower bound tau
//      for the m-th largest candidate, so every winner scores >= tau;
//   2. the candidates >= tau are compacted (in index order) through LDS; if
//      at most 64 survive they are bitonic-sorted across the wave by
//      (score desc, index asc), otherwise (many equal scores) the survivors
//      are merged 64 at a time into a running best-64 list;
//   3. the best m are sorted by block index and written with the local block.
// ---------------------------------------------------------------------------
struct TopkArgs {
  const float* S;   // scores of the window's rows: [B, G, Tw, NB]
  int32_t* idx;     // [B, G, T, k]
  int64_t T, N, rows;
  int64_t t0, Tw;   // this launch's query rows: t0 .. t0 + Tw - 1 (rows = B * G * Tw)
  int32_t NB, k, G, Bk;
  PagedCache pc;  // per-sequence lengths when paged (T == 1)
};

// Row r of a top-k launch: its scores, its output and its local block.
struct TopkRow {
  const float* s;
  int32_t* out;
  int64_t L;
};

__device__ __forceinline__ TopkRow topk_row(const TopkArgs& a, int64_t r) {
  const int64_t bg = r / a.Tw, t = a.t0 + r % a.Tw;
  TopkRow x;
  x.s = a.S + r * a.NB;
  x.out = a.idx + (bg * a.T + t) * a.k;
  x.L = (paged_len(a.pc, bg / a.G, a.N) - a.T + t) / a.Bk;
  return x;
}

// The selection of one row by one wave.
__device__ __forceinline__ void topk_one_row(const TopkArgs& a, const TopkRow& x, int lane,
                                             TopkScratch& sc) {
  const int64_t L = x.L;
  const int m = static_cast<int>(L < a.k - 1 ? L : a.k - 1);
  int32_t* out = x.out;
  if (m == 0) {
    if (lane < a.k) out[lane] = lane == 0 ? static_cast<int>(L) : -1;
    return;
  }
  float v;
  int vi;
  // the row's pointer and length read as scalars: the buffer resource built
  // from them must be uniform (the pair kernel's fallback otherwise sees
  // them through per-lane copies)
  const uint64_t sp = reinterpret_cast<uint64_t>(x.s);
  const uint32_t sp_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sp >> 32));
  const uint32_t sp_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sp));
  const float* src = reinterpret_cast<const float*>((static_cast<uint64_t>(sp_hi) << 32) | sp_lo);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(L));
  const int nc = wave_topk<16, false>(src, n, 0, 64, m, lane, sc, v, vi);
  if (nc < 0) {
    write_selection(out, vi, m, static_cast<int>(L), a.k, lane);
    return;
  }
  // The nc >= m compacted candidates are in ascending block order.  Sorting
  // their scores alone gives the m-th best score vm (finite); the best m are
  // the candidates scoring above vm and, of those equal to it, the first ones
  // in block order, as many as are still missing.  Their order in the list is
  // their output slot.
  const float c = lane < nc ? sc.v[lane] : -INFINITY;
  const int cidx = lane < nc ? sc.i[lane] : INT_MAX;
  const float sv = nc <= 16   ? sort_desc_values<16>(c, lane)
                   : nc <= 32 ? sort_desc_values<32>(c, lane)
                              : sort_desc_values<64>(c, lane);
  const float vm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), m - 1));
  const unsigned long long above = __ballot(c > vm);
  const unsigned long long equal = __ballot(c == vm);
  const bool sel = (c > vm) | ((c == vm) & (lanes_below(equal) < m - __popcll(above)));
  const unsigned long long bm = __ballot(sel);
  if (sel) out[lanes_below(bm)] = cidx;
  if ((lane >= m) & (lane < a.k)) out[lane] = lane == m ? static_cast<int>(L) : -1;
}

__global__ void __launch_bounds__(256) topk_rows_kernel(TopkArgs a) {
  __shared__ TopkScratch sc[4];
  // the wave index read as a scalar: the row's bookkeeping (divisions for
  // its position and local block, its pointers) runs on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= a.rows) return;
  topk_one_row(a, topk_row(a, row), lane, sc[wave]);
}

// Lanes below this one inside its half-wave that are set in `mask`, plus
// base: mbcnt over the whole wave counts, for an upper-half lane, every set
// lane of the lower half, so those are taken off the base there.
__device__ __forceinline__ int half_rank(unsigned long long mask, bool upper, int base) {
  const unsigned lo = static_cast<unsigned>(mask), hi = static_cast<unsigned>(mask >> 32);
  const int b = upper ? base - static_cast<int>(__popc(lo)) : base;
  return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, b));
}

// Two rows per wave, one in each half-wave (rows of at most 32 x 32
// candidates, k <= 16, fewer than 2^31 rows; with more picks the m-th
// largest of only 32 lane maxima lets most of a row through).  Half-lane h
// holds its row's candidates h + 32 r in registers, and the threshold and
// ranking steps of topk_one_row run on both halves at once, so that every
// sorting network serves two rows.  The candidates reaching either half's
// threshold are compacted into one list in wave order (each row's in block
// order), then split into the two halves.  If more than 32 of one row (or
// 64 of both) reach the threshold, both rows go to topk_one_row instead.
constexpr int kPairChunks = 32;

__global__ void __launch_bounds__(256) topk_pair_kernel(TopkArgs a) {
  __shared__ TopkScratch sc[4];
  const int lane = threadIdx.x & 63, h = lane & 31;
  const bool upper = lane >= 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t r0 = (blockIdx.x * 4u + static_cast<uint32_t>(wave)) * 2u;
  if (r0 >= static_cast<uint64_t>(a.rows)) return;
  const bool two = r0 + 1u < static_cast<uint64_t>(a.rows);
  // scalar bookkeeping: one 32-bit division for both rows; Bk is a power of
  // two and the position N' - T + t of a query row is never negative
  const uint32_t Tw = static_cast<uint32_t>(a.Tw);
  const uint32_t bg0 = r0 / Tw, tw0 = r0 - bg0 * Tw;
  const uint32_t bg1 = tw0 + 1u == Tw ? bg0 + 1u : bg0, tw1 = tw0 + 1u == Tw ? 0u : tw0 + 1u;
  const int bks = __builtin_ctz(static_cast<unsigned>(a.Bk));
  auto row_L = [&](uint32_t bg, uint32_t tw) {
    const int64_t len = a.pc.table ? paged_len(a.pc, bg / static_cast<uint32_t>(a.G), a.N) : a.N;
    return static_cast<int>((len - a.T + a.t0 + tw) >> bks);
  };
  TopkRow x0, x1;
  x0.s = a.S + static_cast<int64_t>(r0) * a.NB;
  x0.out = a.idx + (static_cast<int64_t>(bg0) * a.T + a.t0 + tw0) * a.k;
  x0.L = row_L(bg0, tw0);
  x1.s = x0.s + a.NB;
  x1.out = a.idx + (static_cast<int64_t>(bg1) * a.T + a.t0 + tw1) * a.k;
  x1.L = two ? row_L(bg1, tw1) : 0;
  const int L0 = static_cast<int>(x0.L), L1 = static_cast<int>(x1.L);
  const int m0 = min(L0, a.k - 1), m1 = min(L1, a.k - 1);
  const int n = upper ? L1 : L0;  // this lane's row: candidates, picks
  const int m = upper ? m1 : m0;
  TopkScratch& s = sc[wave];

  // Each row through a raw buffer of its own candidates (a load past the
  // row's end returns 0 and reads nothing), one half-wave's loads at a time.
  // The upper half's loads carry the sc0 cache bit (its reads skip the
  // per-CU cache; the scores are read once): the two groups differ in an
  // immediate, so they stay two groups under a uniform resource each
  // instead of being merged into one load on a per-lane resource.
  const auto rs0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x0.s), 0, L0 * 4,
                                                     kBufferFormat32);
  const auto rs1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x1.s), 0, L1 * 4,
                                                     kBufferFormat32);
  float x[kPairChunks];
  if (upper) {
#pragma unroll
    for (int r = 0; r < kPairChunks; ++r)
      x[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs1, 4 * h + 128 * r, 0, 1));
  } else {
#pragma unroll
    for (int r = 0; r < kPairChunks; ++r)
      x[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs0, 4 * h + 128 * r, 0, 0));
  }
  const int lim = n - h;
#pragma unroll
  for (int r = 0; r < kPairChunks; ++r) x[r] = 32 * r < lim ? x[r] : -INFINITY;
  float lm = -INFINITY;
#pragma unroll
  for (int r = 0; r < kPairChunks; ++r) lm = fmaxf(lm, x[r]);
  // the m-th largest lane max of each half (kept above -inf, see wave_topk)
  const int msel = 4 * ((upper ? 32 : 0) + (m > 0 ? m : 1) - 1);
  const float tau = fmaxf(__int_as_float(__builtin_amdgcn_ds_bpermute(
                              msel, __float_as_int(sort_desc_values<32>(lm, lane)))),
                          -FLT_MAX);
  // compaction of both rows' candidates >= their tau into one list (every
  // lane stores; a non-candidate to its spare entry 64 + lane); entries
  // carry the block index and, in bit 16, the row
  const int nch = (max(L0, L1) + 31) >> 5;  // chunks holding a candidate of either row
  const int tag = h | (upper ? 1 << 16 : 0);
  int cnt = 0;  // saturates at 128: positions stay below 192
#pragma unroll
  for (int r = 0; r < kPairChunks; ++r) {
    if (r < nch) {
      const bool f = x[r] >= tau;
      const unsigned long long bal = __ballot(f);
      const unsigned bal_lo = static_cast<unsigned>(bal), bal_hi = static_cast<unsigned>(bal >> 32);
      const int pos = __builtin_amdgcn_mbcnt_hi(bal_hi, __builtin_amdgcn_mbcnt_lo(bal_lo, cnt));
      const int slot = f ? pos : 64 + lane;
      s.v[slot] = x[r];
      s.i[slot] = tag + 32 * r;
      cnt = min(cnt + static_cast<int>(__popcll(bal)), 128);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // the list's entry of this lane, its row, and its place in that row's list
  const bool live = lane < cnt;
  const float ev = s.v[lane];
  const int ei = s.i[lane];
  const bool eup = (ei >> 16) != 0;
  const unsigned long long in1 = __ballot(live & eup), in0 = __ballot(live & !eup);
  const int c0 = static_cast<int>(__popcll(in0)), c1 = static_cast<int>(__popcll(in1));
  if ((cnt > 64) | (max(c0, c1) > 32)) {
    topk_one_row(a, x0, lane, s);
    if (two) topk_one_row(a, x1, lane, s);
    return;
  }
  // split: row r0's entries to lanes 0.., row r0 + 1's to lanes 32.., each
  // in list order (block order)
  if (live) {
    const int dst = eup ? 32 + lanes_below(in1) : lanes_below(in0);
    s.v[dst] = ev;
    s.i[dst] = ei & 0xFFFF;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // ranking as in topk_one_row, per half
  const int cn = upper ? c1 : c0;
  const float c = h < cn ? s.v[lane] : -INFINITY;
  const int cidx = h < cn ? s.i[lane] : INT_MAX;
  const float sv =
      max(c0, c1) <= 16 ? sort_desc_values<16>(c, lane) : sort_desc_values<32>(c, lane);
  const float vm = __int_as_float(__builtin_amdgcn_ds_bpermute(msel, __float_as_int(sv)));
  const unsigned long long above = __ballot(c > vm);
  const int n_above =
      __popc(upper ? static_cast<unsigned>(above >> 32) : static_cast<unsigned>(above));
  const bool sel = (c > vm) | ((c == vm) & (half_rank(__ballot(c == vm), upper, 0) < m - n_above));
  const unsigned long long bm = __ballot(sel);
  if (upper & !two) return;
  int32_t* out = upper ? x1.out : x0.out;
  if (sel) out[half_rank(bm, upper, 0)] = cidx;
  if ((h >= m) & (h < a.k)) out[h] = h == m ? n : -1;
}

// Long rows, few of them (decode): four waves per row, each takes every
// fourth 64-candidate chunk; the four best-m lists meet in LDS and wave 0
// orders them and writes the selection.
__global__ void __launch_bounds__(256) topk_wide_kernel(TopkArgs a) {
  __shared__ WideTopkLds t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const TopkRow x = topk_row(a, blockIdx.x);
  const int64_t L = x.L;
  const int m = static_cast<int>(L < a.k - 1 ? L : a.k - 1);
  int32_t* out = x.out;
  if (m == 0) {
    if (wave == 0 && lane < a.k) out[lane] = lane == 0 ? static_cast<int>(L) : -1;
    return;
  }
  wide_topk_part1(x.s, static_cast<int>(L), m, lane, wave, t);
  __syncthreads();
  if (wave != 0) return;
  const int v = wide_topk_part2(static_cast<int>(L), m, lane, t);
  if (lane < a.k) out[lane] = v;
}

hipError_t launch_topk_rows(const float* S, int32_t* idx, int64_t B, int64_t T, int64_t t0,
                            int64_t Tw, int64_t N, int G, int Bk, int k, const PagedCache& pc,
                            hipStream_t st) {
  TopkArgs a;
  a.G = G;
  a.pc = pc;
  a.S = S;
  a.idx = idx;
  a.T = T;
  a.t0 = t0;
  a.Tw = Tw;
  a.N = N;
  a.rows = B * G * Tw;
  a.Bk = Bk;
  a.NB = static_cast<int32_t>((N + Bk - 1) / Bk);
  a.k = k;
  TimedLaunch tl(MSA_KERNEL_TOPK, st);
  if (a.rows <= 4096 && a.NB >= 1024) {
    // few long rows: spread each row over a workgroup
    hipLaunchKernelGGL(topk_wide_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(256), 0, st, a);
  } else if (a.k <= 16 && a.NB <= 32 * kPairChunks && a.rows < (int64_t{1} << 31)) {
    const int64_t grid = (a.rows + 7) / 8;
    hipLaunchKernelGGL(topk_pair_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, a);
  } else {
    const int64_t grid = (a.rows + 3) / 4;
    hipLaunchKernelGGL(topk_rows_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace msa
