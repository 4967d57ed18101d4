// msa_topk.h -- wave-level pieces of the exp-free top-k (stage 3): branch-free
// compare-exchanges over lane exchanges, bitonic sorts and merges, the
// threshold-and-compact selection of one row by one wave, and the four-wave
// selection of a long row.  Shared by the top-k kernels and the one-call
// decode kernel.
#pragma once

#include <float.h>
#include <limits.h>
#include <math.h>

#include "msa_common.h"

namespace msa {

// Word 3 of a raw (stride 0) buffer resource for untyped dword loads on this
// architecture family: DATA_FORMAT (bits 15-18) = 4, 32-bit elements; the
// other fields 0.  A load whose byte offset is at or past the resource's
// byte count returns 0 and reads nothing.
constexpr int kBufferFormat32 = 4 << 15;

// Non-short-circuit operators keep the comparisons branch-free (selects, not
// exec-mask branches).
__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
  return (av > bv) | ((av == bv) & (ai < bi));
}

// The value of lane (lane ^ S), S a power of two below 64, by the cheapest
// exchange for each distance: a DPP quad permutation for 1 and 2 (every lane
// has a source, so no old value is kept), a swizzle (inside each half-wave)
// for 4 to 16, a permute for 32.
template <int S>
__device__ __forceinline__ int xlane(int x) {
  if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);
  else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);
  else if constexpr (S < 32) return __builtin_amdgcn_ds_swizzle(x, 0x1F | (S << 10));
  else
    return __builtin_amdgcn_ds_bpermute(
        (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) ^ 32) << 2, x);
}

// Compare-exchange directions as wave masks.  Lane l keeps the first-ranked
// of its pair at stage (size, stride) of a bitonic sort when bit `stride` of
// l is clear exactly in runs whose direction is `first`: the run of size
// `size` holding l goes first-ranked-first when bit `size` of l is clear or
// size == nmax (the last merge of runs of nmax lanes).  Used through
// __builtin_amdgcn_inverse_ballot_w64, the per-lane condition is a constant
// in scalar registers: no vector instruction per stage.
constexpr unsigned long long keep_lanes(int size, int stride, int nmax, bool first) {
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l) {
    const bool run_first = (((l & size) == 0) || size == nmax) == first;
    if (((l & stride) == 0) == run_first) m |= 1ull << l;
  }
  return m;
}

static_assert(keep_lanes(2, 1, 64, true) == 0x9999999999999999ull, "pairs (0,1) up, (2,3) down");
static_assert(keep_lanes(64, 32, 64, true) == 0x00000000FFFFFFFFull, "last stage: low half first");
static_assert(keep_lanes(16, 8, 16, true) == 0x00FF00FF00FF00FFull, "runs of 16 all first");

template <unsigned long long K>
__device__ __forceinline__ bool lane_in() {
  return __builtin_amdgcn_inverse_ballot_w64(K);
}

template <int S>
__device__ __forceinline__ float xlane(float x) {
  return __int_as_float(xlane<S>(__float_as_int(x)));
}

// Bitonic sort of one (score, index) pair per lane, from the merge of SIZE
// runs at distance STRIDE on; best_first puts the best pair in lane 0.  Each
// compare-exchange takes one comparison: keep says whether this lane ends with
// the better pair of the two (for two equal pairs either choice leaves the
// same pair).
template <int SIZE, int STRIDE, int NMAX>
__device__ __forceinline__ void bitonic_steps(float& v, int& i, int lane, bool best_first) {
  const float pv = xlane<STRIDE>(v);
  const int pi = xlane<STRIDE>(i);
  const bool keep = best_first ? lane_in<keep_lanes(SIZE, STRIDE, 0, true)>()
                               : lane_in<keep_lanes(SIZE, STRIDE, 0, false)>();
  const bool take = beats(pv, pi, v, i) == keep;
  v = take ? pv : v;
  i = take ? pi : i;
  if constexpr (STRIDE > 1)
    bitonic_steps<SIZE, STRIDE / 2, NMAX>(v, i, lane, best_first);
  else if constexpr (SIZE < NMAX)
    bitonic_steps<SIZE * 2, SIZE, NMAX>(v, i, lane, best_first);
}

// Sorts each run of NMAX consecutive lanes (NMAX = 64: the whole wave).
template <int NMAX = 64>
__device__ __forceinline__ void bitonic64(float& v, int& i, int lane, bool best_first) {
  bitonic_steps<2, 1, NMAX>(v, i, lane, best_first);
}

// Merge of a best-first bitonic sequence into best-first order.
template <int STRIDE = 32>
__device__ __forceinline__ void bitonic_merge64(float& v, int& i, int lane) {
  const float pv = xlane<STRIDE>(v);
  const int pi = xlane<STRIDE>(i);
  const bool take = beats(pv, pi, v, i) == lane_in<keep_lanes(64, STRIDE, 64, true)>();
  v = take ? pv : v;
  i = take ? pi : i;
  if constexpr (STRIDE > 1) bitonic_merge64<STRIDE / 2>(v, i, lane);
}

// Values sorted descending within each run of NMAX consecutive lanes (lane 0
// the largest; NMAX = 64: the whole wave).
template <int NMAX = 64, int SIZE = 2, int STRIDE = 1>
__device__ __forceinline__ float sort_desc_values(float v, int lane) {
  const float pv = xlane<STRIDE>(v);
  const bool keep = lane_in<keep_lanes(SIZE, STRIDE, NMAX, true)>();
  v = ((pv > v) == keep) ? pv : v;  // keep: the larger of the two
  if constexpr (STRIDE > 1)
    return sort_desc_values<NMAX, SIZE, STRIDE / 2>(v, lane);
  else if constexpr (SIZE < NMAX)
    return sort_desc_values<NMAX, SIZE * 2, SIZE>(v, lane);
  else
    return v;
}

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0));
}

// Per-wave LDS scratch of the threshold-and-compact selection: the compacted
// candidates (at most 64 are ever read), the spare entries 64 + lane, and
// room for compacted positions up to 191, so that every lane stores every
// chunk without a bounds test or an exec-mask branch.
constexpr int kTopkScratch = 192;
struct TopkScratch {
  float v[kTopkScratch];
  int i[kTopkScratch];
};

// Best m candidates (score desc, index asc) among src[e] for e = e0 + lane +
// step*i < n, left best-first in lanes 0..m-1 (m <= 63).  The first R strided
// chunks are loaded once into registers, all loads in flight together; any
// remainder is re-read from memory.
// Returns the number of candidates compacted into sc in ascending index
// order (all those >= the threshold, a superset of the best m), or -1 when
// there were more than 64 (the best m then came from a running merge).  With
// SORT false the compacted candidates are left unsorted and v / vi are set
// only on the merge path.
template <int R, bool SORT = true>
__device__ __forceinline__ int wave_topk(const float* src, int n, int e0, int step, int m,
                                         int lane, TopkScratch& sc, float& v, int& vi) {
  // The first R chunks through a raw buffer of n floats: a load at or past
  // the row's end returns 0 without a memory access, and needs no address
  // clamp (the chunk offsets become immediate offsets of one lane offset).
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), 0, n * 4,
                                                    kBufferFormat32);
  float x[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    x[r] = __int_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (e0 + lane + step * r), 0, 0));
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = lane < n - e0 - step * r ? x[r] : -INFINITY;
  const int rest = e0 + step * R;
  float lm = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) lm = fmaxf(lm, x[r]);
  for (int e = rest + lane; e < n; e += step) lm = fmaxf(lm, src[e]);
  // The m-th largest lane max: at least m candidates reach it.  Kept above
  // -inf (a wave whose part of the row holds fewer than m candidates), so
  // that the -inf fill past the row's end never passes the test.
  const float tau = fmaxf(__shfl(sort_desc_values(lm, lane), m - 1), -FLT_MAX);
  v = -INFINITY;
  vi = INT_MAX;
  // candidates >= tau, compacted in index order; cnt counts them (the same in
  // every lane), saturating at 128 so that positions stay below 192
  int cnt = 0;
  // every lane stores: a kept candidate at its compacted position, any
  // other value in the lane's own spare entry 64 + lane (never read)
  auto chunk = [&](int c0, float xv) {
    const bool f = xv >= tau;
    const unsigned long long bal = __ballot(f);
    const unsigned bal_lo = static_cast<unsigned>(bal), bal_hi = static_cast<unsigned>(bal >> 32);
    const int pos = __builtin_amdgcn_mbcnt_hi(bal_hi, __builtin_amdgcn_mbcnt_lo(bal_lo, cnt));
    const int slot = f ? pos : 64 + lane;
    sc.v[slot] = xv;
    sc.i[slot] = c0 + lane;
    cnt = min(cnt + static_cast<int>(__popcll(bal)), 128);
  };
  auto merge = [&](int c0, float xv) {
    const int e = c0 + lane;
    const bool f = (e < n) & (xv >= tau);
    if (!__ballot(f)) return;
    float cvv = f ? xv : -INFINITY;
    int cii = f ? e : INT_MAX;
    bitonic64(cvv, cii, lane, false);
    if (beats(cvv, cii, v, vi)) {
      v = cvv;
      vi = cii;
    }
    bitonic_merge64(v, vi, lane);
  };
  // chunks from nch on hold no candidate: no compaction work (a uniform
  // branch; the loads above stay unconditional so that none of them waits
  // before the next is issued)
  const int nch = n > e0 ? (n - e0 + step - 1) / step : 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < nch) chunk(e0 + step * r, x[r]);
  for (int c0 = rest; c0 < n; c0 += step) {
    const int e = c0 + lane;
    chunk(c0, e < n ? src[e] : -INFINITY);
  }
  if (cnt <= 64) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if constexpr (!SORT) return cnt;
    if (lane < cnt) {
      v = sc.v[lane];
      vi = sc.i[lane];
    }
    // sort only as many lanes as hold candidates
    if (cnt <= 16)
      bitonic64<16>(v, vi, lane, true);
    else if (cnt <= 32)
      bitonic64<32>(v, vi, lane, true);
    else
      bitonic64(v, vi, lane, true);
    return cnt;
  } else {
    // many equal scores at the threshold: merge 64 candidates at a time into
    // a running best-64 list
#pragma unroll
    for (int r = 0; r < R; ++r) merge(e0 + step * r, x[r]);
    for (int c0 = rest; c0 < n; c0 += step) {
      const int e = c0 + lane;
      merge(c0, e < n ? src[e] : -INFINITY);
    }
    return -1;
  }
}

// Ascending sort of the keys of each 16-lane row (bitonic, from the merge of
// SIZE runs at distance STRIDE on).
template <int SIZE = 2, int STRIDE = 1>
__device__ __forceinline__ int sort_asc16(int key, int lane) {
  const int pk = xlane<STRIDE>(key);
  const bool keep = lane_in<keep_lanes(SIZE, STRIDE, 16, true)>();
  key = ((pk < key) == keep) ? pk : key;  // keep: the smaller of the two
  if constexpr (STRIDE > 1)
    return sort_asc16<SIZE, STRIDE / 2>(key, lane);
  else if constexpr (SIZE < 16)
    return sort_asc16<SIZE * 2, SIZE>(key, lane);
  else
    return key;
}

// Ascending sort of the keys across the wave.
template <int SIZE = 2, int STRIDE = 1>
__device__ __forceinline__ int sort_asc64(int key, int lane) {
  const int pk = xlane<STRIDE>(key);
  const bool keep = lane_in<keep_lanes(SIZE, STRIDE, 64, true)>();
  key = ((pk < key) == keep) ? pk : key;  // keep: the smaller of the two
  if constexpr (STRIDE > 1)
    return sort_asc64<SIZE, STRIDE / 2>(key, lane);
  else if constexpr (SIZE < 64)
    return sort_asc64<SIZE * 2, SIZE>(key, lane);
  else
    return key;
}

// Lanes 0..m-1 hold block ids; the selection's entry of each lane < k: the
// ids ascending, then the local block L, then -1 padding (m < k <= 64).
__device__ __forceinline__ int selection_value(int vi, int m, int L, int lane) {
  const int key0 = lane < m ? vi : INT_MAX;
  const int key = m <= 15 ? sort_asc16(key0, lane) : sort_asc64(key0, lane);
  return lane < m ? key : (lane == m ? L : -1);
}

__device__ __forceinline__ void write_selection(int32_t* out, int vi, int m, int L, int k,
                                                int lane) {
  const int v = selection_value(vi, m, L, lane);
  if (lane < k) out[lane] = v;
}

// Selection of one long row by four waves (waves 0..3 of the workgroup), in
// two parts around a workgroup barrier.  Part 1: each wave takes every fourth
// 64-candidate chunk of s[0..L) and leaves its best m in LDS.  Part 2 (wave 0
// only): orders the four lists and returns lane's selection entry (lanes < k).
struct WideTopkLds {
  TopkScratch sc[4];
  float mv[4][64];
  int mi[4][64];
};

__device__ __forceinline__ void wide_topk_part1(const float* s, int L, int m, int lane, int wave,
                                                WideTopkLds& t) {
  float v;
  int vi;
  wave_topk<8>(s, L, 64 * wave, 256, m, lane, t.sc[wave], v, vi);
  if (m <= 15) {
    // Each wave's list is sorted best-first; odd waves store theirs reversed,
    // so that every 32 entries form a bitonic sequence and two merge stages
    // (instead of a whole sort) order the 64.
    if (lane < 16) {
      const int pos = wave * 16 + ((wave & 1) ? 15 - lane : lane);
      t.mv[0][pos] = lane < m ? v : -INFINITY;
      t.mi[0][pos] = lane < m ? vi : INT_MAX;
    }
  } else {
    t.mv[wave][lane] = lane < m ? v : -INFINITY;
    t.mi[wave][lane] = lane < m ? vi : INT_MAX;
  }
}

__device__ __forceinline__ int wide_topk_part2(int L, int m, int lane, WideTopkLds& t) {
  float v;
  int vi;
  if (m <= 15) {
    v = t.mv[0][lane];
    vi = t.mi[0][lane];
    bitonic_steps<32, 16, 64>(v, vi, lane, true);
  } else {
    // Up to 63 per wave: wave 0 merges the other lists into its own one at a
    // time (its list best-first against the other reversed: the better of
    // each pair is the best 64 of the two, a bitonic sequence).
    v = t.mv[0][lane];
    vi = t.mi[0][lane];
#pragma unroll 1
    for (int w = 1; w < 4; ++w) {
      const float u = t.mv[w][63 - lane];
      const int ui = t.mi[w][63 - lane];
      if (beats(u, ui, v, vi)) {
        v = u;
        vi = ui;
      }
      bitonic_merge64(v, vi, lane);
    }
  }
  return selection_value(vi, m, L, lane);
}

}  // namespace msa
