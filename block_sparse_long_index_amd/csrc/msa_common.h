// msa_common.h -- device helpers shared by the MSA kernels (gfx950 only).
#pragma once

#include "msa_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;   // d_h and d_I supported by these kernels
constexpr int kBlock = 128;     // Bk supported by these kernels
constexpr int kRowBytes = kHeadDim * 2;  // one bf16 row of 128 values

// 1/sqrt(128) in double; the fp32 score is the fp32 nearest to dot * this
// value (one fp64 multiply, one rounding), i.e. the fp32 nearest to the exact
// score whenever the dot product itself is exact.
constexpr double kInvSqrt128 = 0.088388347648318440550;

// 16-byte load marked non-temporal: for data read exactly once (partial
// results in the combine), so that it does not displace reused lines in L2.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_once(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_to_f32(u16 h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware instruction (no denormal range handling: results
// below 2^-126 flush to zero, which softmax weights can afford).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
//   A: lane l holds row (l % 32), k = 8*(l/32) .. +7
//   B: lane l holds column (l % 32), k = 8*(l/32) .. +7
//   D: lane l, element r holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).
//   A: lane l holds row (l % 16), k = 8*(l/16) .. +7
//   B: lane l holds column (l % 16), k = 8*(l/16) .. +7
//   D: lane l, element r holds row 4*(l/16) + r, column l % 16
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp8 (OCP e4m3) operands: 32 values = 8 dwords per lane.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 as_i32x8(uint4 lo, uint4 hi) {
  i32x8 v;
  v[0] = static_cast<int>(lo.x); v[1] = static_cast<int>(lo.y);
  v[2] = static_cast<int>(lo.z); v[3] = static_cast<int>(lo.w);
  v[4] = static_cast<int>(hi.x); v[5] = static_cast<int>(hi.y);
  v[6] = static_cast<int>(hi.z); v[7] = static_cast<int>(hi.w);
  return v;
}

// D(32x32) += A(32x64) * B(64x32), e4m3 in (format code 0 for both operands,
// no block scales), fp32 accumulate.
//   A: lane l holds row (l % 32) and 32 of the 64 k values, the same 32 for
//      the lanes of one half-wave (l / 32); B: lane l holds column (l % 32)
//      and the same k values as A's lanes of its half-wave.  Any fixed
//      assignment of k to (half, byte) works as long as A and B agree; here
//      half h holds k = 32h .. 32h+31 in byte order.
//   D: as for the bf16 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16) += A(16x128) * B(128x16), e4m3 in: lane quarter l / 16 holds
// k = 32*(l/16) .. +31 of row / column l % 16; D as for the bf16 16x16 MFMA.
__device__ __forceinline__ f32x4 mfma16_f8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Row r of a 128 x 128 bf16 tile in LDS is 256 B = 16 chunks of 16 B.  Chunk
// c of row r is stored at chunk position c ^ (r & 15): sixteen consecutive
// rows read at the same logical chunk then hit sixteen different chunk
// positions, which covers all LDS banks once.
__device__ __forceinline__ int swz(int r, int c) {
  return (r << 8) + ((c ^ (r & 15)) << 4);
}

// Paged decode caches (PagedCache, msa_internal.h): lengths are clamped to
// [1, cap] and page ids to [0, pages - 1], so that bad table contents give
// wrong results but never an access outside the pool.
__device__ __forceinline__ int64_t paged_len(const PagedCache& pc, int64_t b, int64_t cap) {
  if (!pc.table) return cap;
  const int64_t n = pc.lens[b];
  return n < 1 ? 1 : (n > cap ? cap : n);
}

__device__ __forceinline__ int64_t paged_page(const PagedCache& pc, int64_t b, int64_t j) {
  const int64_t pg = pc.table[b * pc.nb + j];
  return pg < 0 ? 0 : (pg >= pc.pages ? pc.pages - 1 : pg);
}

// Exchanges between the two half-waves (lane l and lane l ^ 32) with
// v_permlane32_swap, a VALU lane swap that needs no LDS round trip.  The
// swap of (a, b) leaves lanes 0-31 holding a's two halves and lanes 32-63
// holding b's, one per returned register.
__device__ __forceinline__ float halves_max2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(x[l], x[l ^ 32]) in lane l (the same value in both lanes).
__device__ __forceinline__ float halves_max(float x) { return halves_max2(x, x); }

// x[l] + x[l ^ 32] in lane l; equal to x + __shfl_xor(x, 32) bit for bit
// (the sum of two values does not depend on their order).
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lanes 0-31: a[l] + a[l + 32]; lanes 32-63: b[l - 32] + b[l].
__device__ __forceinline__ float halves_sum2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16_swap, then
// the half-wave swap); the sum equals the two __shfl_xor steps bit for bit.
__device__ __forceinline__ float quads_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return halves_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quads_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return halves_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return fmaxf(a, fmaxf(b, c));
}

// max(m, the 16 values of an accumulator tile) as a tree of three-input maxima
// (v_max3_f32), depth three.
__device__ __forceinline__ float max16(float m, const f32x16& c) {
  const float a = max3(c[0], c[1], c[2]), b = max3(c[3], c[4], c[5]);
  const float d = max3(c[6], c[7], c[8]), e = max3(c[9], c[10], c[11]);
  const float f = max3(c[12], c[13], c[14]);
  return max3(m, max3(a, b, d), max3(e, f, c[15]));
}

}  // namespace msa
