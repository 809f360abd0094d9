// Device-side building blocks shared by the argmax and sampling kernels.
//
// Everything here is written for gfx950 (CDNA4): 64-lane wavefronts, LDS
// reductions, 16-byte vector loads.  Floating-point rules follow the
// sampler's definition (Arc PR #222, section 3; penalties and the uniform as
// documented in include/arcs.h):
//   * a logit is widened to float32 exactly; NaN counts as -inf;
//   * -0 and +0 are the same value (keys are built from the canonical +0);
//   * the order of the filters is (value descending, id ascending).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arcs.h"

namespace arcs {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// NaN -> -inf (an ordered compare is false only for NaN).
__device__ __forceinline__ float canon_nan(float z) { return (z == z) ? z : -__builtin_inff(); }

// Order-preserving unsigned key of a float32 without NaN; -0 and +0 share
// the key of +0.  key(a) < key(b) iff a < b.
__device__ __forceinline__ uint32_t ord_key(float z) {
  uint32_t b = __float_as_uint(z + 0.0f);  // -0 + 0 = +0 under round-to-nearest
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t b = k ^ ((uint32_t)((int32_t)(~k) >> 31) | 0x80000000u);
  return __uint_as_float(b);
}

// Signed 16-bit keys of two packed bfloat16 values (raw bit order kept):
// a bf16 pattern s maps to s for s >= 0 and to s ^ 0x7FFF otherwise, so that
// signed comparison of keys is value order.  Positive NaN patterns land
// above +inf, negative NaN patterns below -inf, -0 just below +0: callers
// check the row maximum for those cases and take an exact slow path.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 bf16x2_keys(uint32_t x) {
  s16x2 v = __builtin_bit_cast(s16x2, x);
  s16x2 s = (v >> (s16x2)15) & (s16x2)0x7FFF;
  return v ^ s;
}
__device__ __forceinline__ s16x2 max2(s16x2 a, s16x2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ int max_halves(s16x2 a) { return a.x > a.y ? (int)a.x : (int)a.y; }
// Packed signed 16-bit max / min of two pairs of raw bf16 patterns.
__device__ __forceinline__ s16x2 as_s16x2(uint32_t x) { return __builtin_bit_cast(s16x2, x); }
__device__ __forceinline__ uint32_t pk_max_u(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_s16x2(a), as_s16x2(b)));
}
__device__ __forceinline__ uint32_t pk_min_u(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(as_s16x2(a), as_s16x2(b)));
}
__device__ __forceinline__ int f32_key_signed(uint32_t b) {
  return (int)(b ^ ((uint32_t)((int32_t)b >> 31) & 0x7FFFFFFFu));
}

// ---------------------------------------------------------------------------
// wave / block reductions (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { int t = __shfl_xor(v, o, kWave); v = v > t ? v : t; }
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { float t = __shfl_xor(v, o, kWave); v = v > t ? v : t; }
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// inclusive prefix sum across the wave
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint64_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output k of the generator
// started from state `seed` mixes seed + k * gamma.  The sampler uses output
// n + 1 with n = step * 2^32 + row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t splitmix64_counter_output(uint64_t seed, uint64_t row, uint64_t step) {
  uint64_t n = (step << 32) + row;
  return splitmix64_mix(seed + (n + 1) * 0x9E3779B97F4A7C15ull);
}

// ---------------------------------------------------------------------------
// fixed-point weights: W = floor(w * 2^F) for w in [0, 1], F <= 62.
// Exact for every float32 w (see the argument in the comment below).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t to_fixed(float w, float scale) {
  // x = w * 2^F is exact.  hi = trunc(x / 2^32) has at most 24 significant
  // bits, so (float)hi * 2^32 is exact and x - hi * 2^32 is the exact low
  // part (< 2^32), truncated to an integer by the conversion.
  float x = w * scale;
  float hf = x * 0x1p-32f;
  uint32_t hi = (uint32_t)hf;
  float lof = x - (float)hi * 0x1p32f;
  uint32_t lo = (uint32_t)lof;
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// ---------------------------------------------------------------------------
// DPP wave primitives (wave64, gfx9 DPP controls): register-to-register
// cross-lane moves, no LDS traffic.  Totals are taken from lane 63 and
// broadcast with v_readlane.
//   0xB1 quad_perm[1,0,3,2]  0x4E quad_perm[2,3,0,1]  0x141 row_half_mirror
//   0x140 row_mirror  0x111/0x112/0x114/0x118 row_shr 1/2/4/8
//   0x142 row_bcast:15 (rows 1,3 via row_mask 0xA)  0x143 row_bcast:31 (rows 2,3 via 0xC)
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __uint_as_float(dpp_u32<CTRL, ROWMASK>(__float_as_uint(old), __float_as_uint(v)));
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  const uint64_t o = __builtin_bit_cast(uint64_t, old), x = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_u32<CTRL, ROWMASK>((uint32_t)o, (uint32_t)x);
  const uint32_t hi = dpp_u32<CTRL, ROWMASK>((uint32_t)(o >> 32), (uint32_t)(x >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane63_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, 63), hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp_wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(0.0, v);
  v += dpp_f64<0x4E>(0.0, v);
  v += dpp_f64<0x141>(0.0, v);
  v += dpp_f64<0x140>(0.0, v);
  v += dpp_f64<0x142, 0xA>(0.0, v);
  v += dpp_f64<0x143, 0xC>(0.0, v);
  return readlane63_f64(v);
}
__device__ __forceinline__ float dpp_wave_max_f32(float v) {
  const float ni = -__builtin_inff();
  float t;
  t = dpp_f32<0xB1>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x4E>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x141>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x140>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x142, 0xA>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x143, 0xC>(ni, v); v = v > t ? v : t;
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
// Reductions over lanes 0..7 only (one record per wave of a 512-thread
// workgroup; the other lanes hold the identity): three butterfly steps inside
// the first half-row, the result read from lane 0.  Same pairing as the first
// three steps of the whole-wave versions, so sums come out identical.
// N = 16: a fourth step over the row of 16 lanes (row_mirror: lane i reads
// lane 15 - i, which after the first three holds the other octet's result).
template <int N = 8>
__device__ __forceinline__ float dpp_octet_max_f32(float v) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  const float ni = -__builtin_inff();
  float t;
  t = dpp_f32<0xB1>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x4E>(ni, v); v = v > t ? v : t;
  t = dpp_f32<0x141>(ni, v); v = v > t ? v : t;
  if constexpr (N == 16) { t = dpp_f32<0x140>(ni, v); v = v > t ? v : t; }
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
}
template <int N = 8>
__device__ __forceinline__ double dpp_octet_sum_f64(double v) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  v += dpp_f64<0xB1>(0.0, v);
  v += dpp_f64<0x4E>(0.0, v);
  v += dpp_f64<0x141>(0.0, v);
  if constexpr (N == 16) v += dpp_f64<0x140>(0.0, v);
  return readlane_f64(v, 0);
}
template <int N = 8>
__device__ __forceinline__ uint32_t dpp_octet_min_u32(uint32_t v) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  const uint32_t id = 0xFFFFFFFFu;
  uint32_t t;
  t = dpp_u32<0xB1>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x4E>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x141>(id, v); v = v < t ? v : t;
  if constexpr (N == 16) { t = dpp_u32<0x140>(id, v); v = v < t ? v : t; }
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
}
// 2^t in double precision: t = n + f with n = rint(t) and |f| <= 1/2, 2^f
// from the Taylor series of exp(f ln 2) to degree 9 (relative error about
// 1e-11 over the interval), scaled by 2^n.  t below -1100, and -inf, give 0;
// t above 1023 gives +inf.  The coefficients are (ln 2)^k / k!.
__device__ __forceinline__ double exp2_f64(double t) {
  t = t > -1100.0 ? t : -1100.0;
  const double n = __builtin_rint(t);
  const double f = t - n;
  double p = 0x1.b5253d395e7c4p-24;
  p = __builtin_fma(p, f, 0x1.62c0223a5c824p-20);
  p = __builtin_fma(p, f, 0x1.ffcbfc588b0c7p-17);
  p = __builtin_fma(p, f, 0x1.430912f86c787p-13);
  p = __builtin_fma(p, f, 0x1.5d87fe78a6731p-10);
  p = __builtin_fma(p, f, 0x1.3b2ab6fba4e77p-7);
  p = __builtin_fma(p, f, 0x1.c6b08d704a0c0p-5);
  p = __builtin_fma(p, f, 0x1.ebfbdff82c58fp-3);
  p = __builtin_fma(p, f, 0x1.62e42fefa39efp-1);
  p = __builtin_fma(p, f, 1.0);
  return __builtin_ldexp(p, (int)n);
}
// 2^t in double precision from a table T64[j] = 2^(j/64) (j = 0..63, filled
// by exp2_f64): t = n + j/64 + r with 64 n + j = rint(64 t) and |r| <= 1/128,
// 2^r from its Taylor series to degree 3 (relative error below 4e-11), the
// product scaled by 2^n.  t below -1100, and -inf, give 0; t above 1023
// gives +inf.  Three multiply-adds and one table read in place of ten.
__device__ __forceinline__ double exp2_f64_tab(double t, const double* T64) {
  t = t > -1100.0 ? t : -1100.0;
  const double s = __builtin_rint(t * 64.0);
  const double r = __builtin_fma(s, -0.015625, t);  // t - s / 64, exact
  const int si = (int)s;
  double p = __builtin_fma(0x1.c6b08d704a0c0p-5, r, 0x1.ebfbdff82c58fp-3);
  p = __builtin_fma(p, r, 0x1.62e42fefa39efp-1);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(T64[si & 63] * p, si >> 6);
}

// inclusive prefix sums across the wave (lane order)
__device__ __forceinline__ double dpp_wave_incl_scan_f64(double v) {
  v += dpp_f64<0x111>(0.0, v);
  v += dpp_f64<0x112>(0.0, v);
  v += dpp_f64<0x114>(0.0, v);
  v += dpp_f64<0x118>(0.0, v);
  v += dpp_f64<0x142, 0xA>(0.0, v);
  v += dpp_f64<0x143, 0xC>(0.0, v);
  return v;
}
__device__ __forceinline__ uint32_t dpp_wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<0x111>(0u, v);
  v += dpp_u32<0x112>(0u, v);
  v += dpp_u32<0x114>(0u, v);
  v += dpp_u32<0x118>(0u, v);
  v += dpp_u32<0x142, 0xA>(0u, v);
  v += dpp_u32<0x143, 0xC>(0u, v);
  return v;
}
// minimum across the wave (same value in every lane)
__device__ __forceinline__ uint32_t dpp_wave_min_u32(uint32_t v) {
  const uint32_t id = 0xFFFFFFFFu;
  uint32_t t;
  t = dpp_u32<0xB1>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x4E>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x141>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x140>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x142, 0xA>(id, v); v = v < t ? v : t;
  t = dpp_u32<0x143, 0xC>(id, v); v = v < t ? v : t;
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// maximum across the wave, signed (same value in every lane)
__device__ __forceinline__ int dpp_wave_max_i32(int v) {
  const uint32_t id = 0x80000000u;
  int t;
  t = (int)dpp_u32<0xB1>(id, (uint32_t)v); v = v > t ? v : t;
  t = (int)dpp_u32<0x4E>(id, (uint32_t)v); v = v > t ? v : t;
  t = (int)dpp_u32<0x141>(id, (uint32_t)v); v = v > t ? v : t;
  t = (int)dpp_u32<0x140>(id, (uint32_t)v); v = v > t ? v : t;
  t = (int)dpp_u32<0x142, 0xA>(id, (uint32_t)v); v = v > t ? v : t;
  t = (int)dpp_u32<0x143, 0xC>(id, (uint32_t)v); v = v > t ? v : t;
  return __builtin_amdgcn_readlane(v, 63);
}
// bitwise OR across the wave (same value in every lane)
__device__ __forceinline__ uint32_t dpp_wave_or_u32(uint32_t v) {
  v |= dpp_u32<0xB1>(0u, v);
  v |= dpp_u32<0x4E>(0u, v);
  v |= dpp_u32<0x141>(0u, v);
  v |= dpp_u32<0x140>(0u, v);
  v |= dpp_u32<0x142, 0xA>(0u, v);
  v |= dpp_u32<0x143, 0xC>(0u, v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// sum across the wave (same value in every lane)
__device__ __forceinline__ uint32_t dpp_wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)dpp_wave_incl_scan_u32(v), 63);
}

}  // namespace arcs
