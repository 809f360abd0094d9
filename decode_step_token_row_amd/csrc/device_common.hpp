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
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { int t = __shfl_xor(v, o, kWave); v = v < t ? v : t; }
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
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
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

}  // namespace arcs
