// Row-wise argmax over [B, V] logits (bf16 or fp32), one workgroup per row.
//
// Arc PR #217 ("device decode loop", "What this does", step 2) computes the
// greedy token on the device into an i32[batch] buffer and checks it bit for
// bit against the host argmax.  This kernel does the same for a batch: one
// HBM pass with 16-byte loads, ties broken by the lowest index.
//
// Hot loop: each 16-byte load holds 8 bf16 (or 4 fp32) values.  Values are
// compared as signed integer keys (packed 16-bit keys and v_pk_max_i16 for
// bf16), which is exact value order for every non-NaN pattern except that
// -0 sorts just below +0.  Rows whose maximum key is a NaN pattern, a zero
// or -inf take an exact float32 slow path instead (NaN counts as -inf,
// -0 == +0).  Per lane the first group reaching the lane maximum is
// remembered; after the block maximum is known, candidate lanes re-read that
// one group to find the lowest index.
#include "device_common.hpp"
#include "launch.hpp"

namespace arcs {

template <bool BF16>
struct KeyTraits;
template <>
struct KeyTraits<true> {  // keys of bf16 patterns as int16 sign-extended
  static constexpr int kPosInf = 0x7F80;
  static constexpr int kNegInf = (int)(short)(0xFF80 ^ 0x7FFF);
  static __device__ __forceinline__ int scalar_key(const char* rowp, int64_t i) {
    short s = ((const short*)rowp)[i];
    return (int)(short)(s ^ ((s >> 15) & 0x7FFF));
  }
  static __device__ __forceinline__ int group_key(u32x4 v) {
    s16x2 k = max2(max2(bf16x2_keys(v.x), bf16x2_keys(v.y)), max2(bf16x2_keys(v.z), bf16x2_keys(v.w)));
    return max_halves(k);
  }
  static __device__ __forceinline__ int elem_key(u32x4 v, int e) {
    uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    short s = (short)((e & 1) ? (w >> 16) : (w & 0xFFFF));
    return (int)(short)(s ^ ((s >> 15) & 0x7FFF));
  }
  static __device__ __forceinline__ float scalar_value(const char* rowp, int64_t i) {
    return bf16_to_f32(((const uint16_t*)rowp)[i]);
  }
};
template <>
struct KeyTraits<false> {  // keys of fp32 patterns as int32
  static constexpr int kPosInf = 0x7F800000;
  static constexpr int kNegInf = (int)(0xFF800000u ^ 0x7FFFFFFFu);
  static __device__ __forceinline__ int scalar_key(const char* rowp, int64_t i) {
    return f32_key_signed(((const uint32_t*)rowp)[i]);
  }
  static __device__ __forceinline__ int group_key(u32x4 v) {
    int a = f32_key_signed(v.x), b = f32_key_signed(v.y), c = f32_key_signed(v.z), d = f32_key_signed(v.w);
    a = a > b ? a : b;
    c = c > d ? c : d;
    return a > c ? a : c;
  }
  static __device__ __forceinline__ int elem_key(u32x4 v, int e) {
    uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    return f32_key_signed(w);
  }
  static __device__ __forceinline__ float scalar_value(const char* rowp, int64_t i) {
    return ((const float*)rowp)[i];
  }
};

template <int NT, bool BF16, bool VEC, int U>
__global__ __launch_bounds__(NT) void argmax_kernel(const void* __restrict__ logits, int64_t V,
                                                    int64_t stride, int32_t* __restrict__ out) {
  using KT = KeyTraits<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;
  constexpr int NW = NT / kWave;
  __shared__ int s_red[NW];
  __shared__ float s_redf[NW];
  __shared__ int s_idx;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const char* rowp = (const char*)logits + (int64_t)blockIdx.x * stride * ES;
  const int64_t n_vec = VEC ? V / EPL : 0;
  const u32x4* rv = (const u32x4*)rowp;

  int best = INT_MIN;
  int64_t bpos = -1;
  bool bgroup = false;
  for (int64_t base = tid; base < n_vec; base += (int64_t)NT * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t j = base + (int64_t)u * NT;
      if (j < n_vec) v[u] = __builtin_nontemporal_load(rv + j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t j = base + (int64_t)u * NT;
      if (j < n_vec) {
        int g = KT::group_key(v[u]);
        if (g > best) { best = g; bpos = j * EPL; bgroup = true; }
      }
    }
  }
  for (int64_t i = n_vec * EPL + tid; i < V; i += NT) {
    int k = KT::scalar_key(rowp, i);
    if (k > best) { best = k; bpos = i; bgroup = false; }
  }

  int wmax = wave_max_i32(best);
  if (lane == 0) s_red[wid] = wmax;
  if (tid == 0) s_idx = INT_MAX;
  __syncthreads();
  int K = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) K = K > s_red[w] ? K : s_red[w];

  const bool special = K > KT::kPosInf || K <= KT::kNegInf || K == 0 || K == -1;
  if (!special) {
    if (best == K) {
      int64_t idx = bpos;
      if (bgroup) {
        u32x4 v = rv[bpos / EPL];
#pragma unroll
        for (int e = EPL - 1; e >= 0; --e)
          if (KT::elem_key(v, e) == K) idx = bpos + e;
      }
      atomicMin(&s_idx, (int)idx);
    }
    __syncthreads();
    if (tid == 0) out[blockIdx.x] = s_idx;
    return;
  }

  // Exact slow path: float32 values, NaN -> -inf, -0 == +0, first index.
  float bf = -__builtin_inff();
  int bi = -1;
  for (int64_t i = tid; i < V; i += NT) {
    float z = canon_nan(KT::scalar_value(rowp, i));
    if (z > bf) { bf = z; bi = (int)i; }
  }
  float wm = wave_max_f32(bf);
  __syncthreads();
  if (lane == 0) s_redf[wid] = wm;
  __syncthreads();
  float M = s_redf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = M > s_redf[w] ? M : s_redf[w];
  if (M == -__builtin_inff()) {
    if (tid == 0) out[blockIdx.x] = 0;
    return;
  }
  if (bf == M) atomicMin(&s_idx, bi);
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = s_idx;
}

// bf16 rows of at most kFastGroups groups of 8 (V % 8 == 0, 16-byte aligned
// rows): kFastNT threads, each owning the groups j = q * kFastNT + tid, with
// all kFastQ loads of the row issued at once through buffer resources that
// cover only the rest of the row (lanes past the end read zeros without
// touching memory).  512 threads x 32 loads (two waves per SIMD, up to 256
// VGPRs each) keep 256 KB per CU in flight.
//
// The pass works on the raw 16-bit patterns as signed integers, with no
// per-element order transform: non-negative floats order like their
// patterns, negative ones in reverse, so a thread's largest value is its
// largest pattern when that is >= 0 and otherwise its smallest pattern.
// Each round reduces its group with packed 16-bit max and min, and the two
// halves of each go into signed 32-bit keys (pattern << 16 | round code)
// reduced with max / min: the round code (31 - q for the maximum, q for the
// minimum) makes the first round holding a thread's extreme win ties.  After
// the block maximum is known, each thread holding it finds the element in
// that round's registers.  Special maxima (NaN patterns, zeros, -inf) take
// the same exact float32 path as the general kernel.
constexpr int kFastNT = 512;
constexpr int kFastQ = 32;
constexpr int64_t kFastGroups = (int64_t)kFastNT * kFastQ;
static_assert(kFastQ <= 32, "round codes and the round switch cover 32 rounds");


__global__ __launch_bounds__(kFastNT) void argmax_fast_kernel(const void* __restrict__ logits, int64_t V,
                                                              int64_t stride, int32_t* __restrict__ out) {
  using KT = KeyTraits<true>;
  constexpr int NW = kFastNT / kWave;
  __shared__ int s_red[NW];
  __shared__ float s_redf[NW];
  __shared__ uint32_t s_idx;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const char* rowp = (const char*)logits + (int64_t)blockIdx.x * stride * 2;
  const u32x4* rv = (const u32x4*)rowp;
  const int ngroups = (int)(V / 8);

  u32x4 d[kFastQ];
  const int voff = tid * 16;
#pragma unroll
  for (int q = 0; q < kFastQ; ++q) {
    const int left = (ngroups - q * kFastNT) * 16;  // bytes of the row from round q on
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rv + (left > 0 ? q * kFastNT : 0)), (short)0, left > 0 ? left : 0, 0x00020000);
    d[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2 /* nt */));
  }
  __builtin_amdgcn_sched_barrier(0);

  int pk = INT_MIN, nk = INT_MAX;  // (largest pattern, 31 - round), (smallest pattern, round)
#pragma unroll
  for (int q = 0; q < kFastQ; ++q) {
    const uint32_t a = pk_max_u(pk_max_u(d[q].x, d[q].y), pk_max_u(d[q].z, d[q].w));
    const uint32_t b = pk_min_u(pk_min_u(d[q].x, d[q].y), pk_min_u(d[q].z, d[q].w));
    int ax = (int)((a << 16) | (uint32_t)(31 - q)), ay = (int)((a & 0xFFFF0000u) | (uint32_t)(31 - q));
    int bx = (int)((b << 16) | (uint32_t)q), by = (int)((b & 0xFFFF0000u) | (uint32_t)q);
    if ((q + 1) * kFastNT > ngroups) {  // a round the row does not fill (uniform)
      const bool valid = tid < ngroups - q * kFastNT;
      ax = valid ? ax : INT_MIN; ay = valid ? ay : INT_MIN;
      bx = valid ? bx : INT_MAX; by = valid ? by : INT_MAX;
    }
    pk = max(max(pk, ax), ay);
    nk = min(min(nk, bx), by);
    // keep the reduction in round order (no deferred trees of per-round keys)
    asm volatile("" : "+v"(pk), "+v"(nk));
  }
  const int cp = pk >> 16, cn = nk >> 16;
  const int raw = cp >= 0 ? cp : cn;
  const int qsel = cp >= 0 ? 31 - (pk & 0xFFFF) : (nk & 0xFFFF);
  int tk = (int)(short)(raw ^ ((raw >> 15) & 0x7FFF));  // the order key of the thread's largest value
  tk = tid < ngroups ? tk : INT_MIN;

  const int wmax = dpp_wave_max_i32(tk);
  if (lane == 0) s_red[wid] = wmax;
  if (tid == 0) s_idx = 0xFFFFFFFFu;
  __syncthreads();
  int K = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) K = K > s_red[w] ? K : s_red[w];

  const bool special = K > KT::kPosInf || K <= KT::kNegInf || K == 0 || K == -1;
  if (!special) {
    // the pattern of the maximum (not +-0, so patterns compare exactly)
    const uint32_t R = (uint32_t)(K ^ ((K >> 15) & 0x7FFF)) & 0xFFFFu;
    uint32_t idx = 0xFFFFFFFFu;
    uint64_t tied = __ballot(tk == K);
    while (tied) {
      const int t = __builtin_ctzll(tied);
      tied &= tied - 1;
      const int qu = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(qsel, t));
      u32x4 v = d[0];
      switch (qu) {
#define ARCS_ROUND_(i) case i: v = d[i]; break;
        ARCS_ROUND_(1) ARCS_ROUND_(2) ARCS_ROUND_(3) ARCS_ROUND_(4) ARCS_ROUND_(5) ARCS_ROUND_(6)
        ARCS_ROUND_(7) ARCS_ROUND_(8) ARCS_ROUND_(9) ARCS_ROUND_(10) ARCS_ROUND_(11) ARCS_ROUND_(12)
        ARCS_ROUND_(13) ARCS_ROUND_(14) ARCS_ROUND_(15) ARCS_ROUND_(16) ARCS_ROUND_(17) ARCS_ROUND_(18)
        ARCS_ROUND_(19) ARCS_ROUND_(20) ARCS_ROUND_(21) ARCS_ROUND_(22) ARCS_ROUND_(23) ARCS_ROUND_(24)
        ARCS_ROUND_(25) ARCS_ROUND_(26) ARCS_ROUND_(27) ARCS_ROUND_(28) ARCS_ROUND_(29) ARCS_ROUND_(30)
        ARCS_ROUND_(31)
#undef ARCS_ROUND_
        default: break;
      }
      uint32_t e = 8;
      e = (v.w >> 16) == R ? 7u : e;
      e = (v.w & 0xFFFFu) == R ? 6u : e;
      e = (v.z >> 16) == R ? 5u : e;
      e = (v.z & 0xFFFFu) == R ? 4u : e;
      e = (v.y >> 16) == R ? 3u : e;
      e = (v.y & 0xFFFFu) == R ? 2u : e;
      e = (v.x >> 16) == R ? 1u : e;
      e = (v.x & 0xFFFFu) == R ? 0u : e;
      if (lane == t && e < 8) {
        const uint32_t i = (uint32_t)(qu * kFastNT + tid) * 8u + e;
        idx = i < idx ? i : idx;
      }
    }
    const uint32_t wmin = dpp_wave_min_u32(idx);
    if (lane == 0 && wmin != 0xFFFFFFFFu) atomicMin(&s_idx, wmin);
    __syncthreads();
    if (tid == 0) out[blockIdx.x] = (int32_t)s_idx;
    return;
  }

  // Exact slow path: float32 values, NaN -> -inf, -0 == +0, first index.
  float bf = -__builtin_inff();
  int bi = -1;
  for (int64_t i = tid; i < V; i += kFastNT) {
    float z = canon_nan(KT::scalar_value(rowp, i));
    if (z > bf) { bf = z; bi = (int)i; }
  }
  float wm = wave_max_f32(bf);
  __syncthreads();
  if (lane == 0) s_redf[wid] = wm;
  __syncthreads();
  float M = s_redf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = M > s_redf[w] ? M : s_redf[w];
  if (M == -__builtin_inff()) {
    if (tid == 0) out[blockIdx.x] = 0;
    return;
  }
  if (bf == M) atomicMin(&s_idx, (uint32_t)bi);
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = (int32_t)s_idx;
}

// Launch configuration chosen per shape on the host side.
constexpr int kArgmaxThreads = 512;
constexpr int kArgmaxUnroll = 8;

hipError_t launch_argmax(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                         bool vec, int32_t* out, hipStream_t stream) {
  dim3 grid((unsigned)B), block(kArgmaxThreads);
  if (dtype == ARCS_DTYPE_BF16 && vec && V % 8 == 0 && V / 8 <= kFastGroups) {
    hipLaunchKernelGGL(argmax_fast_kernel, grid, dim3(kFastNT), 0, stream, logits, V, stride, out);
    return hipGetLastError();
  }
  if (dtype == ARCS_DTYPE_BF16) {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<kArgmaxThreads, true, true, kArgmaxUnroll>), grid, block, 0, stream, logits, V, stride, out);
    else
      hipLaunchKernelGGL((argmax_kernel<kArgmaxThreads, true, false, kArgmaxUnroll>), grid, block, 0, stream, logits, V, stride, out);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<kArgmaxThreads, false, true, kArgmaxUnroll>), grid, block, 0, stream, logits, V, stride, out);
    else
      hipLaunchKernelGGL((argmax_kernel<kArgmaxThreads, false, false, kArgmaxUnroll>), grid, block, 0, stream, logits, V, stride, out);
  }
  return hipGetLastError();
}

}  // namespace arcs
