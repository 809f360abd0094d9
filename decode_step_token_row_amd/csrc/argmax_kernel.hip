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
// VGPRs each) keep 256 KB per CU in flight.  Each thread keeps the data of
// the first group reaching its maximum, so the lowest index is found from
// registers once the block maximum is known.  Special maxima (NaN patterns, zeros, -inf) take the same
// exact float32 path as the general kernel.
constexpr int kFastNT = 512;
constexpr int kFastQ = 32;
constexpr int64_t kFastGroups = (int64_t)kFastNT * kFastQ;

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

  int best = INT_MIN;
  int bq = 0;  // the first of the thread's groups reaching its maximum, and its data
  u32x4 bdat = d[0];
#pragma unroll
  for (int q = 0; q < kFastQ; ++q) {
    int g = KT::group_key(d[q]);
    g = tid < ngroups - q * kFastNT ? g : INT_MIN;
    const bool up = g > best;
    best = up ? g : best;
    bq = up ? q : bq;
    bdat.x = up ? d[q].x : bdat.x; bdat.y = up ? d[q].y : bdat.y;
    bdat.z = up ? d[q].z : bdat.z; bdat.w = up ? d[q].w : bdat.w;
  }

  const int wmax = wave_max_i32(best);
  if (lane == 0) s_red[wid] = wmax;
  if (tid == 0) s_idx = 0xFFFFFFFFu;
  __syncthreads();
  int K = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) K = K > s_red[w] ? K : s_red[w];

  const bool special = K > KT::kPosInf || K <= KT::kNegInf || K == 0 || K == -1;
  if (!special) {
    uint32_t idx = 0xFFFFFFFFu;
    if (best == K) {
      const uint32_t base = (uint32_t)(bq * kFastNT + tid) * 8u;
#pragma unroll
      for (int e = 7; e >= 0; --e)
        if (KT::elem_key(bdat, e) == K) idx = base + (uint32_t)e;
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
