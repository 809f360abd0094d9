// Top-n log-probabilities per row over [B, V] logits (bf16 or fp32), one
// workgroup per row.
//
// Next to the drawn token, the Arc engine's host sampler reports the most
// probable tokens with their log-probabilities, found by a partial sort of
// the probabilities (Arc PR #222, section 3(c)).  Per row, at temperature T:
//   z    = logits widened to float32 (NaN -> -inf, -0 -> +0), m = max z;
//   w_v  = exp((z_v - m) / T), with w = 1 where z_v == m (this covers +inf
//          and a row of -inf, which is then uniform);
//   S    = sum of w;  logprob_v = (z_v - m) / T - ln S (0 - ln S where z_v == m);
// output: the first n ids of the order (z descending, id ascending) and
// their logprobs.
//
// One HBM pass.  Each thread keeps its largest value with the first unit
// that holds it, and an online sum of its weights relative to its own
// maximum, rescaled when that maximum grows, so the normaliser needs no
// second pass.
//
// The bound works at unit granularity: an element's coarse key is its value
// order key << 32 | ~(first id of its unit), and the thread maxima become
// such keys (distinct across threads).  The order (value desc, id asc) only
// refines the coarse order, so the row's first n elements all have coarse
// keys at or above beta, the n-th largest thread key, and only the n threads
// whose key reaches beta can hold them.  beta is found without sorting: each
// wave finds the n-th and the ceil(n/8)-th largest value halves of its 64
// keys by bitwise descents over ballots; the largest of the first 16 values
// and the 8th largest of the second 16 both bound beta from below; the keys
// at or above the higher bound go to LDS, and the one of rank n - 1 among
// them, counted by quads of threads, is beta.
//
// The units of those n threads are read again (from cache), spread over the
// whole workgroup, and their elements with coarse key at or above beta are
// gathered into LDS with their exact keys (at most n * 256); each
// candidate's rank among the candidates is its position in the output.
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace arcs {

constexpr int kLpNT = 1024;
constexpr int kLpNW = kLpNT / kWave;
constexpr int kLpPerThread = 256;                                  // elements a thread owns at most
static_assert((int64_t)kLpNT * kLpPerThread == ARCS_TOP_LOGPROBS_MAX_VOCAB, "vocabulary bound");
constexpr int kLpCap = ARCS_MAX_TOP_LOGPROBS * kLpPerThread;       // candidates at most
constexpr int kLpBatch = 16;                                       // loads in flight per thread
constexpr size_t kLpLds = (size_t)kLpCap * 8 + (size_t)kLpNT * 8;  // candidates + survivors

__device__ __forceinline__ uint64_t lp_key(float z, uint32_t id) {
  return ((uint64_t)ord_key(z) << 32) | (uint64_t)(~id);
}

// How many of the `cnt` keys in `list` (LDS, 16-byte aligned) exceed k,
// stopping once `stop` is reached (checked every 16 keys).  Keys are read two
// at a time, eight reads in flight; reads past the end are clamped to the
// last pair and not counted.
__device__ __forceinline__ int lp_rank(const uint64_t* list, int cnt, uint64_t k, int stop) {
  const u32x4* pairs = (const u32x4*)list;
  const int last = (cnt - 1) >> 1;
  int r = 0;
  for (int j0 = 0; j0 < cnt && r < stop; j0 += 16) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pj = (j0 >> 1) + u;
      v[u] = pairs[pj < last ? pj : last];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + 2 * u;
      const uint64_t a = ((uint64_t)v[u].y << 32) | v[u].x, b = ((uint64_t)v[u].w << 32) | v[u].z;
      r += (int)((j < cnt) & (a > k)) + (int)((j + 1 < cnt) & (b > k));
    }
  }
  return r;
}

// A thread's unit of the row: 16 bytes (8 bf16 or 4 fp32) on the vector
// path, one element otherwise.
template <bool BF16, bool VEC>
struct LpUnit {
  static constexpr int E = VEC ? (BF16 ? 8 : 4) : 1;
  using Raw = typename std::conditional<VEC, u32x4, uint32_t>::type;
  static __device__ __forceinline__ Raw load(const char* rowp, int g) {
    if constexpr (VEC) {
      return __builtin_nontemporal_load(&((const u32x4*)rowp)[g]);  // streamed: read once
    } else if constexpr (BF16) {
      return (uint32_t)((const uint16_t*)rowp)[g] << 16;
    } else {
      return ((const uint32_t*)rowp)[g];
    }
  }
  // raw values: NaN and -0 as they are (the pass copes with both)
  static __device__ __forceinline__ void unpack(const Raw& d, float (&z)[E]) {
    if constexpr (VEC && BF16) {
      z[0] = bf16_lo(d.x); z[1] = bf16_hi(d.x); z[2] = bf16_lo(d.y); z[3] = bf16_hi(d.y);
      z[4] = bf16_lo(d.z); z[5] = bf16_hi(d.z); z[6] = bf16_lo(d.w); z[7] = bf16_hi(d.w);
    } else if constexpr (VEC) {
      z[0] = __uint_as_float(d.x); z[1] = __uint_as_float(d.y);
      z[2] = __uint_as_float(d.z); z[3] = __uint_as_float(d.w);
    } else {
      z[0] = __uint_as_float(d);
    }
  }
  static __device__ __forceinline__ void unpack_canon(const Raw& d, float (&z)[E]) {
    unpack(d, z);
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = canon_nan(z[e]) + 0.0f;  // NaN -> -inf, -0 -> +0
  }
};

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kLpNT, 1) void top_logprobs_kernel(LogprobArgs a) {
  using U = LpUnit<BF16, VEC>;
  constexpr int E = U::E;
  extern __shared__ __attribute__((aligned(16))) unsigned char lp_smem[];
  uint64_t* cand = (uint64_t*)lp_smem;
  uint64_t* surv = cand + kLpCap;
  __shared__ float s_max[kLpNW];
  __shared__ double s_sum[kLpNW];
  __shared__ uint64_t s_beta;
  __shared__ uint32_t s_cnt, s_nsurv;
  __shared__ uint64_t s_wbound[kLpNW], s_wbound8[kLpNW];
  __shared__ int s_owner[ARCS_MAX_TOP_LOGPROBS];  // the threads whose maximum reaches beta

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t row = blockIdx.x;
  const int n = a.n;
  int32_t* oid = a.out_ids + row * n;
  float* olp = a.out_logprobs + row * n;

  // the temperature is checked after the pass (a bad row runs the pass at
  // T = 1 and drops the result), so that no branch on it sits before the
  // row's loads
  const float T0 = a.temperature ? a.temperature[row] : 1.0f;
  const bool bad_t = !(T0 > 0.0f && T0 < __builtin_inff());
  const float T = bad_t ? 1.0f : T0;
  const double cd = 1.4426950408889634 / (double)T;  // log2(e) / T
  const float c = (float)cd;

  const char* rowp = (const char*)a.logits + row * a.stride * (BF16 ? 2 : 4);
  const int ngroups = (int)(VEC ? a.V / E : a.V);
  const int nq = (ngroups + kLpNT - 1) / kLpNT;

  // ---- the pass: thread maximum (first unit) and weights relative to it -----
  // A NaN never wins a comparison, so the maximum is that of the row with NaN
  // as -inf; a NaN weight, or an infinite maximum (inf - inf), leaves s
  // wrong or NaN, and such a thread recounts its weights exactly after the pass.
  float mt = -__builtin_inff();
  double s = 0.0;
  uint32_t first = (uint32_t)tid * E;  // first id of the first unit holding mt
  for (int q0 = 0; q0 < nq; q0 += kLpBatch) {
    // unconditional loads (a lane past the row's end reads its last unit
    // again and ignores it), all issued before the first use: with a branch
    // per unit, or left to the scheduler, they were spread out and waited
    // for one by one
    typename U::Raw d[kLpBatch];
#pragma unroll
    for (int r = 0; r < kLpBatch; ++r) {
      const int g = (q0 + r) * kLpNT + tid;
      d[r] = U::load(rowp, g < ngroups ? g : ngroups - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // no branch on the unit: with the units' uses inside a branch the
    // compiler moved each load into its branch, behind the previous unit's
    // wait.  Lanes past the row's end compute on their copy of the last unit
    // and keep nothing.
#pragma unroll
    for (int r = 0; r < kLpBatch; ++r) {
      const int g = (q0 + r) * kLpNT + tid;
      const bool valid = g < ngroups;
      float z[E];
      U::unpack(d[r], z);
      float gm = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < E; ++e) gm = __builtin_fmaxf(gm, z[e]);  // ignores NaN
      gm = valid ? gm : -__builtin_inff();
      const bool up = gm > mt;
      const float f = __builtin_amdgcn_exp2f((mt - gm) * c);  // 0 when mt is -inf or gm is +inf
      s = up ? s * (double)f : s;
      first = up ? (uint32_t)g * E : first;
      mt = up ? gm : mt;
      // z c - mt c in one fma (the logprobs' error budget holds the
      // difference of one rounding)
      const float nmc = -(mt * c);
      float ws = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) ws += __builtin_amdgcn_exp2f(__builtin_fmaf(z[e], c, nmc));
      s += valid ? (double)ws : 0.0;
    }
  }
  if (bad_t) {  // the same in every thread of the workgroup
    if (tid < n) { oid[tid] = -1; olp[tid] = __builtin_nanf(""); }
    if (tid == 0 && a.out_status) a.out_status[row] = ARCS_ROW_BAD_TEMPERATURE;
    return;
  }
  const bool owns = tid < ngroups;
  if (owns && !(s == s && __builtin_fabsf(mt) < __builtin_inff())) {
    // exact weights: w = 1 where z == mt (+inf, or a thread of -inf), NaN as -inf
    s = 0.0;
    for (int q = 0; q < nq; ++q) {
      const int g = q * kLpNT + tid;
      if (g >= ngroups) break;
      float z[E];
      U::unpack_canon(U::load(rowp, g), z);
#pragma unroll
      for (int e = 0; e < E; ++e) s += z[e] == mt ? 1.0 : (double)__builtin_amdgcn_exp2f((z[e] - mt) * c);
    }
  }

  // ---- row maximum and the wave bounds, normaliser and survivors ------------------
  // thread keys (coarse): value order key << 32 | ~(first id of the unit); each wave's
  // n-th largest key by a descent over ballots: the largest p with n keys at
  // or above it.  With fewer threads holding elements than n, every element
  // is a candidate (beta = 0).
  const uint64_t tkey = owns ? lp_key(mt, first) : 0ull;
  const bool few = ngroups < n;
  // Also each wave's ceil(n/8)-th largest key: eight waves with that many
  // keys at or above a value put n keys there, so the 8th largest of those 16
  // values is a lower bound for beta too, and usually a much higher one.
  // The descents run on the value half of the keys (32 steps): n keys with
  // value key >= v are n keys >= v << 32, so the bounds stay valid; value
  // ties can let more keys survive, never more than the 1024 thread keys.
  uint32_t p = 0u, p8 = 0u;
  if (!few) {
    const int n8 = (n + 7) / 8;
    const uint32_t th = (uint32_t)(tkey >> 32);
    // bf16 values: the low 16 bits of every value key are equal for one sign
    // (0 for positive values, all ones for negative ones), so the descent
    // stops at bit 16: the bound it gives keeps the same keys
    constexpr int kLowBit = BF16 ? 16 : 0;
#pragma unroll
    for (int b = 31; b >= kLowBit; --b) {
      const uint32_t c1 = p | (1u << b), c8 = p8 | (1u << b);
      p = __builtin_popcountll(__ballot(th >= c1)) >= n ? c1 : p;
      p8 = __builtin_popcountll(__ballot(th >= c8)) >= n8 ? c8 : p8;
    }
  }
  const float wm = dpp_wave_max_f32(mt);
  if (lane == 0) { s_max[wid] = wm; s_wbound[wid] = (uint64_t)p << 32; s_wbound8[wid] = (uint64_t)p8 << 32; }
  if (tid == 0) { s_cnt = 0u; s_nsurv = 0u; }
  if (few && tid < ngroups) s_owner[tid] = tid;
  __syncthreads();
  float m = s_max[0];
#pragma unroll
  for (int w = 1; w < kLpNW; ++w) m = s_max[w] > m ? s_max[w] : m;
  const double f = mt == m ? 1.0 : exp2(((double)mt - (double)m) * cd);
  const double ws = dpp_wave_sum_f64(owns ? s * f : 0.0);
  if (lane == 0) s_sum[wid] = ws;
  if (!few) {
    // the largest wave bound is a lower bound for beta: the keys at or above
    // it (at most n per wave, save value ties) go to LDS
    uint64_t lb = s_wbound[0];
#pragma unroll
    for (int w = 1; w < kLpNW; ++w) lb = s_wbound[w] > lb ? s_wbound[w] : lb;
    {
      // the 8th largest wave value of p8: raise lb to it (ties count once
      // each).  Lane w < 16 ranks wave w's value against the others; the
      // lane of rank 7 holds it.
      const int wl = lane < kLpNW ? lane : 0;
      const uint64_t vw = s_wbound8[wl];
      int above = 0;  // values strictly above vw, and equal ones before it
#pragma unroll
      for (int u = 0; u < kLpNW; ++u) {
        const uint64_t vu = s_wbound8[u];
        above += (vu > vw || (vu == vw && u < wl)) ? 1 : 0;
      }
      const uint64_t sel = __ballot(lane < kLpNW && above == 7);
      const int sl = __builtin_ctzll(sel | (1ull << 63));  // exactly one lane of rank 7
      const uint64_t x = sel ? ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(vw >> 32), sl) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)vw, sl)
                             : 0ull;
      lb = x > lb ? x : lb;
    }
    const bool keep = owns && tkey >= lb;
    const uint64_t mask = __ballot(keep);
    uint32_t base = 0;
    if (lane == 0 && mask) base = atomicAdd(&s_nsurv, (uint32_t)__builtin_popcountll(mask));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
    if (keep) surv[base + (uint32_t)__builtin_popcountll(mask & ((1ull << lane) - 1ull))] = tkey;
  }
  __syncthreads();
  double S = 0.0;
#pragma unroll
  for (int w = 0; w < kLpNW; ++w) S += s_sum[w];
  const double lnS = log(S);

  // ---- beta: the n-th largest thread key ----------------------------------------
  uint64_t beta = 0ull;
  const int nown = few ? ngroups : n;
  if (!few) {
    const int ns = (int)s_nsurv;
    // a survivor's rank: up to 256 survivors take a quad of threads each,
    // every thread counting over a quarter of the list
    const int split = ns <= kLpNT / 4 ? 4 : 1;
    const int si = tid / split, part = tid - si * split;
    const int chunk = ((ns + 2 * split - 1) / (2 * split)) * 2;  // even: pair reads stay aligned
    const int j0 = part * chunk < ns ? part * chunk : ns;
    const int j1 = j0 + chunk < ns ? j0 + chunk : ns;
    uint64_t k = 0ull;
    int rr = 0;
    if (si < ns) {
      k = surv[si];
      rr = lp_rank(surv + j0, j1 - j0, k, kLpCap);
    }
    if (split == 4) {
      rr += __shfl_xor(rr, 1);
      rr += __shfl_xor(rr, 2);
    }
    if (si < ns && part == 0) {
      if (rr == n - 1) s_beta = k;
      if (rr < n) s_owner[rr] = (int)((~(uint32_t)k) / (uint32_t)E) % kLpNT;
    }
    __syncthreads();
    beta = s_beta;
  }

  // ---- gather every element at or above beta ----------------------------------
  const float vb = beta ? key_value((uint32_t)(beta >> 32)) : -__builtin_inff();
  auto scan = [&](const typename U::Raw& dr, int g) {
    float z[E];
    U::unpack_canon(dr, z);
    float gm = z[0];
#pragma unroll
    for (int e = 1; e < E; ++e) gm = z[e] > gm ? z[e] : gm;
    if (gm >= vb) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lp_key(z[e], (uint32_t)g * E) >= beta) {  // coarse key: the unit's first id
          const uint32_t slot = atomicAdd(&s_cnt, 1u);
          if (slot < (uint32_t)kLpCap) cand[slot] = lp_key(z[e], (uint32_t)g * E + (uint32_t)e);
        }
      }
    }
  };
  // item (c, q): unit q of owner c, that is unit q * kLpNT + s_owner[c]
  const int items = nown * nq;
  for (int it = tid; it < items; it += kLpNT) {
    const int q = it / nown;
    const int g = q * kLpNT + s_owner[it - q * nown];
    if (g < ngroups) scan(U::load(rowp, g), g);
  }
  __syncthreads();
  const int nc = (int)(s_cnt < (uint32_t)kLpCap ? s_cnt : (uint32_t)kLpCap);

  // ---- the first n candidates in order, and their logprobs --------------------
  auto emit = [&](int r, uint64_t k) {
    const float z = key_value((uint32_t)(k >> 32));
    const double lw = z == m ? 0.0 : ((double)z - (double)m) / (double)T;
    oid[r] = (int32_t)(~(uint32_t)k);
    olp[r] = (float)(lw - lnS);
  };
  for (int i = tid; i < nc; i += kLpNT) {
    const uint64_t k = cand[i];
    const int r = lp_rank(cand, nc, k, n);
    if (r < n) emit(r, k);
  }
  if (tid >= nc && tid < n) {  // the row has fewer than n elements
    oid[tid] = -1;
    olp[tid] = -__builtin_inff();
  }
  if (tid == 0 && a.out_status) a.out_status[row] = ARCS_ROW_OK;
}

hipError_t launch_top_logprobs(const LogprobArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream) {
  const bool bf16 = dtype == ARCS_DTYPE_BF16;
  const bool v = vec && a.V % (bf16 ? 8 : 4) == 0;
  const void* fn = bf16 ? (v ? (const void*)top_logprobs_kernel<true, true> : (const void*)top_logprobs_kernel<true, false>)
                        : (v ? (const void*)top_logprobs_kernel<false, true> : (const void*)top_logprobs_kernel<false, false>);
  static std::atomic<int> done[4];
  const int which = (bf16 ? 2 : 0) + (v ? 1 : 0);
  if (!done[which].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLpLds);
    if (e != hipSuccess) return e;
    done[which].store(1, std::memory_order_release);
  }
  dim3 grid((unsigned)B), block(kLpNT);
  if (bf16) {
    if (v) hipLaunchKernelGGL((top_logprobs_kernel<true, true>), grid, block, kLpLds, stream, a);
    else hipLaunchKernelGGL((top_logprobs_kernel<true, false>), grid, block, kLpLds, stream, a);
  } else {
    if (v) hipLaunchKernelGGL((top_logprobs_kernel<false, true>), grid, block, kLpLds, stream, a);
    else hipLaunchKernelGGL((top_logprobs_kernel<false, false>), grid, block, kLpLds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace arcs
