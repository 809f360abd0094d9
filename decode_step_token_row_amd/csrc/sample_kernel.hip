// Batched token sampling over [B, V] logits, one workgroup per row.
//
// The method follows the Arc engine's pages:
//   * Arc PR #222 ("ARC_SAMPLE_ON_DEVICE"), section 3(b): after the
//     temperature softmax, top-k zeroes the rest, a top-p walk and a min-p
//     scan read the sorted probabilities, and a multinomial draw reads the
//     unsorted vector; under top_k = -1, top_p = 1, min_p = 0 nothing reads
//     the sort, so none is done.
//   * Arc PR #222, section 3(a): a penalty with multiplier 0 is a no-op.
//   * Arc PR #217 ("device decode loop", "Default OFF"): SplitMix64 drives
//     the device draw; the token id stays in device memory.
// No full-vocabulary sort is done anywhere.
//
// Two kernels:
//
// sample_summary_kernel (bf16 rows, 16-byte aligned, V <= 131072, V % 8 == 0,
//   no active penalties): the row is read from HBM exactly once, 8 x 16-byte
//   loads per lane in flight.  Each thread turns every group of 8 logits into
//   weights e = exp2(z*log2(e)/T - K_t) (K_t an integer reference from the
//   thread's first group, so rescaling between threads is an exact power of
//   two) and leaves a per-group summary in LDS: the group weight sum (fp32,
//   summed in id order) for no-filter rows, the group maximum (bf16) for
//   filter rows, plus an fp64 per-thread weight total.  After the pass:
//     greedy rows   -> block max, lowest index (one group re-read);
//     no filter     -> the draw scans per-thread chunk totals, then the
//                      chunk's group sums, then one group's 8 weights;
//     any filter    -> a lower bound on the cutoff from the group maxima
//                      (min-p's closed-form threshold, a group-count bound
//                      for top-k, a group-mass bound for top-p), the groups
//                      above it re-read and their candidates gathered into
//                      LDS, sorted by (value desc, id asc), the kept prefix
//                      cut, re-sorted by id, and the inverse-CDF draw done
//                      on it.
//   Rows the fast path cannot take exactly (NaN or +inf logits, extreme
//   values, more than kCandCap candidates, penalties) run the general
//   pipeline instead.
//
// sample_kernel (everything else): the general streaming pipeline of
//   sample_common.hpp -- pass A for max/argmax, fixed-point softmax mass,
//   radix-select cutoff over order-preserving keys, id-order draw -- with
//   re-walks of the row served from L2 / the Infinity Cache.
#include <atomic>

#include "sample_common.hpp"

namespace arcs {

constexpr int64_t kSummaryMaxV = (int64_t)kMaxGroups * 8;  // 131072

// ---------------------------------------------------------------------------
// general kernel
// ---------------------------------------------------------------------------
template <bool BF16, bool VEC, bool PEN>
__global__ __launch_bounds__(kNT) void sample_kernel(SampleArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const Smem sm = carve_smem(smem_raw, kUnionGeneric, a.bitmap_words);
  arcs_row_params P;
  PenCtx pc;
  uint32_t path;
  if (!row_prologue<BF16, PEN>(a, row, sm, sh, P, pc, path)) return;
  generic_row<BF16, VEC>(a, row, P, pc, path, sm, sh);
}

// ---------------------------------------------------------------------------
// summary kernel helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// 8 bf16 of a group -> float32, penalties applied to history ids.
template <bool PEN>
__device__ __forceinline__ void unpack8(u32x4 d, int64_t g0, int n, const PenCtx& pc, float (&z)[8]) {
  z[0] = bf16_lo(d.x); z[1] = bf16_hi(d.x);
  z[2] = bf16_lo(d.y); z[3] = bf16_hi(d.y);
  z[4] = bf16_lo(d.z); z[5] = bf16_hi(d.z);
  z[6] = bf16_lo(d.w); z[7] = bf16_hi(d.w);
  if (PEN && pc.on && n > 0) apply_penalties<8>(z, g0, n, pc);
}

// Weight of z relative to the integer reference K in log2 units:
// exp2(z*c - K) with c = chi + clo (chi rounded down, clo > 0, so -inf
// logits give exactly 0).
__device__ __forceinline__ float wexp(float z, float chi, float clo, float negK) {
  const float t = __builtin_fmaf(z, clo, __builtin_fmaf(z, chi, negK));
  return __builtin_amdgcn_exp2f(t);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Block-wide inclusive fp64 scan; also returns the block total.
__device__ __forceinline__ double block_incl_scan_f64(double v, Shared& sh, double& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_incl_scan_f64(v, lane);
  __syncthreads();
  if (lane == kWave - 1) sh.f64[wid] = v;
  __syncthreads();
  double off = 0.0, t = 0.0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const double x = sh.f64[w];
    off += (w < wid) ? x : 0.0;
    t += x;
  }
  total = t;
  return v + off;
}

// Bitonic sort (ascending) of one (key, payload) per lane across a wave.
__device__ __forceinline__ void wave_bitonic_sort(uint64_t& key, float& pay, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t ok = __shfl_xor(key, j, kWave);
      const float op = __shfl_xor(pay, j, kWave);
      const bool up = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      const bool take = lower ? (up ? ok < key : ok > key) : (up ? ok > key : ok < key);
      if (take) { key = ok; pay = op; }
    }
  }
}

// Bitonic sort (ascending) of n = 2^p (key, payload) pairs in LDS, whole block.
__device__ __forceinline__ void block_bitonic_sort(uint64_t* keys, float* pay, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kNT) {
        const int p = i ^ j;
        if (p > i) {
          const bool up = (i & k) == 0;
          const uint64_t x = keys[i], y = keys[p];
          if ((x > y) == up) {
            keys[i] = y; keys[p] = x;
            const float t = pay[i]; pay[i] = pay[p]; pay[p] = t;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Sort key of a candidate: ascending order = value descending, id ascending.
__device__ __forceinline__ uint64_t cand_key(float z, int64_t idx) {
  return ((uint64_t)(~ord_key(z)) << 32) | (uint64_t)(uint32_t)idx;
}

// ---------------------------------------------------------------------------
// summary kernel
// ---------------------------------------------------------------------------
constexpr int kU = 16;                   // groups per thread in flight (16 x 16 B loads)
constexpr int kQ = kMaxGroups / kNT;     // groups per thread over the row (16)

// Sequential group weight: the sum, in id order, of the 8 weights of a group.
__device__ __forceinline__ float group_weight(const float (&z)[8], float chi, float clo, float negK) {
  float s = wexp(z[0], chi, clo, negK);
#pragma unroll
  for (int e = 1; e < 8; ++e) s += wexp(z[e], chi, clo, negK);
  return s;
}

// Orders one wave's LDS stores before its later LDS loads from other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Block-wide inclusive fp64 scan with DPP inside waves; also returns the total.
__device__ __forceinline__ double block_scan_f64(double v, Shared& sh, double& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = dpp_wave_incl_scan_f64(v);
  __syncthreads();
  if (lane == kWave - 1) sh.f64[wid] = v;
  __syncthreads();
  double off = 0.0, t = 0.0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const double x = sh.f64[w];
    off += (w < wid) ? x : 0.0;
    t += x;
  }
  total = t;
  return v + off;
}

// Inverse-CDF draw in id order over per-thread group sums.  summ[q] is the
// weight of group q * kNT + tid (in the thread's frame 2^-K_t, elements
// below zmask excluded); dk = K_t - K* moves it to the common frame.  The
// target u * S_K is located in three steps: the group round (kNT
// consecutive groups), the thread inside the round (block scan), the element
// inside the thread's group (sequential fp32 partial sums, the same
// operations that produced summ).  Returns false when S_K is zero or not
// finite (uniform across the block); else id and S_K.
__device__ __forceinline__ bool round_draw(const float (&summ)[kQ], const u32x4* rv, float zmask, float chi,
                                           float clo, float negK, int dk, double u, Shared& sh, int64_t& id,
                                           double& S_K) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const double r = dpp_wave_sum_f64(__builtin_ldexp((double)summ[q], dk));
    if (lane == 0) sh.qt[q * kNW + wid] = r;
  }
  __syncthreads();
  if (wid == 0) {
    // lane q < kQ: the total of group round q (ids [q*kNT*8, (q+1)*kNT*8))
    double rt = 0.0;
    if (lane < kQ)
      for (int w = 0; w < kNW; ++w) rt += sh.qt[lane * kNW + w];
    const double incl = dpp_wave_incl_scan_f64(rt);
    const double tot = readlane63_f64(incl);
    const double t = u * tot;
    const uint64_t hit = __ballot(lane < kQ && rt > 0.0 && incl > t);
    const uint64_t nz = __ballot(lane < kQ && rt > 0.0);
    const int qs = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
    const double before = __shfl(incl - rt, qs, kWave);
    if (lane == 0) {
      sh.i32[1] = qs;
      sh.f64[kNW] = before;
      sh.f64[kNW + 1] = tot;
      sh.i32[4] = INT_MAX;
      sh.i32[5] = -1;
    }
  }
  __syncthreads();
  const int qs = __builtin_amdgcn_readfirstlane(sh.i32[1]);
  const double before_round = sh.f64[kNW];
  S_K = sh.f64[kNW + 1];
  if (!(S_K > 0.0) || !(S_K < 1e300)) return false;
  const double t = u * S_K;
  float mine_f = 0.0f;
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    if (q == qs) mine_f = summ[q];
  const double mine = __builtin_ldexp((double)mine_f, dk);
  double tot;
  const double incl = before_round + block_scan_f64(mine, sh, tot);
  if (mine > 0.0 && incl > t) atomicMin(&sh.i32[4], tid);
  if (mine > 0.0) atomicMax(&sh.i32[5], tid);
  __syncthreads();
  int owner = sh.i32[4];
  if (owner == INT_MAX) owner = sh.i32[5] < 0 ? 0 : sh.i32[5];  // rounding: the last thread with mass
  if (tid == owner) {
    const int jg = qs * kNT + tid;
    const double bl = incl - mine;
    float z[8];
    unpack8<false>(rv[jg], 0, 8, PenCtx{}, z);
    float acc = 0.0f, prev = 0.0f;
    int pe = -1, last_e = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = z[e] >= zmask ? wexp(z[e], chi, clo, negK) : 0.0f;
      acc = (e == 0) ? w : acc + w;
      const bool pos = acc > prev;
      if (pos) last_e = e;
      if (pe < 0 && pos && bl + __builtin_ldexp((double)acc, dk) > t) pe = e;
      prev = acc;
    }
    if (pe < 0) pe = last_e;
    sh.u64[10] = (uint64_t)(jg * 8 + pe);
  }
  __syncthreads();
  id = (int64_t)sh.u64[10];
  return true;
}

// Re-reads the row (from cache) and replaces summ[q] by the weight of
// group q * kNT + tid restricted to elements z >= zmask, summed in id order.
__device__ __forceinline__ void masked_group_sums(const u32x4* rv, int ngroups, float zmask, float chi, float clo,
                                                  float negK, float (&summ)[kQ]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < kQ / kU; ++it) {
    if (it * kNT * kU >= ngroups) {
#pragma unroll
      for (int u = 0; u < kU; ++u) summ[it * kU + u] = 0.0f;
      continue;
    }
    u32x4 d[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = (it * kU + u) * kNT + tid;
      d[u] = rv[j < ngroups ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = it * kU + u;
      float z[8];
      unpack8<false>(d[u], 0, 8, PenCtx{}, z);
      float acc = z[0] >= zmask ? wexp(z[0], chi, clo, negK) : 0.0f;
#pragma unroll
      for (int e = 1; e < 8; ++e) acc += z[e] >= zmask ? wexp(z[e], chi, clo, negK) : 0.0f;
      summ[q] = q * kNT + tid < ngroups ? acc : 0.0f;
    }
  }
}

// One row on the summary path.  Returns false (uniformly across the block)
// when the row must be redone by the general pipeline.
//
// Group j holds ids [8j, 8j+8); thread t owns the groups j = q*kNT + t
// (q < kQ), so each 16-byte load instruction of a wave reads 1 KB of
// contiguous logits and groups are in id order along (q, t).  The pass keeps,
// per owned group, one float in registers: the group weight sum for
// no-filter rows, the group maximum otherwise.  Each thread's weights use its
// own integer reference exponent K_t (from its first group, kept in LDS for
// the others), so sums from different threads rescale exactly by powers of
// two into the frame K* = floor(max * log2(e) / T).
__device__ __forceinline__ bool stream_row(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                           uint32_t path, const Smem& sm, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t V = a.V;
  const int ngroups = (int)(V / 8);
  const char* rowp = (const char*)a.logits + row * a.stride * 2;
  const u32x4* rv = (const u32x4*)rowp;
  path |= ARCS_PATH_RESIDENT;

  const bool greedy = P.temperature == 0.0f || P.top_k == 1;
  const bool kon = P.top_k >= 1 && (int64_t)P.top_k < V;
  const bool pon = P.top_p < 1.0f;
  const bool mon = P.min_p > 0.0f;
  const bool nofilter = !greedy && !kon && !pon && !mon;

  // temperature coefficient c = log2(e) / T = chi + clo, chi rounded down, clo > 0
  float chi = 0.0f, clo = 0.0f;
  if (!greedy) {
    const double c = 1.4426950408889634 / (double)P.temperature;
    chi = (float)c;
    if ((double)chi >= c) chi = key_value(ord_key(chi) - 1u);
    clo = (float)(c - (double)chi);
    if (!(clo > 0.0f)) clo = 1e-30f;
    // temperatures so extreme that z * c leaves the float range: general path
    if (!(c >= 1e-30 && c <= 1e30)) return false;
  }

  // ---- the HBM pass -------------------------------------------------------------
  float best = -__builtin_inff();
  int bq = -1;
  u32x4 bdat = {0u, 0u, 0u, 0u};  // the first group holding this thread's maximum
  float summ[kQ];                 // per owned group: weight sum (no filter) or maximum
  double lsum = 0.0;              // top-p rows: this thread's weight total (frame K_t)
  float negK = 0.0f;              // -K_t
  bool kset = false, bad = false;
#pragma unroll
  for (int it = 0; it < kQ / kU; ++it) {
    if (it * kNT * kU >= ngroups) {
#pragma unroll
      for (int u = 0; u < kU; ++u) summ[it * kU + u] = nofilter ? 0.0f : -__builtin_inff();
      continue;
    }
    // all kU loads are issued before any use (the scheduling barrier keeps
    // the compiler from waiting on one load before issuing the next); groups
    // past the row read group 0 and their results are discarded
    u32x4 d[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = (it * kU + u) * kNT + tid;
      d[u] = __builtin_nontemporal_load(rv + (j < ngroups ? j : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = it * kU + u;
      const bool valid = q * kNT + tid < ngroups;
      const u32x4 dv = d[u];
      float z[8];
      unpack8<false>(dv, 0, 8, PenCtx{}, z);
      float g = max2f(max3f(max3f(z[0], z[1], z[2]), z[3], z[4]), max3f(z[5], z[6], z[7]));
      g = valid ? g : -__builtin_inff();
      const bool up = g > best;
      best = up ? g : best;
      bq = up ? q : bq;
      bdat.x = up ? dv.x : bdat.x; bdat.y = up ? dv.y : bdat.y;
      bdat.z = up ? dv.z : bdat.z; bdat.w = up ? dv.w : bdat.w;
      if (greedy) continue;
      if (!kset && g > -__builtin_inff()) {
        kset = true;
        const float x = g * chi;
        if (x > -1048576.0f && x < 1048576.0f) negK = -__builtin_floorf(x);
        else if (!(g == -__builtin_inff())) bad = true;
      }
      if (nofilter) {
        const float s = group_weight(z, chi, clo, negK);
        summ[q] = valid ? s : 0.0f;
      } else {
        summ[q] = g;
        if (pon) {
          const float s = group_weight(z, chi, clo, negK);
          lsum += valid ? (double)s : 0.0;
        }
      }
    }
  }
  sm.kref[tid] = negK;

  // ---- block maximum and lowest argmax ---------------------------------------
  {
    const float wm = dpp_wave_max_f32(best);
    if (lane == 0) sh.bs.f32[wid] = wm;
    if (tid == 0) sh.u64[0] = (uint64_t)INT64_MAX;
    __syncthreads();
    float m = sh.bs.f32[0];
#pragma unroll
    for (int w = 1; w < kNW; ++w) m = m > sh.bs.f32[w] ? m : sh.bs.f32[w];
    if (m == m && best == m && bq >= 0) {
      float z[8];
      unpack8<false>(bdat, 0, 8, PenCtx{}, z);
      int idx = INT_MAX;
#pragma unroll
      for (int e = 7; e >= 0; --e)
        if (z[e] == m) idx = (bq * kNT + tid) * 8 + e;
      atomicMin((unsigned long long*)&sh.u64[0], (unsigned long long)idx);
    }
    __syncthreads();
    if (tid == 0) {
      sh.f32[0] = m;
      sh.u64[1] = (m == -__builtin_inff()) ? 0ull : sh.u64[0];
    }
    __syncthreads();
  }
  const float m = sh.f32[0];
  const int64_t argmax = (int64_t)sh.u64[1];

  // NaN or +inf present: the general pipeline handles them exactly.
  if (!(m == m) || m == __builtin_inff()) return false;

  if (greedy) {
    path |= ARCS_PATH_GREEDY;
    if (tid == 0) {
      a.out_ids[row] = (int32_t)argmax;
      if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      if (a.stats) {
        arcs_row_stats st = {};
        st.id = (int32_t)argmax; st.argmax = (int32_t)argmax; st.kept = 0; st.cut_index = (int32_t)argmax;
        st.cut_value = m; st.max_logit = m; st.status = 0; st.path = path;
        st.mass_total = 0.0; st.mass_kept = 0.0; st.uniform = -1.0;
        a.stats[row] = st;
      }
    }
    if (a.out_probs)
      for (int64_t i = tid; i < V; i += kNT) a.out_probs[row * V + i] = (i == argmax) ? 1.0f : 0.0f;
    return true;
  }

  // all -inf (every id equally likely) or a maximum too large for the
  // exponent frame: general path
  if (m == -__builtin_inff() || !(m * chi > -1048576.0f && m * chi < 1048576.0f)) return false;
  const float negKs = -__builtin_floorf(m * chi);
  const int dk = (int)(negKs - negK);  // K_t - K*, exact

  // ---- uniform --------------------------------------------------------------------
  double u;
  if (a.uniforms) {
    u = a.uniforms[row];
  } else {
    const uint64_t x = splitmix64_counter_output(a.seed, (uint64_t)row, a.step);
    u = (double)(x >> 11) * 0x1p-53;
  }

  int64_t id = -1;
  int64_t L = V;
  double S = 0.0, S_K = 0.0;
  uint32_t cut_key = 0u;
  int64_t cut_idx = -1;

  if (nofilter) {
    // ---- no filter: per-round totals, then one round's threads, then one group ------
    path |= ARCS_PATH_SORT_SKIP;
    bool bad_any = __syncthreads_or(bad ? 1 : 0) != 0;
    if (bad_any) return false;
    if (!round_draw(summ, rv, -__builtin_inff(), chi, clo, negK, dk, u, sh, id, S)) return false;
    S_K = S;
  } else {
    // ---- filters --------------------------------------------------------------------
    path |= ARCS_PATH_CUTOFF;
    // total mass (top-p only; the other filters need none)
    {
      const double wsum = dpp_wave_sum_f64(__builtin_ldexp(lsum, dk));
      if (lane == 0) sh.f64[wid] = wsum;
      const int bad_any = __syncthreads_or(bad ? 1 : 0);
      double tt = 0.0;
#pragma unroll
      for (int w = 0; w < kNW; ++w) tt += sh.f64[w];
      S = tt;
      if (bad_any || (pon && (!(S > 0.0) || !(S < 1e300)))) {
        __syncthreads();
        return false;
      }
    }
    const double Pm = pon ? (double)P.top_p * S : 0.0;
    // A lower bound on every value the kept set can hold.  min-p: its
    // closed-form threshold m + T ln(min_p), taken a little low here in
    // float arithmetic (the exact threshold is applied to the candidates).
    float zlo = -__builtin_inff();
    if (mon) {
      const float lnmp = __logf(P.min_p);
      const float x = __builtin_fmaf(P.temperature, lnmp, m);
      zlo = x - (1e-5f * (__builtin_fabsf(m) + __builtin_fabsf(P.temperature * lnmp)) + 1e-30f);
    }
    // groups whose maximum reaches zlo
    uint32_t myg = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) myg += summ[q] >= zlo ? 1u : 0u;
    if (tid == 0) {
      sh.cnt2[0] = 0u; sh.cnt2[1] = 0u; sh.mass2[0] = 0.0f; sh.mass2[1] = 0.0f;
      sh.i32[7] = 0;
    }
    __syncthreads();
    {
      const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)dpp_wave_incl_scan_u32(myg), 63);
      if (lane == 0) atomicAdd(&sh.i32[7], (int)wc);
    }
    __syncthreads();
    const uint32_t groups_m = (uint32_t)sh.i32[7];
    // top-k / top-p bounds by bisection over the group maxima (bf16 values,
    // 16-bit order keys): the largest key K with >= k groups whose maximum
    // reaches K (each such maximum is an element), resp. whose maxima weigh
    // at least P (a lower bound of the mass at or above K).  Only needed when
    // the min-p bound leaves too many groups.
    float zkp = -__builtin_inff();
    if ((kon || pon) && (!mon || groups_m > (uint32_t)(kCandCap / 8))) {
      float wq[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) wq[q] = pon ? wexp(summ[q], chi, clo, negKs) : 0.0f;
      const uint32_t k_need = kon ? (uint32_t)P.top_k : 0xFFFFFFFFu;
      const float p_need = pon ? (float)(Pm * (1.0 + 1e-4)) : __builtin_inff();
      // 16-bit order keys of bf16 values: 0x007F is -inf (a bound that always
      // holds), 0xFF80 is +inf, keys outside [0x007F, 0xFF80] are NaNs (for
      // which no maximum compares >=).  Invariant: the predicate holds at lo.
      uint32_t lo_k = 0x7Fu, hi_k = 0x10000u, lo_p = 0x7Fu, hi_p = 0x10000u;
      for (int step = 0; step < 17; ++step) {
        const uint32_t mid_k = (lo_k + hi_k) >> 1, mid_p = (lo_p + hi_p) >> 1;
        const float tk = key_value(mid_k << 16 | ((mid_k & 0x8000u) ? 0u : 0xFFFFu));
        const float tp = key_value(mid_p << 16 | ((mid_p & 0x8000u) ? 0u : 0xFFFFu));
        uint32_t c = 0;
        float ms = 0.0f;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          c += summ[q] >= tk ? 1u : 0u;
          ms += summ[q] >= tp ? wq[q] : 0.0f;
        }
        const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)dpp_wave_incl_scan_u32(c), 63);
        const float wmass = dpp_wave_sum_f32(ms);
        const int slot = step & 1;
        if (lane == 0) { atomicAdd(&sh.cnt2[slot], wc); atomicAdd(&sh.mass2[slot], wmass); }
        __syncthreads();
        const uint32_t tc = sh.cnt2[slot];
        const float tm = sh.mass2[slot];
        __syncthreads();
        if (tid == 0) { sh.cnt2[slot] = 0u; sh.mass2[slot] = 0.0f; }
        if (tc >= k_need) lo_k = mid_k; else hi_k = mid_k;
        if (tm >= p_need) lo_p = mid_p; else hi_p = mid_p;
        if (hi_k - lo_k <= 1 && hi_p - lo_p <= 1) break;
      }
      const float bk = kon ? key_value(lo_k << 16 | ((lo_k & 0x8000u) ? 0u : 0xFFFFu)) : -__builtin_inff();
      const float bp = pon ? key_value(lo_p << 16 | ((lo_p & 0x8000u) ? 0u : 0xFFFFu)) : -__builtin_inff();
      zkp = bk > bp ? bk : bp;
    }
    const float zc = zlo > zkp ? zlo : zkp;  // candidates: z >= zc
    // min-p alone with many groups above its bound: the kept set is
    // {z >= zt}, drawn from in id order without any ordering by value
    const bool minp_stream = mon && !kon && !pon && groups_m > (uint32_t)(kCandCap / 8);
    // list the groups to re-read
    if (tid == 0) sh.i32[0] = 0;
    __syncthreads();
    if (!minp_stream) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (summ[q] >= zc && summ[q] > -__builtin_inff()) {
          const int slot = atomicAdd(&sh.i32[0], 1);
          if (slot < kGroupCap) sm.glist[slot] = q * kNT + tid;
        }
      }
    }
    // the exact min-p threshold: the smallest float z with
    // ((double)z - m) / T >= ln(min_p), computed by one thread meanwhile
    if (tid == 0) {
      float zt = -__builtin_inff();
      if (mon) {
        const double lnmp = log((double)P.min_p), T = (double)P.temperature, md = (double)m;
        auto keep = [&](float z) { return ((double)z - md) / T >= lnmp; };
        zt = (float)(md + T * lnmp);
        if (zt < -FLT_MAX) zt = -FLT_MAX;
        if (keep(zt)) {
          for (int i = 0; i < 64; ++i) {
            const float dn = key_value(ord_key(zt) - 1u);
            if (!keep(dn)) break;
            zt = dn;
          }
        } else {
          for (int i = 0; i < 64 && !keep(zt); ++i) zt = key_value(ord_key(zt) + 1u);
        }
        if (zt > m) zt = m;
      }
      sh.f32[1] = zt;
      sh.i32[3] = 0;
      sh.i32[6] = 0;
    }
    __syncthreads();
    const int ng = sh.i32[0];
    const float zt = sh.f32[1];
    if (minp_stream) {
      path |= ARCS_PATH_MINP_FLOOR;
      masked_group_sums(rv, ngroups, zt, chi, clo, negK, summ);
      if (!round_draw(summ, rv, zt, chi, clo, negK, dk, u, sh, id, S_K)) return false;
      L = -1;  // counted by the debug outputs
      cut_key = ord_key(zt);
      cut_idx = INT64_MAX;
    } else {
    if (ng > kGroupCap) return false;
    // re-read the listed groups, one per thread, and gather the candidates
    const float zcut = zt > zc ? zt : zc;
    for (int i = tid; i < ng; i += kNT) {
      const int j = sm.glist[i];
      const float nk = sm.kref[j % kNT];
      const int dkj = (int)(negKs - nk);
      float z[8];
      unpack8<false>(rv[j], 0, 8, PenCtx{}, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (z[e] >= zcut && z[e] > -__builtin_inff()) {
          const int slot = atomicAdd(&sh.i32[3], 1);
          if (slot < kCandCap) {
            sm.ckey[slot] = cand_key(z[e], (int64_t)j * 8 + e);
            sm.cw[slot] = __builtin_ldexpf(wexp(z[e], chi, clo, nk), dkj);
          }
        }
      }
    }
    __syncthreads();
    const int nc = sh.i32[3];
    if (nc > kCandCap || nc == 0) {
      __syncthreads();
      return false;
    }
    // the candidate set is {z >= zcut}, a prefix of the order
    // (value desc, id asc); the min-p set lies inside it when zcut == zt
    const bool minp_complete = mon && !(zkp > zt);
    if (minp_complete) path |= ARCS_PATH_MINP_FLOOR;

    constexpr int64_t INF = INT64_MAX;
    if (nc <= kSmallSort) {
      // ---- small candidate set: wave 0 ranks every candidate against all others ----
      if (wid == 0) {
        // rank by (value desc, id asc) = ascending key
        if (lane < nc) {
          const uint64_t myk = sm.ckey[lane];
          int r = 0;
          for (int i = 0; i < nc; ++i) r += sm.ckey[i] < myk ? 1 : 0;
          sm.skey[r] = myk;
          sm.sw[r] = sm.cw[lane];
        }
        wave_lds_sync();
        // in-order fp64 prefix of the sorted weights (lane i sums entries 0..i)
        double cum = 0.0;
        uint64_t key = ~0ull;
        float w = 0.0f;
        if (lane < nc) {
          key = sm.skey[lane];
          w = sm.sw[lane];
          for (int i = 0; i <= lane; ++i) cum += (double)sm.sw[i];
        }
        const int64_t Lk = (kon && (int64_t)P.top_k <= nc) ? (int64_t)P.top_k : INF;
        int64_t Lp = INF;
        if (pon) {
          const uint64_t hit = __ballot(lane < nc && cum >= Pm);
          if (hit) Lp = __builtin_ctzll(hit) + 1;
        }
        const int64_t Lm = minp_complete ? (int64_t)nc : INF;
        int64_t Lw = Lk < Lp ? Lk : Lp;
        Lw = Lw < Lm ? Lw : Lm;
        if (Lw == INF) {
          if (lane == 0) sh.i32[6] = -1;
        } else {
          const double sk = __shfl(cum, (int)Lw - 1, kWave);
          const uint64_t ck = __shfl(key, (int)Lw - 1, kWave);
          const double t = u * sk;
          // the kept entries in id order: rank by id among the first Lw
          const uint32_t myid = (uint32_t)(key & 0xFFFFFFFFull);
          double c2 = 0.0;
          bool mine = false;
          if (lane < Lw) {
            for (int i = 0; i < Lw; ++i) {
              const uint32_t oid = (uint32_t)(sm.skey[i] & 0xFFFFFFFFull);
              if (oid <= myid) c2 += (double)sm.sw[i];
            }
            mine = w > 0.0f && c2 > t && c2 - (double)w <= t;
          }
          const uint64_t hit = __ballot(mine);
          const uint64_t nz = __ballot(lane < Lw && w > 0.0f);
          // rounding can leave t past the last boundary: take the largest kept id with weight
          int ls;
          if (hit) {
            ls = __builtin_ctzll(hit);
          } else {
            uint32_t bestid = 0u;
            int bl = 0;
            for (int i = 0; i < (int)Lw; ++i) {
              const uint32_t oid = (uint32_t)(sm.skey[i] & 0xFFFFFFFFull);
              if (sm.sw[i] > 0.0f && oid >= bestid) { bestid = oid; bl = i; }
            }
            ls = nz ? bl : 0;
          }
          const uint64_t pid = __shfl(key, ls, kWave);
          if (lane == 0) {
            sh.u64[10] = pid & 0xFFFFFFFFull;
            sh.u64[11] = (uint64_t)Lw;
            sh.f64[kNW + 1] = sk;
            sh.u64[12] = ck;
          }
        }
      }
      __syncthreads();
    } else {
      // ---- larger candidate set: block bitonic sort in LDS ------------------------
      int n2 = 128;
      while (n2 < nc) n2 <<= 1;
      for (int i = nc + tid; i < n2; i += kNT) { sm.ckey[i] = ~0ull; sm.cw[i] = 0.0f; }
      if (tid == 0) { sh.u64[13] = (uint64_t)INF; sh.u64[14] = (uint64_t)INF; }
      __syncthreads();
      block_bitonic_sort(sm.ckey, sm.cw, n2);
      // prefix mass over the sorted order (ENT consecutive entries per thread)
      constexpr int ENT = kCandCap / kNT;
      double loc[ENT];
      double lsum_c = 0.0;
#pragma unroll
      for (int j = 0; j < ENT; ++j) {
        const int i = tid * ENT + j;
        lsum_c += (i < nc) ? (double)sm.cw[i] : 0.0;
        loc[j] = lsum_c;
      }
      double tot;
      const double incl = block_scan_f64(lsum_c, sh, tot);
      const double excl = incl - lsum_c;
      if (pon) {
#pragma unroll
        for (int j = 0; j < ENT; ++j) {
          const int i = tid * ENT + j;
          if (i < nc && excl + loc[j] >= Pm) {
            atomicMin((unsigned long long*)&sh.u64[13], (unsigned long long)(i + 1));
            break;
          }
        }
      }
      __syncthreads();
      const int64_t Lk = (kon && (int64_t)P.top_k <= nc) ? (int64_t)P.top_k : INF;
      const int64_t Lp = (int64_t)sh.u64[13];
      const int64_t Lm = minp_complete ? (int64_t)nc : INF;
      int64_t Lw = Lk < Lp ? Lk : Lp;
      Lw = Lw < Lm ? Lw : Lm;
      if (Lw == INF) {
        if (tid == 0) sh.i32[6] = -1;
        __syncthreads();
      } else {
#pragma unroll
        for (int j = 0; j < ENT; ++j) {
          const int i = tid * ENT + j;
          if (i == Lw - 1) { sh.f64[kNW + 1] = excl + loc[j]; sh.u64[12] = sm.ckey[i]; }
        }
        __syncthreads();
        const double sk = sh.f64[kNW + 1];
        const double t = u * sk;
        // keep the first Lw entries, re-sorted by id
        int m2 = 2;
        while (m2 < Lw) m2 <<= 1;
        for (int i = tid; i < n2; i += kNT) {
          if (i < Lw) sm.ckey[i] &= 0xFFFFFFFFull;
          else { sm.ckey[i] = ~0ull; sm.cw[i] = 0.0f; }
        }
        __syncthreads();
        block_bitonic_sort(sm.ckey, sm.cw, m2);
        double ls2 = 0.0;
#pragma unroll
        for (int j = 0; j < ENT; ++j) {
          const int i = tid * ENT + j;
          ls2 += (i < Lw) ? (double)sm.cw[i] : 0.0;
          loc[j] = ls2;
        }
        double tot2;
        const double incl2 = block_scan_f64(ls2, sh, tot2);
        const double excl2 = incl2 - ls2;
#pragma unroll
        for (int j = 0; j < ENT; ++j) {
          const int i = tid * ENT + j;
          if (i < Lw && sm.cw[i] > 0.0f && excl2 + loc[j] > t) {
            atomicMin((unsigned long long*)&sh.u64[14], (unsigned long long)i);
            break;
          }
        }
        __syncthreads();
        if (tid == 0) {
          int64_t pos = (int64_t)sh.u64[14];
          if (pos == INF) {  // rounding left t at the very end: the last kept id with weight
            pos = Lw - 1;
            while (pos > 0 && !(sm.cw[pos] > 0.0f)) --pos;
          }
          sh.u64[10] = sm.ckey[pos] & 0xFFFFFFFFull;
          sh.u64[11] = (uint64_t)Lw;
        }
        __syncthreads();
      }
    }
    if (sh.i32[6] < 0) {
      __syncthreads();
      return false;
    }
    id = (int64_t)sh.u64[10];
    L = (int64_t)sh.u64[11];
    S_K = sh.f64[kNW + 1];
    const uint64_t ck = sh.u64[12];
    cut_key = ~(uint32_t)(ck >> 32);
    cut_idx = (int64_t)(ck & 0xFFFFFFFFull);
    }
  }

  if (tid == 0) {
    a.out_ids[row] = (int32_t)id;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
  }

  // ---- debug outputs (the row is read again) ---------------------------------------
  if (a.stats || a.out_probs) {
    const bool all_kept = (path & ARCS_PATH_SORT_SKIP) != 0;
    uint32_t kmin = 0xFFFFFFFFu;
    int64_t kmin_idx = -1;
    uint32_t nkept = 0;
    double wtot = 0.0;
    for (int j = tid; j < ngroups; j += kNT) {
      const float nk = sm.kref[j % kNT];
      const int dkj = (int)(negKs - nk);
      float z[8];
      unpack8<false>(rv[j], 0, 8, PenCtx{}, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t idx = (int64_t)j * 8 + e;
        const uint32_t k = ord_key(z[e]);
        const bool kept = all_kept || k > cut_key || (k == cut_key && idx <= cut_idx);
        if (a.out_probs) {
          const double w = (double)__builtin_ldexpf(wexp(z[e], chi, clo, nk), dkj);
          a.out_probs[row * V + idx] = kept ? (float)(w / S_K) : 0.0f;
        }
        if (kept && (k < kmin || (k == kmin && idx > kmin_idx))) { kmin = k; kmin_idx = idx; }
        nkept += kept ? 1u : 0u;
        wtot += (double)__builtin_ldexpf(wexp(z[e], chi, clo, nk), dkj);
      }
    }
    if (a.stats) {
      if (tid == 0) sh.u64[9] = ~0ull;
      __syncthreads();
      const uint64_t packed =
          ((uint64_t)kmin << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(kmin_idx < 0 ? 0 : kmin_idx));
      if (kmin_idx >= 0) atomicMin((unsigned long long*)&sh.u64[9], (unsigned long long)packed);
      const uint32_t wk = (uint32_t)__builtin_amdgcn_readlane((int)dpp_wave_incl_scan_u32(nkept), 63);
      const double wt = dpp_wave_sum_f64(wtot);
      if (lane == 0) {
        sh.qt[wid] = wt;
        sh.qt[kNW + wid] = (double)wk;
      }
      __syncthreads();
      if (L < 0 || S == 0.0) {
        double a0 = 0.0, a1 = 0.0;
        for (int w = 0; w < kNW; ++w) { a0 += sh.qt[w]; a1 += sh.qt[kNW + w]; }
        if (L < 0) L = (int64_t)a1;
        if (S == 0.0) S = a0;
      }
      if (tid == 0) {
        const uint64_t pk = sh.u64[9];
        // masses reported relative to the row max, as sums of exp((z - m) / T)
        const double to_m = exp2((double)(-negKs) - (double)m * ((double)chi + (double)clo));
        arcs_row_stats st = {};
        st.id = (int32_t)id; st.argmax = (int32_t)argmax; st.kept = (int32_t)L;
        st.cut_index = (int32_t)(0xFFFFFFFFu - (uint32_t)(pk & 0xFFFFFFFFu));
        st.cut_value = key_value((uint32_t)(pk >> 32));
        st.max_logit = m; st.status = 0; st.path = path;
        st.mass_total = S * to_m;
        st.mass_kept = S_K * to_m;
        st.uniform = u;
        a.stats[row] = st;
      }
    }
  }
  return true;
}

template <bool PEN>
__global__ __launch_bounds__(kNT) void sample_summary_kernel(SampleArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const Smem sm = carve_smem(smem_raw, kUnionSummary, a.bitmap_words);
  arcs_row_params P;
  PenCtx pc;
  uint32_t path;
  if (!row_prologue<true, PEN>(a, row, sm, sh, P, pc, path)) return;
  // Rows with active penalties take the general pipeline; the summary path
  // handles the rest.
  if (pc.on || !stream_row(a, row, P, path, sm, sh)) {
    __syncthreads();
    generic_row<true, true>(a, row, P, pc, path, sm, sh);
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <class Kern>
hipError_t launch_one(Kern kernel, bool summary, const SampleArgs& a, int64_t B, size_t lds, hipStream_t stream,
                      std::atomic<int>& attr_done) {
  if (!attr_done.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sample_lds_bytes(summary, true, summary ? kSummaryMaxV : kMaxPenVocab));
    if (e != hipSuccess) return e;
    attr_done.store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)B), dim3(kNT), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream) {
  const bool pen = a.pen_tables != 0;
  static std::atomic<int> done[10];
  if (dtype == ARCS_DTYPE_BF16 && vec && a.V <= kSummaryMaxV && a.V % 8 == 0) {
    const size_t lds = sample_lds_bytes(true, pen, a.V);
    return pen ? launch_one(sample_summary_kernel<true>, true, a, B, lds, stream, done[0])
               : launch_one(sample_summary_kernel<false>, true, a, B, lds, stream, done[1]);
  }
  const size_t lds = sample_lds_bytes(false, pen, a.V);
  if (dtype == ARCS_DTYPE_BF16) {
    if (vec)
      return pen ? launch_one(sample_kernel<true, true, true>, false, a, B, lds, stream, done[2])
                 : launch_one(sample_kernel<true, true, false>, false, a, B, lds, stream, done[3]);
    return pen ? launch_one(sample_kernel<true, false, true>, false, a, B, lds, stream, done[4])
               : launch_one(sample_kernel<true, false, false>, false, a, B, lds, stream, done[5]);
  }
  if (vec)
    return pen ? launch_one(sample_kernel<false, true, true>, false, a, B, lds, stream, done[6])
               : launch_one(sample_kernel<false, true, false>, false, a, B, lds, stream, done[7]);
  return pen ? launch_one(sample_kernel<false, false, true>, false, a, B, lds, stream, done[8])
             : launch_one(sample_kernel<false, false, false>, false, a, B, lds, stream, done[9]);
}

}  // namespace arcs
