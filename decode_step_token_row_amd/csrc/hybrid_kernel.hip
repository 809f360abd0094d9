// Baseline nucleus (top-p) selector: the hybrid the pages report for their
// device sampler (Arc PR #194, squashed commit #130, "hybrid nucleus
// selector"), written for gfx950 so that it can be timed against
// arcs_sample on the same rows.  Per row, at temperature T and top_p:
//   z = bf16 logits widened (NaN -> -inf), m = max z, w = exp((z - m) / T),
//   S = sum of w, target = top_p * S;
//   enumeration: the ids in the order (value desc, id asc) are taken one at
//     a time while the running mass stays under the target, for at most
//     `budget` ids; if the target is reached the kept set is that prefix;
//   otherwise threshold bisection: 32 halvings of the 32-bit value key find
//     the largest key theta whose mass of {key >= theta} reaches the target,
//     and the kept set is every id with key >= theta (ties at the boundary
//     value all kept: the pages' "wider" behaviour);
//   draw: the first kept id, in id order, whose running weight exceeds u * S_K,
//     u the SplitMix64 uniform of (seed, row, step) as in arcs_sample.
// top_p >= 1 keeps every id.  The budget changes only which algorithm finds
// the set, and the set only through the tie rule.
//
// One 512-thread workgroup per row, the row in registers (32 rounds of one
// 16-byte group of 8 values per thread, as the sampling kernel holds it).
// The enumeration keeps each thread's largest key not yet taken; a step is a
// block maximum over those, and only the thread that gave up its key scans
// its 256 values again.  Each bisection step is a full pass over the
// registers (a weight per value) and a block sum.  Weights are fp32
// (exp2 of an fp32 argument), sums fp64.
#include "device_common.hpp"
#include "launch.hpp"

namespace arcs {

constexpr int kHyNT = 512;
constexpr int kHyNW = kHyNT / kWave;
constexpr int kHyQ = 32;  // rounds: V <= 8 * kHyQ * kHyNT = 131072

struct HybridShared {
  uint64_t wkey[kHyNW];
  double wsum[kHyNW];
  uint32_t wcnt[kHyNW];
  double rt[kHyQ * kHyNW];  // draw: each wave's kept mass per round
};

__device__ __forceinline__ uint64_t hy_key(float z, uint32_t id) {
  return ((uint64_t)ord_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ void hy_unpack(u32x4 d, float (&z)[8]) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[2 * i] = canon_nan(bf16_lo(w[i]));
    z[2 * i + 1] = canon_nan(bf16_hi(w[i]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = z[e] == 0.0f ? 0.0f : z[e];  // -0 -> +0
}

// Round q's 16 bytes through an opaque copy: every pass widens its own copy,
// so the compiler cannot keep all 256 widened values live across passes.
__device__ __forceinline__ u32x4 hy_round(const u32x4 (&d)[kHyQ], int q) {
  u32x4 v = d[q];
  asm volatile("" : "+v"(v));
  return v;
}

// Round qs (known only at run time) by a static scan of the registers: an
// indexed read would move the whole array to scratch memory.
__device__ __forceinline__ u32x4 hy_select(const u32x4 (&d)[kHyQ], int qs) {
  u32x4 v = d[0];
#pragma unroll
  for (int q = 1; q < kHyQ; ++q) {
    v.x = q == qs ? d[q].x : v.x; v.y = q == qs ? d[q].y : v.y;
    v.z = q == qs ? d[q].z : v.z; v.w = q == qs ? d[q].w : v.w;
  }
  return v;
}

__device__ __forceinline__ float hy_weight(float z, float m, float c) {
  return z == m ? 1.0f : __builtin_amdgcn_exp2f((z - m) * c);
}

__device__ __forceinline__ uint64_t hy_wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t t = __shfl_xor(v, o);
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ double hy_block_sum(double v, HybridShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const double ws = dpp_wave_sum_f64(v);
  if (lane == 0) sh.wsum[wid] = ws;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kHyNW; ++w) s += sh.wsum[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ uint64_t hy_block_max_u64(uint64_t v, HybridShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint64_t wm = hy_wave_max_u64(v);
  if (lane == 0) sh.wkey[wid] = wm;
  __syncthreads();
  uint64_t m = 0;
#pragma unroll
  for (int w = 0; w < kHyNW; ++w) m = sh.wkey[w] > m ? sh.wkey[w] : m;
  __syncthreads();
  return m;
}

// The thread's largest key below `below` (0 if none).
__device__ __forceinline__ uint64_t hy_local_next(const u32x4 (&d)[kHyQ], int ngroups, uint64_t below) {
  // opaque: the ids of the thread's 256 values are formed here on every
  // call, not hoisted out of the caller's loop (256 live registers)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  uint64_t best = 0;
#pragma unroll
  for (int q = 0; q < kHyQ; ++q) {
    const int g = q * kHyNT + tid;
    if (g < ngroups) {
      float z[8];
      hy_unpack(hy_round(d, q), z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint64_t k = hy_key(z[e], (uint32_t)(g * 8 + e));
        best = (k < below && k > best) ? k : best;
      }
    }
  }
  return best;
}

__global__ __launch_bounds__(kHyNT) void hybrid_nucleus_kernel(HybridArgs a) {
  __shared__ HybridShared sh;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int ngroups = (int)(a.V / 8);
  const float T = a.temperature[row];
  const float top_p = a.top_p[row];
  int status = ARCS_ROW_OK;
  if (!(T > 0.0f) || !(T < __builtin_inff())) status = ARCS_ROW_BAD_TEMPERATURE;
  else if (!(top_p > 0.0f)) status = ARCS_ROW_BAD_TOP_P;
  if (status != ARCS_ROW_OK) {
    if (tid == 0) {
      a.out_ids[row] = -1;
      if (a.out_kept) a.out_kept[row] = 0;
      if (a.out_status) a.out_status[row] = status;
    }
    return;
  }
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  u32x4 d[kHyQ];
#pragma unroll
  for (int q = 0; q < kHyQ; ++q) {
    const int g = q * kHyNT + tid;
    d[q] = g < ngroups ? rv[g] : u32x4{0u, 0u, 0u, 0u};
  }
  // the maximum and the mass
  float tm = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < kHyQ; ++q) {
    if (q * kHyNT + tid < ngroups) {
      float z[8];
      hy_unpack(hy_round(d, q), z);
#pragma unroll
      for (int e = 0; e < 8; ++e) tm = z[e] > tm ? z[e] : tm;
    }
  }
  const float wm = dpp_wave_max_f32(tm);
  if (lane == 0) sh.wsum[wid] = (double)wm;
  __syncthreads();
  float m = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kHyNW; ++w) m = (float)sh.wsum[w] > m ? (float)sh.wsum[w] : m;
  __syncthreads();
  const float c = (float)(1.4426950408889634 / (double)T);
  double part = 0.0;
#pragma unroll
  for (int q = 0; q < kHyQ; ++q) {
    if (q * kHyNT + tid < ngroups) {
      float z[8];
      hy_unpack(hy_round(d, q), z);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += hy_weight(z[e], m, c);
      part += (double)s;
    }
  }
  const double S = hy_block_sum(part, sh);
  const double target = (double)top_p * S;
  const bool all = !(top_p < 1.0f);

  // enumeration, at most `budget` ids
  bool wide = false;
  uint64_t kcut = 0;      // strict: keys >= kcut kept
  uint32_t theta = 0u;    // wide: value keys >= theta kept
  int64_t L = 0;
  if (all) {
    kcut = 0;
    L = a.V;
  } else {
    uint64_t mine = hy_local_next(d, ngroups, ~0ull);
    double cum = 0.0;
    bool done = false;
    for (int it = 0; it < a.budget; ++it) {
      const uint64_t k = hy_block_max_u64(mine, sh);
      if (k == 0) break;  // (no key left: cannot happen before the mass is reached)
      if (mine == k) mine = hy_local_next(d, ngroups, k);  // this thread gave up its key
      const float z = key_value((uint32_t)(k >> 32));
      cum += (double)hy_weight(z, m, c);
      ++L;
      kcut = k;
      if (cum >= target) { done = true; break; }
    }
    if (!done) {
      // threshold bisection over the value key: the largest theta whose mass
      // of {key >= theta} reaches the target
      wide = true;
      uint32_t lo = 0u, hi = 0xFFFFFFFFu;
      for (int it = 0; it < 32; ++it) {
        const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) / 2);
        double pm = 0.0;
#pragma unroll
        for (int q = 0; q < kHyQ; ++q) {
          if (q * kHyNT + tid < ngroups) {
            float z[8];
            hy_unpack(hy_round(d, q), z);
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s += ord_key(z[e]) >= mid ? hy_weight(z[e], m, c) : 0.0f;
            pm += (double)s;
          }
        }
        const double mass = hy_block_sum(pm, sh);
        if (mass >= target) lo = mid;
        else hi = mid - 1u;
      }
      theta = lo;
    }
  }

  // the draw in id order over the kept set: each wave's kept mass per round,
  // then the round, the wave, the lane and the element
  uint32_t cnt = 0;
  auto kept = [&](float z, uint32_t id) {
    return all || (wide ? ord_key(z) >= theta : hy_key(z, id) >= kcut);
  };
#pragma unroll
  for (int q = 0; q < kHyQ; ++q) {
    const int g = q * kHyNT + tid;
    double s = 0.0;
    if (g < ngroups) {
      float z[8];
      hy_unpack(hy_round(d, q), z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool k = kept(z[e], (uint32_t)(g * 8 + e));
        s += k ? (double)hy_weight(z[e], m, c) : 0.0;
        cnt += k ? 1u : 0u;
      }
    }
    const double incl = dpp_wave_incl_scan_f64(s);
    if (lane == kWave - 1) sh.rt[q * kHyNW + wid] = incl;
  }
  const uint32_t wc = dpp_wave_sum_u32(cnt);
  if (lane == 0) sh.wcnt[wid] = wc;
  __syncthreads();
  if (wide) {
    L = 0;
#pragma unroll
    for (int w = 0; w < kHyNW; ++w) L += sh.wcnt[w];
  }
  const uint64_t x = splitmix64_counter_output(a.seed, (uint64_t)row, a.step);
  const double u = (double)(x >> 11) * 0x1p-53;
  // every wave: the total, the round and the wave (same sums, same order)
  double SK = 0.0;
  for (int i = 0; i < kHyQ * kHyNW; ++i) SK += sh.rt[i];
  const double t = u * SK;
  double cum = 0.0, base = 0.0, base_last = 0.0;
  int sel = -1, last = 0;
  for (int i = 0; i < kHyQ * kHyNW; ++i) {
    const double r = sh.rt[i];
    if (r > 0.0) {
      if (sel < 0 && cum + r > t) { sel = i; base = cum; }
      last = i;
      base_last = cum;
    }
    cum += r;
  }
  if (sel < 0) { sel = last; base = base_last; }  // rounding: the last with weight
  const int qs = sel / kHyNW, ws = sel % kHyNW;
  if (wid == ws) {
    const int g = qs * kHyNT + tid;
    float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    double w8[8];
    double s = 0.0;
    if (g < ngroups) hy_unpack(hy_select(d, qs), z);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w8[e] = (g < ngroups && kept(z[e], (uint32_t)(g * 8 + e))) ? (double)hy_weight(z[e], m, c) : 0.0;
      s += w8[e];
    }
    const double incl = dpp_wave_incl_scan_f64(s);
    const uint64_t hit = __ballot(s > 0.0 && base + incl > t);
    const uint64_t nz = __ballot(s > 0.0);
    const int ls = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
    if (lane == ls) {
      double acc = base + (incl - s);
      int pe = -1, le = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc += w8[e];
        if (w8[e] > 0.0) {
          if (pe < 0 && acc > t) pe = e;
          le = e;
        }
      }
      if (pe < 0) pe = le;
      a.out_ids[row] = g * 8 + pe;
      if (a.out_kept) a.out_kept[row] = (int32_t)L;
      if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
    }
  }
}

hipError_t launch_hybrid_nucleus(const HybridArgs& a, int64_t B, hipStream_t stream) {
  hipLaunchKernelGGL(hybrid_nucleus_kernel, dim3((unsigned)B), dim3(kHyNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace arcs
