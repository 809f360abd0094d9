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
// sample_summary_kernel (bf16 rows, 16-byte aligned, V <= 131072, V % 8 == 0):
//   the row is read from HBM exactly once, all 16 loads of 16 bytes per lane
//   issued before any is used.  Each thread turns every group of 8 logits
//   (penalised through LDS tables when the row has active penalties) into
//   its maximum and, for rows without filters or with top-p, its weight
//   exp2(z*log2(e)/T - K_t) (K_t an integer reference exponent of the thread,
//   so moving sums between frames is an exact power of two), and leaves one
//   float per group in LDS: the weight sum for rows without filters, the
//   maximum for the others.  After the pass, per-wave records and one wave
//   give the row's maximum, mass and min-p threshold, and then:
//     greedy rows   -> the lowest index of the maximum, from registers;
//     no filter     -> an id-order draw over the group sums;
//     any filter    -> a bound below which nothing is kept (the min-p
//                      threshold, or a histogram of the threads' largest
//                      group maxima for top-k / top-p), the elements above it
//                      gathered into LDS as candidates (mostly from
//                      registers), the cut L = min(L_k, L_p, L_m) found by one
//                      wave for small sets or by a radix select for large
//                      ones, and the inverse-CDF draw in id order.
//   Rows the fast path cannot take exactly (signalling NaN, +inf, extreme
//   values or temperatures, more than kCandCap candidates) run the general
//   pipeline in the same workgroup.
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
  if (a.deferred_only && a.out_ids[row] != kDeferredId) return;
  const Smem sm = carve_smem(smem_raw, false, a.bitmap_words);
  arcs_row_params P = a.params[row];
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

// 8 bf16 of a group -> float32.
__device__ __forceinline__ void unpack8(u32x4 d, float (&z)[8]) {
  z[0] = bf16_lo(d.x); z[1] = bf16_hi(d.x);
  z[2] = bf16_lo(d.y); z[3] = bf16_hi(d.y);
  z[4] = bf16_lo(d.z); z[5] = bf16_hi(d.z);
  z[6] = bf16_lo(d.w); z[7] = bf16_hi(d.w);
}


// The history ids among the 8 elements of the group at g0 (a multiple of 8)
// are penalised from their own logit and their occurrence count in the LDS
// tables: one pass of the loop per history id in the group (groups without
// one cost a bitmap read), rather than a branch per element.  The operations
// are those of the general path's table (the same binary32 sequence).
__device__ __forceinline__ void penalize8(float (&z)[8], int64_t g0, const PenCtx& pc) {
  const uint32_t w = (uint32_t)(g0 >> 5), s5 = (uint32_t)(g0 & 31);
  const uint32_t word = pc.bitmap[w];
  uint32_t bits = (word >> s5) & 0xFFu;
  if (!bits) return;
  uint32_t r = (uint32_t)pc.wprefix[w] + (uint32_t)__builtin_popcount(word & ((1u << s5) - 1u));
  do {
    const int e = __builtin_ctz(bits);
    bits &= bits - 1u;
    const uint32_t cnt = pc.pcount[r++];
    float ze = z[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) ze = e == k ? z[k] : ze;
    const float pz = penalize(canon_nan(ze), cnt, pc);
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = e == k ? pz : z[k];
  } while (bits);
}

// The values z' of group j (elements 8j .. 8j + 7) from its 16 bytes: the
// bf16 widened, then, on rows with active penalties, the history ids among
// them replaced by their penalised logits from the LDS tables.
template <bool PEN>
__device__ __forceinline__ void load_z8(u32x4 d, int j, const PenCtx& pc, float (&z)[8]) {
  unpack8(d, z);
  if (PEN && pc.on) penalize8(z, (int64_t)j * 8, pc);
}

// Maximum of a group.  v_max ignores quiet NaNs (the same as treating them
// as -inf); a signalling NaN makes the result NaN, which the caller checks.
__device__ __forceinline__ float group_max(const float (&z)[8]) {
  return max2f(max3f(max3f(z[0], z[1], z[2]), z[3], z[4]), max3f(z[5], z[6], z[7]));
}

// Weight of z relative to the integer reference K in log2 units:
// exp2(z*c - K) with c = chi + clo (chi rounded down, clo > 0, so -inf
// logits give exactly 0).
__device__ __forceinline__ float wexp(float z, float chi, float clo, float negK) {
  const float t = __builtin_fmaf(z, clo, __builtin_fmaf(z, chi, negK));
  return __builtin_amdgcn_exp2f(t);
}

// Weight of a group: its 8 weights summed in id order.  The draw repeats
// exactly these operations inside the group it lands in.
__device__ __forceinline__ float group_weight(const float (&z)[8], float chi, float clo, float negK) {
  float s = wexp(z[0], chi, clo, negK);
#pragma unroll
  for (int e = 1; e < 8; ++e) s += wexp(z[e], chi, clo, negK);
  return s;
}

// A value the same in every lane, moved to scalar registers.
__device__ __forceinline__ float uniform_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ double uniform_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Orders one wave's LDS stores before its later LDS loads from other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sort key of a candidate: ascending order = value descending, id ascending.
__device__ __forceinline__ uint64_t cand_key(float z, int64_t idx) {
  return ((uint64_t)(~ord_key(z)) << 32) | (uint64_t)(uint32_t)idx;
}

// ---------------------------------------------------------------------------
// summary kernel
// ---------------------------------------------------------------------------
constexpr int kQ = kMaxGroups / kNT;  // groups per thread (16)

// The row's groups owned by this thread: group j = q * kNT + tid holds ids
// [8j, 8j + 8), so one load instruction of a wave reads 1 KB of contiguous
// logits.  Each round q goes through a buffer resource that covers only the
// rest of the row, so lanes past the row's end read zeros without touching
// memory (their results are discarded), and the only per-lane address is
// tid * 16.  All kQ loads are issued before any of them is used.
__device__ __forceinline__ void issue_row_loads(const u32x4* rv, int ngroups, u32x4 (&d)[kQ]) {
  const int voff = threadIdx.x * 16;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int left = (ngroups - q * kNT) * 16;  // bytes of the row from round q on
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rv + (left > 0 ? q * kNT : 0)), (short)0, left > 0 ? left : 0, 0x00020000);
    d[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2 /* nt */));
  }
  __builtin_amdgcn_sched_barrier(0);
}


// The min-p threshold: the smallest float z with (z - m) >= T ln(min_p) in
// double arithmetic (tdl = T ln(min_p)).  The 64 lanes of the wave test 64
// consecutive floats around m + tdl at once; the same value is returned in
// every lane.  ok = false if the boundary was not found (never expected).
__device__ __forceinline__ float minp_threshold(float m, double tdl, bool& ok) {
  const int lane = threadIdx.x & (kWave - 1);
  const double md = (double)m;
  const double e = md + tdl;
  const float z0 = e < -(double)FLT_MAX ? -FLT_MAX : (float)e;
  // keys below that of -FLT_MAX are NaNs, for which the test is false
  const uint32_t k0 = ord_key(z0) - 32u;
  const float zl = key_value(k0 + (uint32_t)lane);
  const uint64_t b = __ballot(((double)zl - md) >= tdl);
  ok = b != 0 && (b & 1ull) == 0;
  const float zt = key_value(k0 + (uint32_t)(ok ? __builtin_ctzll(b) : 32));
  return zt < m ? zt : m;
}

// What a row does after the pass (decided by wave 0, broadcast through LDS).
enum RowMode : int32_t {
  kModeFallback = 0,  // the general pipeline
  kModeGreedy = 1,    // argmax
  kModeNoFilter = 2,  // id-order draw over all weights
  kModeMinpStream = 3,  // id-order draw over the weights at or above the min-p threshold
  kModeCand = 4,      // candidates above a known bound
  kModeHist = 5       // candidates above a bound from a histogram of thread maxima
};

// Which entries a draw keeps: order key above th, or equal to it with an id
// at most istar.
struct KeepCut {
  uint32_t th;
  int64_t istar;
};
__device__ __forceinline__ bool keep_cut(float z, int64_t idx, const KeepCut& c) {
  const uint32_t k = ord_key(z);
  return k > c.th || (k == c.th && idx <= c.istar);
}

// Inverse-CDF draw in id order over sm.tsum (group j's weight at j).  With
// `thread_frames`, group j's value is in the frame 2^-K_t of the thread t
// that owns it (kref[t] = -K_t); otherwise in the row frame K*.
// Wave w takes the groups w*kNT .. w*kNT + kNT - 1, its lane l the 16
// consecutive groups from w*kNT + 16l (all owned by wave l/4): the round
// totals locate the wave, a wave scan the lane, the lane's 16 sums the group,
// and one re-read of that group the element (entries `cut` drops weigh 0).
// The drawing lane writes the output row.  Returns false (uniformly) when
// the total weight is zero or not finite; else S (the total).  With `sync`
// the id is left in sh.u64[10] for the whole block; otherwise waves other
// than the drawing one return at once.
template <bool PEN>
__device__ __forceinline__ bool tsum_draw(const SampleArgs& a, int64_t row, const u32x4* rv, const PenCtx& pc,
                                          const Smem& sm, Shared& sh, bool thread_frames, KeepCut cut, float chi,
                                          float clo, float negks, double u, bool sync, double& S) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  // lane l: groups wid*kNT + 16l + i, owned by threads 16l + i
  double v[16];
  const float4* src = (const float4*)(sm.tsum + wid * kNT + lane * 16);
  const float4* kr = (const float4*)(sm.kref + lane * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = src[i];
    float4 k = {negks, negks, negks, negks};
    if (thread_frames) k = kr[i];
    v[4 * i] = __builtin_ldexp((double)f.x, (int)(negks - k.x));
    v[4 * i + 1] = __builtin_ldexp((double)f.y, (int)(negks - k.y));
    v[4 * i + 2] = __builtin_ldexp((double)f.z, (int)(negks - k.z));
    v[4 * i + 3] = __builtin_ldexp((double)f.w, (int)(negks - k.w));
  }
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) part += v[i];
  const double incl = dpp_wave_incl_scan_f64(part);
  if (lane == kWave - 1) sh.rtot[wid] = incl;
  __syncthreads();
  // every thread: the total, in wave order, and the wave the target lies in
  double cum = 0.0, before = 0.0, before_last = 0.0;
  int qs = -1, qlast = 0;
  S = 0.0;
  for (int w = 0; w < kNW; ++w) S += sh.rtot[w];
  if (!(S > 0.0) || !(S < 1e300)) return false;
  const double t = u * S;
  for (int w = 0; w < kNW; ++w) {
    const double r = sh.rtot[w];
    if (r > 0.0) {
      if (qs < 0 && cum + r > t) { qs = w; before = cum; }
      qlast = w;
      before_last = cum;
    }
    cum += r;
  }
  if (qs < 0) { qs = qlast; before = before_last; }  // rounding: the last wave with weight
  if (wid == qs) {
    const uint64_t hit = __ballot(part > 0.0 && before + incl > t);
    const uint64_t nz = __ballot(part > 0.0);
    const int ls = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(nz);
    if (lane == ls) {
      double bl = before + (incl - part), bsel = 0.0, blast = 0.0;
      int is = -1, ilast = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double w = v[i];
        if (v[i] > 0.0) {
          if (is < 0 && bl + w > t) { is = i; bsel = bl; }
          ilast = i;
          blast = bl;
        }
        bl += w;
      }
      if (is < 0) { is = ilast; bsel = blast; }
      const int owner = lane * 16 + is;  // the thread that owns the group
      const int j = wid * kNT + owner;
      // the group's weights as the owner computed them: the running sum
      // ends at exactly the group's value
      const float nk = thread_frames ? sm.kref[owner] : negks;
      const int dsh = (int)(negks - nk);
      float z[8];
      load_z8<PEN>(rv[j], j, pc, z);
      float acc = 0.0f, prev = 0.0f;
      int pe = -1, last_e = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = keep_cut(z[e], (int64_t)j * 8 + e, cut) ? wexp(z[e], chi, clo, nk) : 0.0f;
        acc = (e == 0) ? w : acc + w;
        const bool pos = acc > prev;
        if (pos) last_e = e;
        if (pe < 0 && pos && bsel + __builtin_ldexp((double)acc, dsh) > t) pe = e;
        prev = acc;
      }
      if (pe < 0) pe = last_e;
      const int32_t id = j * 8 + pe;
      a.out_ids[row] = id;
      if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      sh.u64[10] = (uint64_t)id;
    }
  }
  if (sync) __syncthreads();
  return true;
}


// Gathers this thread's elements z >= bound (bound finite) into the candidate
// list sm.ckey / sm.cw with their weights in the row frame (-negks): the two
// largest groups from registers (counted first, one wave scan, one LDS atomic
// per wave on the block count sh.i32[3]), any other group at or above the
// bound re-read from memory (rare).  A count above kCandCap means the list is
// incomplete.  Threads whose largest group lies below the bound hold nothing,
// and a wave where that holds for every lane does nothing.
template <bool PEN>
__device__ __forceinline__ void gather_candidates(const u32x4* rv, const PenCtx& pc, const Smem& sm, Shared& sh,
                                                  float bound, float best, int bq, float best2, int sq, u32x4 da,
                                                  u32x4 db, float chi, float clo, float negks) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const bool pa = bq >= 0 && best >= bound;
  const bool pb = sq >= 0 && best2 >= bound;
  if (!__ballot(pa)) return;
  float za[8], zb[8];
  unpack8(da, za);
  unpack8(db, zb);
  if (PEN && pc.on) {
    if (pa) penalize8(za, (int64_t)(bq * kNT + tid) * 8, pc);
    if (pb) penalize8(zb, (int64_t)(sq * kNT + tid) * 8, pc);
  }
  uint32_t n = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    n += pa && za[e] >= bound ? 1u : 0u;
    n += pb && zb[e] >= bound ? 1u : 0u;
  }
  if (__ballot(n != 0)) {
    const uint32_t incl = dpp_wave_incl_scan_u32(n);
    uint32_t base = 0;
    if (lane == kWave - 1) base = (uint32_t)atomicAdd(&sh.i32[3], (int)incl);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
    uint32_t pos = base + incl - n;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 0 ? pa : pb) {
        const int64_t i0 = (int64_t)((h == 0 ? bq : sq) * kNT + tid) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = h == 0 ? za[e] : zb[e];
          if (z >= bound) {
            if (pos < (uint32_t)kCandCap) {
              sm.ckey[pos] = cand_key(z, i0 + e);
              sm.cw[pos] = wexp(z, chi, clo, negks);
            }
            ++pos;
          }
        }
      }
    }
  }
  // other groups at or above the bound (only where the second largest is): re-read
  if (!__ballot(pb)) return;
  uint32_t xmask = 0;
  if (pb) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) xmask |= (q != bq && q != sq && sm.tsum[q * kNT + tid] >= bound) ? (1u << q) : 0u;
  }
  if (!__ballot(xmask != 0)) return;
  // all of them in flight at once; each round's entries placed with one LDS
  // atomic per wave
  u32x4 xd[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    if ((xmask >> q) & 1u) xd[q] = rv[q * kNT + tid];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const bool mine = (xmask >> q) & 1u;
    if (!__ballot(mine)) continue;
    const int j = q * kNT + tid;
    float zx[8];
    uint32_t m8 = 0;
    if (mine) {
      load_z8<PEN>(xd[q], j, pc, zx);
#pragma unroll
      for (int e = 0; e < 8; ++e) m8 |= zx[e] >= bound ? (1u << e) : 0u;
    }
    const uint32_t nq = (uint32_t)__builtin_popcount(m8);
    const uint32_t qincl = dpp_wave_incl_scan_u32(nq);
    uint32_t qbase = 0;
    if (lane == kWave - 1) qbase = (uint32_t)atomicAdd(&sh.i32[3], (int)qincl);
    qbase = (uint32_t)__builtin_amdgcn_readlane((int)qbase, kWave - 1);
    uint32_t slot = qbase + qincl - nq;
    while (m8) {
      const int e = __builtin_ctz(m8);
      m8 &= m8 - 1u;
      if (slot < (uint32_t)kCandCap) {
        sm.ckey[slot] = cand_key(zx[e], (int64_t)j * 8 + e);
        sm.cw[slot] = wexp(zx[e], chi, clo, negks);
      }
      ++slot;
    }
  }
}

// Cut and draw over nc <= kSmallSort candidates, by one wave (lane i holds
// candidate i: its key and its weight in the row frame): rank by key with lane reads, an fp64 scan of
// the weights in (value desc, id asc) order for L = min(L_k, L_p, L_m), then a
// rank by id among the kept prefix and a second scan for the id-order draw.
// Writes the output row and sh.u64[10..12] / sh.f64[kNW+1] (id, L, cut key,
// S_K).  Returns 1 when drawn, 0 when no prefix length is known from the
// candidates, 2 (nothing written) when `lazy_cap` > 0 and the kept mass
// reaches it.
__device__ __forceinline__ int small_cut_draw(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh, int nc,
                                               uint64_t key, float w, bool kon, int top_k, bool pon, double Pm,
                                               bool minp_complete, float zt, double u,
                                              double lazy_cap) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int64_t INF = INT64_MAX;
  const bool in = lane < nc;
  key = in ? key : ~0ull;
  w = in ? w : 0.0f;
  // rank by (value desc, id asc) = ascending key
  const uint32_t khi = (uint32_t)(key >> 32), klo = (uint32_t)key;
  uint32_t r = 0;
  for (int j = 0; j < nc; ++j) {
    const uint32_t oh = (uint32_t)__builtin_amdgcn_readlane((int)khi, j);
    const uint32_t ol = (uint32_t)__builtin_amdgcn_readlane((int)klo, j);
    r += (oh < khi || (oh == khi && ol < klo)) ? 1u : 0u;
  }
  wave_lds_sync();
  if (in) { sm.skey[r] = key; sm.sw[r] = w; }
  wave_lds_sync();
  const uint64_t skey = in ? sm.skey[lane] : ~0ull;
  const float sw = in ? sm.sw[lane] : 0.0f;
  const double cum = dpp_wave_incl_scan_f64((double)sw);
  const int64_t Lk = (kon && (int64_t)top_k <= nc) ? (int64_t)top_k : INF;
  int64_t Lp = INF;
  if (pon) {
    const uint64_t hit = __ballot(in && cum >= Pm);
    if (hit) Lp = __builtin_ctzll(hit) + 1;
  }
  int64_t Lm = INF;
  if (minp_complete) Lm = __builtin_popcountll(__ballot(in && key_value(~(uint32_t)(skey >> 32)) >= zt));
  int64_t Lw = Lk < Lp ? Lk : Lp;
  Lw = Lw < Lm ? Lw : Lm;
  if (Lw == INF || Lw < 1) return 0;
  const int lc = (int)Lw - 1;
  const uint64_t cb = __builtin_bit_cast(uint64_t, cum);
  const double sk = __builtin_bit_cast(
      double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(cb >> 32), lc) << 32) |
                  (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)cb, lc));
  // top-p left out while the row's mass is only bounded below: the cut
  // stands when the kept mass stays under top_p times that bound
  if (lazy_cap > 0.0 && !(sk < lazy_cap)) return 2;
  const uint64_t ck = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(skey >> 32), lc) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)skey, lc);
  const double t = u * sk;
  // the kept entries in id order: rank by id, then an in-order scan
  const bool kept = lane < Lw;
  const uint32_t myid = (uint32_t)skey;
  uint32_t r2 = 0;
  for (int j = 0; j < (int)Lw; ++j) r2 += (uint32_t)__builtin_amdgcn_readlane((int)myid, j) < myid ? 1u : 0u;
  wave_lds_sync();
  if (kept) { sm.skey[r2] = myid; sm.sw[r2] = sw; }
  wave_lds_sync();
  const uint32_t id2 = kept ? (uint32_t)sm.skey[lane] : 0u;
  const float w2 = kept ? sm.sw[lane] : 0.0f;
  const double c2 = dpp_wave_incl_scan_f64((double)w2);
  const uint64_t hit = __ballot(kept && w2 > 0.0f && c2 > t);
  const uint64_t nz = __ballot(kept && w2 > 0.0f);
  // rounding can leave t past the last boundary: the last kept id with weight
  const int ls = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
  const uint32_t pid = (uint32_t)__builtin_amdgcn_readlane((int)id2, ls);
  if (lane == 0) {
    sh.u64[10] = pid;
    sh.u64[11] = (uint64_t)Lw;
    sh.f64[kNW + 1] = sk;
    sh.u64[12] = ck;
    a.out_ids[row] = (int32_t)pid;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
  }
  return 1;
}

// Cut over nc > kSmallSort candidates (keys and row-frame weights in LDS, in
// no particular order) without sorting them.  A radix descent over the value
// order keys, 8 bits a level from the highest bit in which the candidates'
// keys differ down to bit `lowbit` (16 when every value is a widened bf16,
// whose low 16 key bits follow from its sign; 0 otherwise), with per-digit
// counts and 2^-50 fixed-point masses, finds the value theta of the L-th
// entry in (value desc, id asc) order, L = min(L_k, L_p, L_m), and the count
// and mass above it.  How many ties at theta are kept follows in closed
// form (they weigh the same); when not all are, a descent over their ids
// (9 + 8 bits; ids < 2^17) finds the last kept one.  The bins live at
// sm.hcnt / sm.hmass (inside the group area, free at this point).  Returns
// false (uniformly) when the candidates reach no target; kept_mass is the
// kept entries' weight (from the 2^-50 fixed-point sums; masses are tracked
// when `track_mass`, which top-p needs).
constexpr double kFixScale = 1125899906842624.0;  // 2^50: weights < 2, at most 4096 of them
__device__ __forceinline__ uint64_t to_fix50(float w) { return (uint64_t)((double)w * kFixScale); }

template <int NT = kNT>
__device__ __forceinline__ bool large_cut_select(const Smem& sm, Shared& sh, int nc, int lowbit, bool kon, int top_k,
                                                 bool pon, double Pm, bool minp_complete, float zt, KeepCut& cut,
                                                 int64_t& L, double& kept_mass,
                                                 bool track_mass) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  constexpr int ENT = kCandCap / NT;
  uint32_t* hc = sm.hcnt;
  uint64_t* hm = sm.hmass;
  constexpr uint64_t NONE = ~0ull;
  for (int i = tid; i < 512; i += NT) { hc[i] = 0u; hm[i] = 0ull; }
  if (tid == 0) { sh.u64[13] = 0ull; sh.u64[14] = 0ull; sh.i32[1] = INT_MIN; sh.i32[2] = INT_MAX; }
  __syncthreads();
  // the span of the value keys: min and max (as int atomics on flipped keys)
  {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int r = 0; r < ENT; ++r) {
      const int i = tid + r * NT;
      if (i < nc) {
        const uint32_t vk = ~(uint32_t)(sm.ckey[i] >> 32);
        kmin = vk < kmin ? vk : kmin;
        kmax = vk > kmax ? vk : kmax;
      }
    }
    kmin = dpp_wave_min_u32(kmin);
    kmax = ~dpp_wave_min_u32(~kmax);
    if (lane == 0) {
      atomicMax(&sh.i32[1], (int)(kmax ^ 0x80000000u));
      atomicMin(&sh.i32[2], (int)(kmin ^ 0x80000000u));
    }
  }
  // the min-p count, with the first level
  if (minp_complete) {
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < ENT; ++r) {
      const int i = tid + r * NT;
      if (i < nc && key_value(~(uint32_t)(sm.ckey[i] >> 32)) >= zt) ++c;
    }
    const uint32_t wc = dpp_wave_sum_u32(c);
    if (lane == 0 && wc) atomicAdd((unsigned long long*)&sh.u64[13], (unsigned long long)wc);
  }
  uint64_t Pfix = NONE;
  if (pon) {
    const double x = Pm * kFixScale;
    Pfix = x < 9.0e18 ? (uint64_t)__builtin_ceil(x) : NONE;
  }
  uint64_t cnt_above = 0, mass_above = 0, c_eq = nc, m_eq = 0;
  __syncthreads();
  const uint32_t vmax = (uint32_t)sh.i32[1] ^ 0x80000000u, vmin = (uint32_t)sh.i32[2] ^ 0x80000000u;
  const uint32_t span = vmin ^ vmax;
  const int hb = span ? 31 - __builtin_clz(span) : -1;  // the highest differing bit
  uint32_t pref = hb >= 0 ? (hb == 31 ? 0u : vmin & ~((2u << hb) - 1u)) : vmin;  // the common bits
  for (int top = hb; top >= lowbit; top -= 8) {
    const int shf = top - 7 > lowbit ? top - 7 : lowbit;
    const uint32_t dmask = (1u << (top - shf + 1)) - 1u;
#pragma unroll
    for (int r = 0; r < ENT; ++r) {
      const int i = tid + r * NT;
      if (i < nc) {
        const uint32_t vk = ~(uint32_t)(sm.ckey[i] >> 32);
        if (top == 31 || (vk >> (top + 1)) == (pref >> (top + 1))) {
          const uint32_t d = (vk >> shf) & dmask;
          atomicAdd(&hc[d], 1u);
          if (track_mass) atomicAdd((unsigned long long*)&hm[d], (unsigned long long)to_fix50(sm.cw[i]));
        }
      }
    }
    __syncthreads();
    if (wid == 0) {
      uint64_t Lc = (kon && top_k <= nc) ? (uint64_t)top_k : NONE;
      if (minp_complete) Lc = sh.u64[13] < Lc ? sh.u64[13] : Lc;
      const uint64_t need_c = Lc == NONE ? NONE : Lc - cnt_above;
      const uint64_t need_m = Pfix == NONE ? NONE : Pfix - mass_above;
      // lane l: digits 255 - 4l .. 252 - 4l, from the top
      uint32_t c[4];
      uint64_t m[4];
      uint64_t ctot = 0, mtot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 255 - 4 * lane - j;
        c[j] = hc[d]; m[j] = hm[d];
        hc[d] = 0u; hm[d] = 0ull;
        ctot += c[j]; mtot += m[j];
      }
      uint64_t cc = wave_incl_scan_u64(ctot, lane) - ctot;
      uint64_t mc = wave_incl_scan_u64(mtot, lane) - mtot;
      int fj = 4;
      uint64_t cb = 0, mb = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (fj == 4 && (cc + c[j] >= need_c || mc + m[j] >= need_m)) { fj = j; cb = cc; mb = mc; }
        cc += c[j]; mc += m[j];
      }
      const uint64_t hit = __ballot(fj < 4);
      if (hit == 0) {
        if (lane == 0) sh.i32[0] = -1;
      } else if (lane == __builtin_ctzll(hit)) {
        sh.i32[0] = 255 - 4 * lane - fj;
        sh.u64[3] = cb; sh.u64[4] = mb; sh.u64[5] = c[fj]; sh.u64[6] = m[fj];
      }
    }
    __syncthreads();
    const int dstar = sh.i32[0];
    if (dstar < 0) return false;  // only at the first level: the candidates reach no target
    cnt_above += sh.u64[3];
    mass_above += sh.u64[4];
    c_eq = sh.u64[5];
    m_eq = sh.u64[6];
    pref |= (uint32_t)dstar << shf;
    __syncthreads();
  }
  if (hb < lowbit) {
    // every candidate holds the same value: all of them are ties at it
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < ENT; ++r) {
      const int i = tid + r * NT;
      if (i < nc) m += to_fix50(sm.cw[i]);
    }
    m = wave_sum_u64(m);
    if (lane == 0) atomicAdd((unsigned long long*)&sh.u64[14], (unsigned long long)m);
    __syncthreads();
    m_eq = sh.u64[14];
    uint64_t Lc0 = (kon && top_k <= nc) ? (uint64_t)top_k : NONE;
    if (minp_complete) Lc0 = sh.u64[13] < Lc0 ? sh.u64[13] : Lc0;
    if (Lc0 == NONE && (Pfix == NONE || m_eq < Pfix)) return false;
  }
  const uint32_t th = lowbit == 16 ? ((pref & 0xFFFF0000u) | ((pref & 0x80000000u) ? 0u : 0xFFFFu)) : pref;
  // ties at theta kept: r of c_eq
  uint64_t Lc = (kon && top_k <= nc) ? (uint64_t)top_k : NONE;
  if (minp_complete) Lc = sh.u64[13] < Lc ? sh.u64[13] : Lc;
  uint64_t r = c_eq;
  if (Lc != NONE && Lc - cnt_above < r) r = Lc - cnt_above;
  if (Pfix != NONE) {
    const uint64_t w_eq = c_eq ? m_eq / c_eq : 0;
    if (w_eq > 0) {
      const uint64_t need = Pfix > mass_above ? Pfix - mass_above : 0;
      uint64_t rp = (need + w_eq - 1) / w_eq;
      rp = rp < 1 ? 1 : rp;
      r = rp < r ? rp : r;
    }
  }
  L = (int64_t)(cnt_above + r);
  kept_mass = (double)(mass_above + r * (c_eq ? m_eq / c_eq : 0)) / kFixScale;
  cut.th = th;
  cut.istar = INT64_MAX;
  if (r < c_eq && c_eq <= (uint64_t)kSmallSort) {
    // few ties: their ids listed in LDS, ranked by one wave
    if (tid == 0) sh.i32[4] = 0;
    __syncthreads();
    uint32_t* ids = (uint32_t*)sm.skey;
#pragma unroll
    for (int q = 0; q < ENT; ++q) {
      const int i = tid + q * NT;
      if (i < nc) {
        const uint64_t k = sm.ckey[i];
        if (~(uint32_t)(k >> 32) == th) {
          const int slot = atomicAdd(&sh.i32[4], 1);
          if (slot < kSmallSort) ids[slot] = (uint32_t)k;
        }
      }
    }
    __syncthreads();
    if (wid == 0) {
      const int n = (int)c_eq;
      const uint32_t my = lane < n ? ids[lane] : 0xFFFFFFFFu;
      uint32_t rank = 0;
      for (int j = 0; j < n; ++j) rank += (uint32_t)__builtin_amdgcn_readlane((int)my, j) < my ? 1u : 0u;
      if (lane < n && rank == (uint32_t)(r - 1)) sh.u64[3] = my;
    }
    __syncthreads();
    cut.istar = (int64_t)sh.u64[3];
  } else if (r < c_eq) {
    // the r-th smallest id among the ties: ids >> 8 (512 bins), then the low 8 bits
    int64_t hi_d = 0;
    uint64_t before = 0;
    for (int lev = 0; lev < 2; ++lev) {
#pragma unroll
      for (int q = 0; q < ENT; ++q) {
        const int i = tid + q * NT;
        if (i < nc) {
          const uint64_t k = sm.ckey[i];
          const uint32_t id = (uint32_t)k;
          if (~(uint32_t)(k >> 32) == th && (lev == 0 || (int64_t)(id >> 8) == hi_d))
            atomicAdd(&hc[lev == 0 ? (id >> 8) : (id & 255u)], 1u);
        }
      }
      __syncthreads();
      if (wid == 0) {
        const int nb = lev == 0 ? 512 : 256, per = nb / kWave;
        uint32_t tot = 0;
        for (int j = 0; j < per; ++j) tot += hc[lane * per + j];
        uint64_t cc = wave_incl_scan_u64(tot, lane) - tot;
        const uint64_t need = r - before;
        int dd = -1;
        uint64_t cb = 0;
        for (int j = 0; j < per; ++j) {
          const uint32_t x = hc[lane * per + j];
          if (dd < 0 && cc + x >= need) { dd = lane * per + j; cb = cc; }
          cc += x;
        }
        for (int j = 0; j < per; ++j) hc[lane * per + j] = 0u;
        const uint64_t hit = __ballot(dd >= 0);
        if (hit != 0 && lane == __builtin_ctzll(hit)) { sh.i32[0] = dd; sh.u64[3] = cb; }
      }
      __syncthreads();
      if (lev == 0) { hi_d = sh.i32[0]; before += sh.u64[3]; }
      else cut.istar = (hi_d << 8) | (int64_t)sh.i32[0];
      __syncthreads();
    }
  }
  return true;
}

// Inverse-CDF draw in id order over the kept candidates (those `cut` keeps),
// from the candidate list alone: weights in 2^-50 fixed point, summed per
// bucket of 256 ids with LDS atomics (exact, so independent of their order),
// one wave scan locates the bucket of t = floor(u * S_K), a second the group
// of 8 ids inside it, and thread 0 walks that group's kept candidates in id
// order.  Writes the output row, sh.u64[10] (id) and sh.f64[kNW + 1] (S_K in
// the row frame).  Returns false (uniformly) when the kept mass is zero.
__device__ __forceinline__ bool cand_draw(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh, int nc,
                                          const KeepCut& cut, uint64_t uf) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  constexpr int ENT = kCandCap / kNT;
  uint64_t* hm = sm.hmass;
  for (int i = tid; i < 512; i += kNT) hm[i] = 0ull;
  if (tid == 0) sh.i32[4] = 0;
  __syncthreads();
  uint32_t myid[ENT];
  uint64_t myw[ENT];
#pragma unroll
  for (int q = 0; q < ENT; ++q) {
    const int i = tid + q * kNT;
    myw[q] = 0ull;
    myid[q] = 0xFFFFFFFFu;
    if (i < nc) {
      const uint64_t k = sm.ckey[i];
      const uint32_t id = (uint32_t)k;
      if (keep_cut(key_value(~(uint32_t)(k >> 32)), (int64_t)id, cut)) {
        myid[q] = id;
        myw[q] = to_fix50(sm.cw[i]);
        if (myw[q]) atomicAdd((unsigned long long*)&hm[id >> 8], (unsigned long long)myw[q]);
      }
    }
  }
  __syncthreads();
  // the bucket: lane l sums buckets 8l .. 8l + 7
  if (wid == 0) {
    uint64_t b[8], tot = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) { b[j] = hm[8 * lane + j]; tot += b[j]; }
    const uint64_t incl = wave_incl_scan_u64(tot, lane);
    const uint64_t SK = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, kWave - 1) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(incl >> 32), kWave - 1) << 32);
    const uint64_t t = __umul64hi(uf, SK);  // floor(u * S_K) < S_K
    uint64_t c = incl - tot;
    int bj = -1;
    uint64_t before = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (bj < 0 && c + b[j] > t) { bj = j; before = c; }
      c += b[j];
    }
    const uint64_t hit = __ballot(bj >= 0);
    if (lane == 0) { sh.u64[7] = SK; sh.u64[8] = t; sh.i32[5] = -1; }
    if (hit != 0 && lane == __builtin_ctzll(hit)) { sh.i32[5] = 8 * lane + bj; sh.u64[9] = before; }
    // the groups of the next step use hm[0 .. 31]
    if (lane < 32) hm[lane] = 0ull;
  }
  __syncthreads();
  const int bstar = sh.i32[5];
  if (bstar < 0) return false;  // no kept mass
  const uint64_t t = sh.u64[8];
#pragma unroll
  for (int q = 0; q < ENT; ++q)
    if (myw[q] && (int)(myid[q] >> 8) == bstar) atomicAdd((unsigned long long*)&hm[(myid[q] >> 3) & 31u], (unsigned long long)myw[q]);
  __syncthreads();
  if (wid == 0) {
    const uint64_t g = lane < 32 ? hm[lane] : 0ull;
    const uint64_t incl = wave_incl_scan_u64(g, lane) + sh.u64[9];
    const uint64_t hit = __ballot(lane < 32 && incl > t);
    if (lane == 0) sh.i32[7] = hit ? __builtin_ctzll(hit) : 31;
    if (hit != 0 && lane == __builtin_ctzll(hit)) sh.u64[9] = incl - g;
  }
  __syncthreads();
  const uint32_t gstar = ((uint32_t)bstar << 5) | (uint32_t)sh.i32[7];
  uint64_t* lst = sm.skey;  // ids in 0..7, weights in 8..15
#pragma unroll
  for (int q = 0; q < ENT; ++q) {
    if (myw[q] && (myid[q] >> 3) == gstar) {
      const int slot = atomicAdd(&sh.i32[4], 1);
      if (slot < 8) { lst[slot] = myid[q]; lst[8 + slot] = myw[q]; }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int n = sh.i32[4] < 8 ? sh.i32[4] : 8;
    uint64_t acc = sh.u64[9];
    uint32_t pid = 0xFFFFFFFFu, last = 0xFFFFFFFFu;
    // the group's kept entries in id order (at most 8)
    for (int r = 0; r < n; ++r) {
      uint32_t best = 0xFFFFFFFFu;
      int bi = -1;
      for (int i = 0; i < n; ++i) {
        const uint32_t id = (uint32_t)lst[i];
        if (id < best && (r == 0 || id > last)) { best = id; bi = i; }
      }
      last = best;
      acc += lst[8 + bi];
      if (pid == 0xFFFFFFFFu && acc > t) pid = best;
    }
    if (pid == 0xFFFFFFFFu) pid = last;  // not reached with exact sums
    a.out_ids[row] = (int32_t)pid;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
    sh.u64[10] = pid;
    sh.f64[kNW + 1] = (double)sh.u64[7] / kFixScale;
  }
  return true;
}

// The row's exact total weight in the row frame (-negks): the row read
// again (from cache), every element weighed; fp64 per thread, one wave sum
// and one LDS sum.  All threads call it; uniform result.
template <bool PEN>
__device__ __forceinline__ double exact_row_mass(const u32x4* rv, const PenCtx& pc, int ngroups, float chi,
                                                 float clo, float negks, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  u32x4 dd[kQ];
  issue_row_loads(rv, ngroups, dd);
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    // the round's bound is formed here, not hoisted out of the unrolled
    // loop: sixteen live lane masks would crowd out the scalar registers
    int lim = ngroups - q * kNT;
    asm volatile("" : "+s"(lim));
    const bool valid = tid < lim;
    float z[8];
    unpack8(dd[q], z);
    if (PEN && pc.on && valid) penalize8(z, (int64_t)(q * kNT + tid) * 8, pc);
    s += valid ? (double)group_weight(z, chi, clo, negks) : 0.0;
  }
  s = dpp_wave_sum_f64(s);
  __syncthreads();
  if (lane == 0) sh.rtot[wid] = s;
  __syncthreads();
  double S = 0.0;
  for (int w = 0; w < kNW; ++w) S += sh.rtot[w];
  return S;
}

// One row on the summary path.  d holds the loads of the row's groups,
// issued by the caller.  Returns false (uniformly across the block) when the
// row must be redone by the general pipeline.
//
// The pass keeps per owned group one float: its weight sum for no-filter
// rows, its maximum otherwise, and notes each thread's two largest groups,
// whose 16 bytes stay in registers for the candidate gathering.  Weights are
// computed in a per-thread frame 2^-K_t (K_t an integer from the thread's
// first finite group, raised when a later group lies far above it), moved
// after the pass to the frame of the wave and then of the row,
// K* = floor(max * log2(e) / T), by exact powers of two.  One barrier
// collects per-wave records; wave 0 turns them into the row's maximum,
// argmax, total weight and min-p threshold and picks what follows (a second
// barrier):
//   no filter    -> the group sums go through LDS to the id-order draw;
//   min-p rows, small rows, or a top-k / top-p bound from a histogram of the
//                   threads' largest group maxima -> the elements above the
//                   bound are gathered into LDS, cut by one wave (at most 64
//                   of them) or by a radix select, and drawn from in id order;
//   min-p alone over more than the list holds -> masked group sums and the
//                   id-order draw.
// What the row's uniform is made from, read at the start of the kernel with
// the parameter record (before the row's loads, so that using it does not
// wait for them): the override of the debug entry point, or the RNG key (by
// value, or from device memory for the keyed entry point).
struct RowRng {
  uint64_t seed, step;
  double u_override;
  bool override_on;
};

__device__ __forceinline__ RowRng load_row_rng(const SampleArgs& a, int64_t row) {
  RowRng r;
  r.override_on = a.uniforms != nullptr;
  r.u_override = r.override_on ? a.uniforms[row] : 0.0;
  r.seed = a.key ? a.key[0] : a.seed;
  r.step = a.key ? a.key[1] : a.step;
  return r;
}

template <bool PEN>
__device__ __forceinline__ bool stream_row(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                           const RowRng& rng, const PenCtx& pc, uint32_t path, const Smem& sm,
                                           Shared& sh, const u32x4 (&d)[kQ]) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t V = a.V;
  const int ngroups = (int)(V / 8);
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  const bool debug = a.stats != nullptr || a.out_probs != nullptr;
  path |= ARCS_PATH_RESIDENT;

  const bool greedy = P.temperature == 0.0f || P.top_k == 1;
  const bool nofilter = !greedy && !(P.top_k >= 1 && (int64_t)P.top_k < V) && !(P.top_p < 1.0f) && !(P.min_p > 0.0f);
  const bool kon = !greedy && P.top_k >= 1 && (int64_t)P.top_k < V;
  const bool pon = !greedy && P.top_p < 1.0f;
  const bool mon = !greedy && P.min_p > 0.0f;
  const bool weights = nofilter || pon;  // weights needed during the pass
  // top-p with top-k: the pass weighs only each group's maximum, which bounds
  // the row's mass from below; a top-k prefix whose mass stays under top_p
  // times that bound is not cut by top-p, and only when it is not is the
  // exact mass computed (a second read of the row).  A prefix of at most k
  // tokens rarely reaches top_p of the mass; a min-p set without top-k holds
  // most of it on exactly the peaked rows where top-p cuts, so those rows
  // weigh every element in the pass.  The penalised kernel always weighs every
  // element: there the second-read code measured slower than what it saves.
  bool lazy = !PEN && pon && kon;

  // temperature coefficient c = log2(e) / T = chi + clo, chi rounded down, clo > 0
  float chi = 0.0f, clo = 0.0f;
  double tdl = 0.0;  // T ln(min_p)
  if (!greedy) {
    const double c = 1.4426950408889634 / (double)P.temperature;
    // temperatures so extreme that z * c leaves the float range: general path
    if (!(c >= 1e-30 && c <= 1e30)) return false;
    chi = (float)c;
    if ((double)chi >= c) chi = key_value(ord_key(chi) - 1u);
    clo = (float)(c - (double)chi);
    if (!(clo > 0.0f)) clo = 1e-30f;
    chi = uniform_f32(chi);
    clo = uniform_f32(clo);
    if (mon) tdl = uniform_f64((double)P.temperature * log((double)P.min_p));
  }

  // the row's uniform, while the loads are in flight
  double u = 0.0;
  if (!greedy) {
    if (rng.override_on) {
      u = rng.u_override;
    } else {
      const uint64_t x = splitmix64_counter_output(rng.seed, (uint64_t)row, rng.step);
      u = (double)(x >> 11) * 0x1p-53;
    }
    u = uniform_f64(u);
  }

  // ---- the pass over the row (loads already in flight) ----------------------------
  float best = -__builtin_inff();
  // the thread's two largest groups (not for no-filter rows): maxima, rounds
  // and data, kept branch-free in registers and stored to LDS after the pass
  float best2 = -__builtin_inff();
  int bq = -1, sq = -1;
  const bool track = !nofilter;
  double lsum = 0.0;             // top-p rows: this thread's weight total (frame K_t)
  float kfr = -__builtin_inff();  // K_t; -inf until the thread's first finite group
  float negk = 0.0f;             // -K_t (0 before the first finite group: weights are 0 there)
  bool bad = false, special = false;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    // the round's bound is formed here, not hoisted out of the unrolled
    // loop: sixteen live lane masks would crowd out the scalar registers
    int lim = ngroups - q * kNT;
    asm volatile("" : "+s"(lim));
    const bool valid = tid < lim;
    float z[8];
    unpack8(d[q], z);
    if (PEN && pc.on && valid) penalize8(z, (int64_t)(q * kNT + tid) * 8, pc);
    float g = group_max(z);
    special = special || !(g == g);
    g = valid && g == g ? g : -__builtin_inff();
    if (track) {
      const bool up1 = g > best;
      const bool up2 = !up1 && g > best2;
      best2 = up1 ? best : (up2 ? g : best2);
      sq = up1 ? bq : (up2 ? q : sq);
      bq = up1 ? q : bq;
    }
    best = max2f(best, g);
    // filter rows: the group maximum; no-filter rows: the group weight (below)
    if ((!greedy && !nofilter)) sm.tsum[q * kNT + tid] = g;
    if (!weights) continue;
    const float x = g * chi;
    if (x > kfr + 64.0f) {
      // the first finite group, or one far above the frame: (re)set it
      if (!(x > -1048576.0f && x < 1048576.0f)) bad = true;
      const float nk = __builtin_floorf(x);
      if (kfr > -__builtin_inff()) {
        const int sh_ = (int)(kfr - nk);
        lsum = __builtin_ldexp(lsum, sh_);
        if (nofilter) {
          for (int p = 0; p < q; ++p) sm.tsum[p * kNT + tid] = __builtin_ldexpf(sm.tsum[p * kNT + tid], sh_);
        }
      }
      kfr = nk;
      negk = -nk;
    }
    const float s = lazy ? wexp(g, chi, clo, negk) : group_weight(z, chi, clo, negk);
    if (nofilter) sm.tsum[q * kNT + tid] = valid ? s : 0.0f;
    else lsum += valid ? (double)s : 0.0;
  }

  u32x4 bdat = d[0], sdat = d[0];
  if (track) {
    // the data of the two largest groups, by a static scan of the registers
#pragma unroll
    for (int q = 1; q < kQ; ++q) {
      bdat.x = q == bq ? d[q].x : bdat.x; bdat.y = q == bq ? d[q].y : bdat.y;
      bdat.z = q == bq ? d[q].z : bdat.z; bdat.w = q == bq ? d[q].w : bdat.w;
      sdat.x = q == sq ? d[q].x : sdat.x; sdat.y = q == sq ? d[q].y : sdat.y;
      sdat.z = q == sq ? d[q].z : sdat.z; sdat.w = q == sq ? d[q].w : sdat.w;
    }
  }

  // ---- wave records ----------------------------------------------------------------
  {
    const float wm = dpp_wave_max_f32(best);
    const float kw = wm > -__builtin_inff() && weights ? __builtin_floorf(wm * chi) : 0.0f;  // K_w >= K_t
    if (nofilter) sm.kref[tid] = negk;
    if (weights && !nofilter) lsum = __builtin_ldexp(lsum, kfr > -__builtin_inff() ? (int)(kfr - kw) : 0);
    const double ws = (pon && !greedy) ? dpp_wave_sum_f64(lsum) : 0.0;
    uint32_t warg = 0xFFFFFFFFu;
    if (greedy) {
      uint32_t idx = 0xFFFFFFFFu;
      if (best == wm && wm > -__builtin_inff()) {
        // bq is the first of the thread's groups holding its maximum
        float z[8];
        load_z8<PEN>(bdat, bq * kNT + tid, pc, z);
#pragma unroll
        for (int e = 7; e >= 0; --e)
          if (z[e] == wm) idx = (uint32_t)(bq * kNT + tid) * 8u + (uint32_t)e;
      }
      warg = dpp_wave_min_u32(idx);
    }
    const uint32_t wflags = __ballot(bad || special) != 0 ? 1u : 0u;
    if (lane == 0) {
      sh.w_max[wid] = wm; sh.w_negk[wid] = -kw; sh.w_sum[wid] = ws;
      sh.w_arg[wid] = warg; sh.w_flags[wid] = wflags;
    }
    if (!greedy && !nofilter) {
      if (tid < kBins) {
        sm.bcnt[tid] = 0u;
        sm.bmass[tid] = 0.0f;
      }
      if (tid == kNT - 1) { sh.i32[3] = 0; sh.i32[6] = 0; }
    }
  }
  __syncthreads();

  // ---- wave 0: the row's values and the mode (lane w reads record w) ----------------
  if (wid == 0) {
    const bool rin = lane < kNW;
    const float rm = rin ? sh.w_max[lane] : -__builtin_inff();
    const float m = dpp_wave_max_f32(rm);
    int32_t mode = kModeFallback;
    float negks = 0.0f, zt = -__builtin_inff(), zc0 = -FLT_MAX;
    double S = 0.0, Pm = 0.0;
    uint32_t argmax = 0u;
    if (__ballot(rin && sh.w_flags[lane] != 0u)) {
      mode = kModeFallback;  // a signalling NaN or an out-of-range exponent frame
    } else if (greedy) {
      mode = kModeGreedy;
      argmax = m > -__builtin_inff() ? dpp_wave_min_u32(rin && rm == m ? sh.w_arg[lane] : 0xFFFFFFFFu) : 0u;
    } else if (m > -__builtin_inff() && m < __builtin_inff() && m * chi > -1048576.0f && m * chi < 1048576.0f) {
      // (all -inf rows, +inf, or a maximum too large for the exponent frame: general path)
      negks = -__builtin_floorf(m * chi);
      if (nofilter) {
        mode = kModeNoFilter;
      } else {
        bool ok = true;
        if (pon) {
          const double x = rin ? __builtin_ldexp(sh.w_sum[lane], (int)(negks - sh.w_negk[lane])) : 0.0;
          S = dpp_wave_sum_f64(x);
          ok = S > 0.0 && S < 1e300;
          Pm = (double)P.top_p * S;
        }
        if (mon) {
          bool found;
          zt = minp_threshold(m, tdl, found);
          ok = ok && found;
          zc0 = zt > -FLT_MAX ? zt : -FLT_MAX;
        }
        // min-p rows gather at the exact threshold; small rows take every
        // element; the others first bound the cut with a histogram
        if (!ok) mode = kModeFallback;
        else mode = (mon || ngroups <= kCandCap / 8) ? kModeCand : kModeHist;
      }
    }
    if (lane == 0) {
      sh.r_m = m; sh.r_negks = negks; sh.r_zt = zt; sh.r_zc = zc0;
      sh.r_S = S; sh.r_Pm = Pm; sh.r_mode = mode; sh.r_arg = argmax;
    }
  }
  __syncthreads();
  const float m = sh.r_m, negks = sh.r_negks, zt = sh.r_zt, zc0 = sh.r_zc;
  double S = sh.r_S;  // a lower bound of the row's mass while `lazy`
  double Pm = sh.r_Pm;
  int32_t mode = sh.r_mode;
  if (mode == kModeFallback) return false;

  if (mode == kModeGreedy) {
    path |= ARCS_PATH_GREEDY;
    const uint32_t argmax = sh.r_arg;
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
      for (int64_t i = tid; i < V; i += kNT) a.out_probs[row * V + i] = (i == (int64_t)argmax) ? 1.0f : 0.0f;
    return true;
  }

  // ---- the candidates z >= zc0 from the registers (min-p rows, small rows) ----------
  int nc = -1;
  if (mode == kModeCand) {
    gather_candidates<PEN>(rv, pc, sm, sh, zc0, best, bq, best2, sq, bdat, sdat, chi, clo, negks);
    __syncthreads();
    nc = sh.i32[3];
    // more than the list holds (min-p rows only): masked sums for min-p alone,
    // else a histogram bound above the threshold
    if (nc > kCandCap) mode = (!kon && !pon) ? kModeMinpStream : kModeHist;
  }

  int64_t id = -1;
  int64_t L = V;
  double S_K = 0.0;
  uint32_t cut_key = 0u;
  int64_t cut_idx = -1;

  if (mode == kModeNoFilter) {
    path |= ARCS_PATH_SORT_SKIP;
    if (!tsum_draw<PEN>(a, row, rv, pc, sm, sh, true, KeepCut{0u, INT64_MAX}, chi, clo, negks, u, debug, S))
      return false;
    if (!debug) return true;
    S_K = S;
    id = (int64_t)sh.u64[10];
  } else if (mode == kModeMinpStream) {
    // ---- min-p alone over many groups: masked sums and the id-order draw ------------
    path |= ARCS_PATH_CUTOFF | ARCS_PATH_MINP_FLOOR;
    {
      u32x4 dd[kQ];
      issue_row_loads(rv, ngroups, dd);  // the row again, from cache
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        float z[8];
        unpack8(dd[q], z);
        if (PEN && pc.on && tid < ngroups - q * kNT) penalize8(z, (int64_t)(q * kNT + tid) * 8, pc);
        const KeepCut cut{ord_key(zt), INT64_MAX};
        const int64_t i0 = (int64_t)(q * kNT + tid) * 8;
        float s = keep_cut(z[0], i0, cut) ? wexp(z[0], chi, clo, negks) : 0.0f;
#pragma unroll
        for (int e = 1; e < 8; ++e) s += keep_cut(z[e], i0 + e, cut) ? wexp(z[e], chi, clo, negks) : 0.0f;
        sm.tsum[q * kNT + tid] = tid < ngroups - q * kNT ? s : 0.0f;
      }
    }
    __syncthreads();
    if (!tsum_draw<PEN>(a, row, rv, pc, sm, sh, false, KeepCut{ord_key(zt), INT64_MAX}, chi, clo, negks, u, debug,
                        S_K))
      return false;
    if (!debug) return true;
    id = (int64_t)sh.u64[10];
    L = -1;  // counted with the debug outputs
    cut_key = ord_key(zt);
    cut_idx = INT64_MAX;
    S = 0.0;
  } else {
    path |= ARCS_PATH_CUTOFF;
    float zc = zc0;
    if (mode == kModeHist) {
      // a histogram of the threads' two largest group maxima by weight, 8
      // bins per unit of log2 weight below the row maximum: counts (top-k)
      // and weights (top-p, a lower bound of the mass above each bin's edge).
      // When the bound lies beyond the last bin (a large k at a low
      // temperature), the histogram is built again with bins 16 times wider.
      float b1 = -__builtin_inff(), b2 = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const float g = sm.tsum[q * kNT + tid];  // the group maxima
        b2 = g > b1 ? b1 : (g > b2 ? g : b2);
        b1 = g > b1 ? g : b1;
      }
      float c8 = (chi + clo) * 8.0f;
      for (int attempt = 0; attempt < 3; ++attempt, c8 *= 0.0625f) {
        if (attempt > 0) {
          if (tid < kBins) {
            sm.bcnt[tid] = 0u;
            sm.bmass[tid] = 0.0f;
          }
          __syncthreads();
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float v = h == 0 ? b1 : b2;
          if (v > -__builtin_inff()) {
            const float x = (m - v) * c8;
            const int bin = x < (float)(kBins - 1) ? (int)x : kBins - 1;
            atomicAdd(&sm.bcnt[bin], 1u);
            if (pon) atomicAdd(&sm.bmass[bin], wexp(v, chi, clo, negks));
          }
        }
        __syncthreads();
        if (wid == 0) {
          // the first bin (from the top) that meets a bound
          const uint4 c4 = ((const uint4*)sm.bcnt)[lane];
          const float4 m4 = ((const float4*)sm.bmass)[lane];
          const uint32_t cl[4] = {c4.x, c4.y, c4.z, c4.w};
          const double ml[4] = {(double)m4.x, (double)m4.y, (double)m4.z, (double)m4.w};
          const uint32_t ctot = cl[0] + cl[1] + cl[2] + cl[3];
          const double mtot = ml[0] + ml[1] + ml[2] + ml[3];
          const uint32_t cex = dpp_wave_incl_scan_u32(ctot) - ctot;
          const double mex = dpp_wave_incl_scan_f64(mtot) - mtot;
          const uint32_t k_need = kon ? (uint32_t)P.top_k : 0xFFFFFFFFu;
          const double p_need = (pon && !lazy) ? Pm * (1.0 + 1e-4) : __builtin_inf();
          int fb = 4;
          uint32_t cc = cex;
          double mc = mex;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cc += cl[i];
            mc += ml[i];
            if (fb == 4 && (cc >= k_need || mc >= p_need)) fb = i;
          }
          const uint64_t hb = __ballot(fb < 4);
          const int lb = hb ? __builtin_ctzll(hb) : 0;
          const int b = hb ? __builtin_amdgcn_readlane(lane * 4 + fb, lb) : kBins - 1;
          float zn = -__builtin_inff();  // -inf: no useful bound
          if (b < kBins - 1) {
            const float edge = (float)(b + 1) / c8;
            const float theta = (m - edge) - (1e-5f * (__builtin_fabsf(m) + edge) + 1e-30f);
            zn = theta > zc ? theta : zc;
          }
          if (lane == 0) { sh.r_zc = zn; sh.i32[3] = 0; }
        }
        __syncthreads();
        if (sh.r_zc > -__builtin_inff()) break;
      }
      zc = sh.r_zc;
      if (!(zc > -__builtin_inff())) return false;
      // ---- gather the candidates z >= zc -------------------------------------------
      gather_candidates<PEN>(rv, pc, sm, sh, zc, best, bq, best2, sq, bdat, sdat, chi, clo, negks);
      __syncthreads();
      nc = sh.i32[3];
    }
    const bool minp_complete = mon && !(zc > zt);
    if (minp_complete) path |= ARCS_PATH_MINP_FLOOR;
    if (nc > kCandCap || nc <= 0) return false;
    if (nc <= kSmallSort) {
      for (;;) {
        if (wid == 0) {
          const uint64_t key = lane < nc ? sm.ckey[lane] : ~0ull;
          const float w = lane < nc ? sm.cw[lane] : 0.0f;
          const double cap = lazy ? (double)P.top_p * S * (1.0 - 1e-5) : 0.0;
          const int rc = small_cut_draw(a, row, sm, sh, nc, key, w, kon, P.top_k, pon && !lazy, Pm, minp_complete,
                                        zt, u, cap);
          if (lane == 0) sh.i32[6] = rc == 1 ? 0 : (rc == 2 ? 1 : -1);
        }
        __syncthreads();
        if (!lazy || sh.i32[6] != 1) break;
        // top-p may cut inside the prefix: the exact mass, then the cut again
        S = exact_row_mass<PEN>(rv, pc, ngroups, chi, clo, negks, sh);
        Pm = (double)P.top_p * S;
        lazy = false;
      }
      if (sh.i32[6] < 0) return false;
      if (!debug) return true;
      id = (int64_t)sh.u64[10];
      L = (int64_t)sh.u64[11];
      S_K = sh.f64[kNW + 1];
      const uint64_t ck = sh.u64[12];
      cut_key = ~(uint32_t)(ck >> 32);
      cut_idx = (int64_t)(ck & 0xFFFFFFFFull);
    } else {
      // a larger set: select the cut, then draw in id order over masked group sums
      KeepCut cut;
      const int lowbit = (PEN && pc.on) ? 0 : 16;
      double kept_mass = 0.0;
      if (!large_cut_select(sm, sh, nc, lowbit, kon, P.top_k, pon && !lazy, Pm, minp_complete, zt, cut, L, kept_mass,
                            pon))
        return false;
      if (lazy && !(kept_mass < (double)P.top_p * S * (1.0 - 1e-5))) {
        // top-p may cut inside the prefix: the exact mass, then the cut again
        S = exact_row_mass<PEN>(rv, pc, ngroups, chi, clo, negks, sh);
        Pm = (double)P.top_p * S;
        lazy = false;
        if (!large_cut_select(sm, sh, nc, lowbit, kon, P.top_k, true, Pm, minp_complete, zt, cut, L, kept_mass, true))
          return false;
      }
      const double ux = u * 0x1p64;  // the uniform as a 64-bit fraction
      const uint64_t uf = ux >= 0x1p64 ? ~0ull : (ux <= 0.0 ? 0ull : (uint64_t)ux);
      if (!cand_draw(a, row, sm, sh, nc, cut, uf)) return false;
      if (!debug) return true;
      __syncthreads();
      id = (int64_t)sh.u64[10];
      S_K = sh.f64[kNW + 1];
      cut_key = cut.th;
      cut_idx = cut.istar;
    }
  }

  // ---- debug outputs (the row is read again) ---------------------------------------
  if (lazy) S = 0.0;  // only a bound: the re-read below gives the mass
  {
    const bool all_kept = (path & ARCS_PATH_SORT_SKIP) != 0;
    uint32_t kmin = 0xFFFFFFFFu;
    int64_t kmin_idx = -1;
    uint64_t amax = 0;  // (key of the maximum, complement of the lowest index holding it)
    uint32_t nkept = 0;
    double wtot = 0.0;
    for (int j = tid; j < ngroups; j += kNT) {
      float z[8];
      load_z8<PEN>(rv[j], j, pc, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t idx = (int64_t)j * 8 + e;
        const uint32_t k = ord_key(z[e] == z[e] ? z[e] : -__builtin_inff());
        const bool kept = all_kept || k > cut_key || (k == cut_key && idx <= cut_idx);
        const double w = (double)wexp(z[e], chi, clo, negks);
        if (a.out_probs) a.out_probs[row * V + idx] = kept ? (float)(w / S_K) : 0.0f;
        if (kept && (k < kmin || (k == kmin && idx > kmin_idx))) { kmin = k; kmin_idx = idx; }
        const uint64_t ak = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
        amax = ak > amax ? ak : amax;
        nkept += kept ? 1u : 0u;
        wtot += w;
      }
    }
    if (a.stats) {
      if (tid == 0) { sh.u64[9] = ~0ull; sh.u64[8] = 0ull; }
      __syncthreads();
      const uint64_t packed =
          ((uint64_t)kmin << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(kmin_idx < 0 ? 0 : kmin_idx));
      if (kmin_idx >= 0) atomicMin((unsigned long long*)&sh.u64[9], (unsigned long long)packed);
      atomicMax((unsigned long long*)&sh.u64[8], (unsigned long long)amax);
      const uint32_t wk = dpp_wave_sum_u32(nkept);
      const double wt = dpp_wave_sum_f64(wtot);
      if (lane == 0) {
        sh.rtot[wid] = wt;
        sh.w_cnt[wid] = wk;
      }
      __syncthreads();
      if (L < 0 || S == 0.0) {
        double a0 = 0.0;
        uint64_t a1 = 0;
        for (int w = 0; w < kNW; ++w) { a0 += sh.rtot[w]; a1 += sh.w_cnt[w]; }
        if (L < 0) L = (int64_t)a1;
        if (S == 0.0) S = a0;
      }
      if (tid == 0) {
        const uint64_t pk = sh.u64[9];
        const uint32_t argmax = 0xFFFFFFFFu - (uint32_t)(sh.u64[8] & 0xFFFFFFFFu);
        // masses reported relative to the row max, as sums of exp((z - m) / T)
        const double to_m = exp2((double)(-negks) - (double)m * ((double)chi + (double)clo));
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

// The penalised summary kernel holds the first kHistRegs * kNT history ids
// of its row in registers, loaded just before the row's own loads: waiting for
// them then leaves the row's loads in flight (loads complete in issue order).
constexpr int kHistRegs = 4;
struct RowHist {
  int64_t h0, h1;
  int32_t id[kHistRegs];  // -1 past the end
};

// Parameter status, history bounds and the history ids, issued before the
// row's loads.  Returns the row's status.
__device__ __forceinline__ int load_row_history(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                                PenCtx& pc, RowHist& hs) {
  const int tid = threadIdx.x;
  const int status = row_param_status(P);
  pc.on = false;
  pc.rep_on = !(P.repetition == 1.0f || P.repetition == 0.0f);
  pc.pres = P.presence; pc.freq = P.frequency; pc.rep = P.repetition;
  pc.zpen = nullptr; pc.pcount = nullptr;
  hs.h0 = 0; hs.h1 = 0;
  if (status == ARCS_ROW_OK && a.hist_ids != nullptr) {
    const bool active = P.presence != 0.0f || P.frequency != 0.0f || pc.rep_on;
    hs.h0 = a.hist_offsets[row];
    hs.h1 = a.hist_offsets[row + 1];
    pc.on = active && hs.h1 > hs.h0;
  }
  // branch-free: buffer loads past a resource's size return 0 without a
  // memory access (rows without active penalties get an empty resource; ids
  // outside [0, V) read past the row's resource and are skipped later)
  const int64_t n = pc.on ? hs.h1 - hs.h0 : 0;
  const int64_t nreg = n < (int64_t)kHistRegs * kNT ? n : (int64_t)kHistRegs * kNT;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pc.on ? a.hist_ids + hs.h0 : a.hist_ids), (short)0, (int)(nreg * 4), 0x00020000);
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k) {
    const int j = k * kNT + tid;
    const int32_t v = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(hr, j * 4, 0, 0);
    hs.id[k] = (int64_t)j < nreg ? v : -1;
  }
  return status;
}

// Visits the row's history ids in [0, V), with their raw logits (read from
// memory) when WITH_RAW: those held in registers, then any beyond them.
template <bool WITH_RAW, class Fn>
__device__ __forceinline__ void for_each_hist_id(const SampleArgs& a, int64_t row, const RowHist& hs, Fn&& f) {
  const uint16_t* rowp = (const uint16_t*)((const char*)a.logits + row * a.stride * 2);
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k)
    if (hs.id[k] >= 0 && (int64_t)hs.id[k] < a.V) f((uint32_t)hs.id[k], WITH_RAW ? bf16_to_f32(rowp[hs.id[k]]) : 0.0f);
  for (int64_t i = hs.h0 + (int64_t)kHistRegs * kNT + threadIdx.x; i < hs.h1; i += kNT) {
    const int32_t id = a.hist_ids[i];
    if (id >= 0 && (int64_t)id < a.V) f((uint32_t)id, WITH_RAW ? bf16_to_f32(rowp[id]) : 0.0f);
  }
}

// Penalty tables of the summary path, built while the row's loads are in
// flight (LDS-only barriers): the bitmap of the history ids over [0, V), the
// number of distinct ids before each bitmap word, and per distinct id (by
// rank, in id order) its occurrence count.  No logit is read here: the pass
// penalises each history id from its own logit.  Returns false when the row
// is finished (its status written).
__device__ __forceinline__ bool summary_pen_tables(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh,
                                                   int status, PenCtx& pc, const RowHist& hs, uint32_t& path) {
  const int tid = threadIdx.x;
  pc.bitmap = sm.bitmap; pc.wprefix = sm.wprefix; pc.zpen = sm.zpen; pc.pcount = sm.pcount;
  if (status == ARCS_ROW_OK && pc.on) {
    const uint32_t bw = a.bitmap_words;
    for (uint32_t i = tid; i < bw; i += kNT) sm.bitmap[i] = 0u;
    lds_barrier();
    for_each_hist_id<false>(a, row, hs, [&](uint32_t id, float) { atomicOr(&sm.bitmap[id >> 5], 1u << (id & 31)); });
    lds_barrier();
    const uint32_t per = (bw + kNT - 1) / kNT;
    const uint32_t w0 = tid * per, w1 = (w0 + per < bw) ? w0 + per : bw;
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; ++w) c += (uint32_t)__builtin_popcount(sm.bitmap[w]);
    uint32_t total;
    const uint32_t incl = block_incl_scan_u32<true>(c, sh.bs, total);
    if (total <= (uint32_t)kMaxDistinct) {
      uint32_t run = incl - c;
      for (uint32_t w = w0; w < w1; ++w) {
        sm.wprefix[w] = (uint16_t)run;
        run += (uint32_t)__builtin_popcount(sm.bitmap[w]);
      }
      for (uint32_t i = tid; i < total; i += kNT) sm.pcount[i] = 0u;
      lds_barrier();
      for_each_hist_id<false>(a, row, hs, [&](uint32_t id, float) {
        atomicAdd(&sm.pcount[pen_rank(id, sm.bitmap, sm.wprefix)], 1u);
      });
      lds_barrier();
    } else {
      status = ARCS_ROW_HISTORY_TOO_LONG;
      pc.on = false;
    }
  }
  if (status != ARCS_ROW_OK) {
    write_row_failure(a, row, status);
    return false;
  }
  path = pc.on ? ARCS_PATH_PENALTY : 0u;
  return true;
}

template <bool PEN>
__global__ __launch_bounds__(kNT) void sample_summary_kernel(SampleArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const Smem sm = carve_smem(smem_raw, true, a.bitmap_words);
  const int ngroups = (int)(a.V / 8);
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  u32x4 d[kQ];
  arcs_row_params P = a.params[row];
  const RowRng rng = load_row_rng(a, row);
  PenCtx pc;
  uint32_t path;
  if (!PEN) {
    // the row's loads go out right after the parameter record's, so that
    // validating it overlaps their latency
    __builtin_amdgcn_sched_barrier(0);
    issue_row_loads(rv, ngroups, d);
    if (!row_prologue<true, false>(a, row, sm, sh, P, pc, path)) return;
    if (!stream_row<false>(a, row, P, rng, pc, path, sm, sh, d)) {
      __syncthreads();
      generic_row<true, true>(a, row, P, pc, path, sm, sh);
    }
  } else {
    // history ids and the raw logits at them first, then the row's loads;
    // the tables are built while those are in flight
    RowHist hs;
    const int status = load_row_history(a, row, P, pc, hs);
    __builtin_amdgcn_sched_barrier(0);
    issue_row_loads(rv, ngroups, d);
    if (!summary_pen_tables(a, row, sm, sh, status, pc, hs, path)) return;
    if (!stream_row<true>(a, row, P, rng, pc, path, sm, sh, d)) {
      __syncthreads();
      if (pc.on) {
        // the general pipeline reads penalised logits per distinct id: built
        // here from the counts and the raw logits (every occurrence of an id
        // writes the same value)
        for_each_hist_id<true>(a, row, hs, [&](uint32_t id, float raw) {
          const uint32_t rk = pen_rank(id, sm.bitmap, sm.wprefix);
          sm.zpen[rk] = penalize(canon_nan(raw), sm.pcount[rk], pc);
        });
        __syncthreads();
      }
      generic_row<true, true>(a, row, P, pc, path, sm, sh);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
// fp32 rows (16-byte aligned, V % 4 == 0, V <= kF32MaxV, no penalty tables),
// one 512-thread workgroup per row, two rows resident per CU so that one
// row's cut and draw overlap the other's HBM read.  An fp32 row (517 KB at
// V = 129,280) does not fit the register file, and its top-p nucleus can hold
// most of the vocabulary, so the row is read twice:
//   pass 1 (HBM): the row maximum, the total mass S and, for rows with top-k
//     or top-p, an LDS histogram of counts and fixed-point masses over bins of
//     log2 weight (kFR bins per unit below an origin O = floor(max0 * c) + 1,
//     max0 the maximum of the first chunk of the row);
//   the bin b* where the first filter's target is crossed (top-k count, top-p
//     mass, or the min-p threshold's bin), widened by one bin on the side of a
//     top-p target that lies within the masses' rounding of the bin's edge;
//   pass 2 (re-read, from cache): the elements above the gathered bins (kept
//     for sure: their wave-round totals and count) and the elements of the
//     gathered bins, placed in LDS as candidates, both told apart by the
//     bins' value edges;
//   the exact cut among the candidates (radix select over their value keys);
//     a crossing found outside the gathered bins moves them by one bin and
//     gathers again, once;
//   the id-order draw: each wave keeps, per round, its total over the 64
//     groups it read (ids in order: round, wave, lane), a scan of those 512
//     totals finds the wave-round holding u * S_K, that wave re-reads its 1 KB
//     of the round and a lane walks its group.
// Weights are exp2(z * c - O) in fp32 (c = log2(e) / T), summed in fp64 per
// 4-element group; candidate weights are exact 2^-50 fixed point.  Bins come
// from one fma of z, so they never decrease as z decreases: bins above the
// gathered ones hold only values above every candidate.  Rows without filters
// skip pass 2; rows with min-p alone keep z >= the min-p threshold and gather
// nothing.  Rows it cannot finish (special values, masses out of range,
// candidate sets over kCandCap, a crossing further off) are left as
// kDeferredId in out_ids for the general kernel launched right after it, which
// skips every other row: inlined here, the general pipeline's register needs
// pushed this kernel into spills.
constexpr int kFT = 512;                                 // threads per row: two rows share a CU
constexpr int kFW = kFT / kWave;                         // waves per row (8)
constexpr int kFQ = 64;                                  // 16-byte rounds per thread
constexpr int kFC = 4;                                   // rounds per chunk (loads in flight per buffer)
constexpr int kFN = kFQ / kFC;                           // chunks per row
constexpr int64_t kF32MaxV = (int64_t)kFQ * kFT * 4;     // 131072
constexpr int kFB = 2048;                                // histogram bins
constexpr int kFRLog = 5;                                // 2^kFRLog bins per unit of log2 weight
constexpr float kFR = (float)(1 << kFRLog);
constexpr int kFS = kFQ * kFW;                           // wave-round slots (512)
static_assert(kFS == 8 * kWave, "the draw's slot scan gives each lane 8 slots");
// dynamic LDS of the fp32 kernel (bytes):
//   [0, 8K)     histogram counts u32[kFB]; then the cut's digit counts (sm.hcnt)
//   [8K, 16K)   histogram masses u32[kFB] (fixed point, per-bin scale); then the
//               cut's digit masses (sm.hmass, 512 u64)
//   [16K, 20K)  pass 1 wave-round weight totals f64[kFS] (slot q * kFW + wave)
//   [20K, 24K)  pass 2 wave-round totals of the elements kept for sure f64[kFS]
//   [24K, 28K)  wave-round fixed-point mass of kept candidates u64[kFS]
//   [28K, 76K)  candidates: keys u64[kCandCap], weights f32[kCandCap]
// The cut's tie ids go to the pass 1 totals' area (free once S is known).
// Two workgroups (rows) fit one CU's LDS.
constexpr size_t kF32OffHmass = (size_t)kFB * 4;
constexpr size_t kF32OffW1 = kF32OffHmass + (size_t)kFB * 4;
constexpr size_t kF32OffW2 = kF32OffW1 + (size_t)kFS * 8;
constexpr size_t kF32OffWfix = kF32OffW2 + (size_t)kFS * 8;
constexpr size_t kF32OffCand = kF32OffWfix + (size_t)kFS * 8;
constexpr size_t kF32OffSort = kF32OffW1;
constexpr size_t kF32Lds = kF32OffCand + (size_t)kCandCap * 12;
static_assert((size_t)kSmallSort * 12 <= (size_t)kFS * 8, "tie ids fit the pass 1 totals' area");
static_assert(2 * (kF32Lds + sizeof(Shared)) <= 160 * 1024, "two fp32 rows per CU");
static_assert(kF32OffW1 >= (size_t)kMaxBins * 4 + 512 * 8,
              "fp32 LDS layout: the cut's digit bins end before the wave-round totals");

__device__ __forceinline__ Smem carve_f32(unsigned char* raw) {
  Smem sm = carve_smem(raw, false, 0);
  sm.ckey = (uint64_t*)(raw + kF32OffCand);
  sm.cw = (float*)(raw + kF32OffCand + (size_t)kCandCap * 8);
  sm.skey = (uint64_t*)(raw + kF32OffSort);
  sm.sw = (float*)(raw + kF32OffSort + (size_t)kSmallSort * 8);
  return sm;
}

// Chunk c of this thread's rounds: round q = c * kFC + r reads group
// q * kFT + tid (ids 4 * (q * kFT + tid) .. + 3) through a buffer resource
// covering the rest of the row; lanes past its end read zeros without a
// memory access and are masked by the caller.  Default cache policy: the row
// is read again from cache.
__device__ __forceinline__ void issue_f32_chunk(const u32x4* rv, int ngroups, int c, u32x4 (&d)[kFC]) {
  const int voff = threadIdx.x * 16;
#pragma unroll
  for (int r = 0; r < kFC; ++r) {
    const int q = c * kFC + r;
    // the round's descriptor is formed here, not hoisted: 64 rounds of
    // descriptors held at once would crowd out the scalar registers
    int left = __builtin_amdgcn_readfirstlane((ngroups - q * kFT) * 16);
    asm volatile("" : "+s"(left));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(rv + (left > 0 ? q * kFT : 0)), (short)0, left > 0 ? left : 0, 0x00020000);
    d[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
  }
}

__device__ __forceinline__ void unpack4(u32x4 d, float (&z)[4]) {
  z[0] = __uint_as_float(d.x); z[1] = __uint_as_float(d.y);
  z[2] = __uint_as_float(d.z); z[3] = __uint_as_float(d.w);
}

// Bin of z: (O - z c) kFR clamped to [0, kFB - 1] (NaN -> 0, -inf -> last).
// Weights in bin b lie in (2^-(b+1)/kFR, 2^-b/kFR] (bin 0 also holds any above
// the origin), so the mass histogram stores w * 2^(floor(b / kFR) + 1 + 13)
// rounded to an integer, at most 2^14 per element below the origin: a u32 bin
// holds 2^17 elements.  Integer LDS atomics are far faster than float ones.
__device__ __forceinline__ uint32_t f32_bin(float z, float ncR, float OR) {
  float b = __builtin_fmaf(z, ncR, OR);
  b = __builtin_fmaxf(b, 0.0f);
  b = __builtin_fminf(b, (float)(kFB - 1));
  return (uint32_t)b;
}
// Only bin 0 can hold weights above 1 (elements above the origin); there
// an element adds at most 4 (2^16 units) and the caller keeps the excess
// max(w - 4, 0) aside.
constexpr int kFMassBits = 13;
__device__ __forceinline__ uint32_t f32_bin_mass(float w, uint32_t b) {
  const float x = __builtin_ldexpf(w, (int)(b >> kFRLog) + 1 + kFMassBits) + 0.5f;
  return (uint32_t)__builtin_fminf(x, 65536.0f);
}
__device__ __forceinline__ double f32_bin_mass_value(uint32_t s, int b) {
  return __builtin_ldexp((double)s, -((b >> kFRLog) + 1 + kFMassBits));
}

// Bin edges as values: E(n) = the largest float z with fma(z, ncR, OR) >= n,
// so that f32_bin(z) >= n exactly when z <= E(n) (the fma falls as z rises);
// E(0) = +inf, E(kFB) = -inf.  The 64 lanes of the wave test 64 consecutive
// floats around the estimate with the same fma; every lane gets the result.
// ok = false if the edge lies outside the window (never expected).
__device__ __forceinline__ float f32_bin_edge(int n, float ncR, float OR, bool& ok) {
  ok = true;
  if (n <= 0) return __builtin_inff();
  if (n >= kFB) return -__builtin_inff();
  const int lane = threadIdx.x & (kWave - 1);
  const double est = ((double)OR - (double)n) / -(double)ncR;
  const float z0 = est > (double)FLT_MAX ? FLT_MAX : (est < -(double)FLT_MAX ? -FLT_MAX : (float)est);
  const uint32_t k0 = ord_key(z0) - 32u;
  const float zl = key_value(k0 + (uint32_t)lane);
  const uint64_t ge = __ballot(__builtin_fmaf(zl, ncR, OR) >= (float)n);
  // true for the low lanes (small z), false above: a non-empty proper prefix
  ok = ge != 0 && ~ge != 0 && (ge & (ge + 1)) == 0;
  return key_value(k0 + (uint32_t)(ok ? 63 - __builtin_clzll(ge) : 0));
}

// Chunks 2.. of the row, with chunks 0 and 1 already in flight in d0 / d1:
// f(d, c) consumes chunk c while the next chunk's loads are in flight.
template <class F>
__device__ __forceinline__ void f32_stream_rest(const u32x4* rv, int ngroups, u32x4 (&d0)[kFC], u32x4 (&d1)[kFC],
                                                F&& f) {
#pragma unroll
  for (int c = 0; c < kFN; c += 2) {
    f(d0, c);
    if (c + 2 < kFN) issue_f32_chunk(rv, ngroups, c + 2, d0);
    f(d1, c + 1);
    if (c + 3 < kFN) issue_f32_chunk(rv, ngroups, c + 3, d1);
  }
}
// The whole row in kFN chunks of kFC rounds, two chunks' loads in flight.
template <class F>
__device__ __forceinline__ void f32_stream(const u32x4* rv, int ngroups, u32x4 (&d0)[kFC], u32x4 (&d1)[kFC],
                                           F&& f) {
  issue_f32_chunk(rv, ngroups, 0, d0);
  issue_f32_chunk(rv, ngroups, 1, d1);
  f32_stream_rest(rv, ngroups, d0, d1, f);
}

// Row values broadcast through LDS after a pass: per-wave records reduced
// by every thread in the same order (identical results in all threads).
// Each call site uses its own slots, so that a wave running ahead into the
// next reduction cannot overwrite a record another wave has yet to read.
__device__ __forceinline__ float f32_block_max(float v, float* slots) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = dpp_wave_max_f32(v);
  if (lane == 0) slots[wid] = v;
  lds_barrier();
  float m = slots[0];
#pragma unroll
  for (int w = 1; w < kFW; ++w) m = max2f(m, slots[w]);
  return m;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Block sum over the kFT threads of an fp32 row (every thread gets it).
__device__ __forceinline__ uint64_t f32_block_sum_u64(uint64_t v, uint64_t* slots) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_sum_u64(v);
  __syncthreads();
  if (lane == 0) slots[wid] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < kFW; ++w) t += slots[w];
  return t;
}

// This wave's total of one round's group values, stored at slot
// q * kFW + wave (every lane of the wave calls it).
__device__ __forceinline__ void f32_round_sum(double* W, int q, float gs) {
  const double s = dpp_wave_sum_f64((double)gs);
  if ((threadIdx.x & (kWave - 1)) == 0) W[q * kFW + threadIdx.x / kWave] = s;
}
// The sum of the kFS slot totals, the same in every wave.
__device__ __forceinline__ double f32_slot_total(const double* W) {
  const int lane = threadIdx.x & (kWave - 1);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += W[lane * 8 + i];
  return dpp_wave_sum_f64(s);
}

// Greedy rows: the lowest index of the maximum (NaN never wins; -0 = +0;
// a row of -inf and NaN gives 0).
__device__ __forceinline__ void f32_greedy(const SampleArgs& a, int64_t row, const u32x4* rv, int ngroups,
                                           u32x4 (&d0)[kFC], u32x4 (&d1)[kFC], Shared& sh, uint32_t path) {
  const int tid = threadIdx.x;
  float best = -__builtin_inff();
  int bidx = INT_MAX;
  auto f = [&](const u32x4 (&d)[kFC], int c) {
#pragma unroll
    for (int r = 0; r < kFC; ++r) {
      const int q = c * kFC + r;
      if (tid < ngroups - q * kFT) {
        float z[4];
        unpack4(d[r], z);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (z[e] > best) { best = z[e]; bidx = (q * kFT + tid) * 4 + e; }
      }
    }
  };
  f32_stream_rest(rv, ngroups, d0, d1, f);  // chunks 0 and 1 are in flight
  if (tid == 0) sh.i32[5] = INT_MAX;
  const float m = f32_block_max(best, sh.w_max);
  if (best == m && bidx != INT_MAX) atomicMin(&sh.i32[5], bidx);
  lds_barrier();
  const int64_t id = m == -__builtin_inff() ? 0 : (int64_t)sh.i32[5];
  path |= ARCS_PATH_GREEDY;
  if (m == __builtin_inff()) path |= ARCS_PATH_SPECIAL;
  if (tid == 0) {
    a.out_ids[row] = (int32_t)id;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
    if (a.stats) {
      arcs_row_stats st = {};
      st.id = (int32_t)id; st.argmax = (int32_t)id; st.kept = 0; st.cut_index = (int32_t)id;
      st.cut_value = m; st.max_logit = m; st.status = 0; st.path = path;
      st.mass_total = 0.0; st.mass_kept = 0.0; st.uniform = -1.0;
      a.stats[row] = st;
    }
  }
  if (a.out_probs)
    for (int64_t i = tid; i < a.V; i += kFT) a.out_probs[row * a.V + i] = (i == id) ? 1.0f : 0.0f;
}

// How a sampled row ends after pass 1.
enum F32Mode : int32_t { kF32Fallback = 0, kF32NoFilter = 1, kF32Thresh = 2, kF32Cand = 3 };

// The draw over the kept set in id order.  W holds each wave-round's kept
// total (fp64 sums of the sure elements' 4-element fp32 group sums), Wfix
// (or null) its kept candidates' fixed-point weights (times fscale).  Every
// wave scans the 512 slot totals (identical results), the wave of the
// crossing slot re-reads its 64 groups of that round and the crossing lane
// walks its group.  Kept elements are those `cut` keeps; an element in bin
// bstar is a candidate (weight from fixed point), one in a bin above it (or
// any kept element when bstar < 0) weighs its fp32 weight; eb / ec are the
// edges E(bstar) / E(bstar + 1): above eb a bin above bstar, in (ec, eb]
// bin bstar.  Returns the id,
// or -1 (uniformly) when the kept mass is not positive.
__device__ __forceinline__ int64_t f32_draw(const u32x4* rv, int ngroups, const double* W, const uint64_t* Wfix,
                                            double u, const KeepCut& cut, int bstar, float eb, float ec, float chi,
                                            float clo, float negO, float cscale, double fscale, Shared& sh,
                                            double& S_K) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  double vs[8];
  double ls = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = lane * 8 + i;
    vs[i] = W[s] + (Wfix ? (double)Wfix[s] * fscale : 0.0);
    ls += vs[i];
  }
  const double incl = dpp_wave_incl_scan_f64(ls);
  const double tot = readlane63_f64(incl);
  S_K = tot;
  if (!(tot > 0.0) || !(tot < 1e300)) return -1;
  const double t = u * tot;
  // the lane holding the crossing slot (rounding: the last lane with weight)
  const uint64_t cross = __ballot(incl > t && ls > 0.0);
  const uint64_t pos = __ballot(ls > 0.0);
  const int kl = cross ? __builtin_ctzll(cross) : 63 - __builtin_clzll(pos);
  // in that lane: the first slot whose running total passes t (rounding:
  // its last slot with weight) and the running total before it
  int sl = -1;
  double acc = incl - ls, sbase = 0.0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!found && vs[i] > 0.0) {
      sl = lane * 8 + i;
      sbase = acc;
      acc += vs[i];
      found = acc > t;
    }
  }
  const int sstar = __builtin_amdgcn_readlane(sl, kl);
  const double base = readlane_f64(sbase, kl);
  const int qs = sstar / kFW, ws = sstar % kFW;
  if (wid == ws) {
    // lane l takes group qs * kFT + ws * 64 + l (ids in order)
    const int g = qs * kFT + ws * kWave + lane;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint64_t fx[4] = {0ull, 0ull, 0ull, 0ull};
    if (g < ngroups) {
      const u32x4 dd = rv[g];
      float z[4];
      unpack4(dd, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t idx = (int64_t)g * 4 + e;
        const float w = wexp(z[e], chi, clo, negO);
        if (bstar < 0) {
          s[e] = keep_cut(z[e], idx, cut) ? w : 0.0f;
        } else {
          s[e] = z[e] > eb ? w : 0.0f;
          fx[e] = (z[e] > ec && !(z[e] > eb) && keep_cut(z[e], idx, cut)) ? to_fix50(w * cscale) : 0ull;
        }
      }
    }
    const float gs = (s[0] + s[1]) + (s[2] + s[3]);
    const uint64_t cf = (fx[0] + fx[1]) + (fx[2] + fx[3]);
    const double v = (double)gs + (double)cf * fscale;
    const double vin = dpp_wave_incl_scan_f64(v);
    const uint64_t lc = __ballot(base + vin > t && v > 0.0);
    const uint64_t lp = __ballot(v > 0.0);
    const int el = lc ? __builtin_ctzll(lc) : (lp ? 63 - __builtin_clzll(lp) : -1);
    if (el < 0 && lane == 0) sh.u64[15] = ~0ull;
    if (lane == el) {
      double a2 = base + vin - v;
      int64_t id = -1, last = -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double we = s[e] > 0.0f ? (double)s[e] : (double)fx[e] * fscale;
        if (we > 0.0 && id < 0) {
          a2 += we;
          last = (int64_t)g * 4 + e;
          if (a2 > t) id = last;
        }
      }
      sh.u64[15] = (uint64_t)(id >= 0 ? id : last);
    }
  }
  lds_barrier();
  return (int64_t)sh.u64[15];
}

// Pass 1 of a sampled row after the origin is known: chunk 0 (in d0),
// chunk 1 (in flight in d1) and the chunks after them.  Per group of 4:
// the maximum, the fp32 weights and their sum (each wave's round total into
// W1), and with HC / HM the histogram counts / masses (exc: the weight
// above bin 0's per-element limit).
template <bool HC, bool HM>
__device__ __forceinline__ void f32_pass1(const u32x4* rv, int ngroups, u32x4 (&d0)[kFC], u32x4 (&d1)[kFC],
                                          float chi, float clo, float negO, float ncR, float OR, uint32_t* hc,
                                          uint32_t* hm, double* W1, float& tmax, float& exc) {
  const int tid = threadIdx.x;
  auto weigh = [&](const u32x4 (&d)[kFC], int ch) {
#pragma unroll
    for (int r = 0; r < kFC; ++r) {
      const int q = ch * kFC + r;
      float gs = 0.0f;
      if (tid < ngroups - q * kFT) {
        float z[4];
        unpack4(d[r], z);
        tmax = max3f(tmax, max2f(z[0], z[1]), max2f(z[2], z[3]));
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = wexp(z[e], chi, clo, negO);
        gs = (w[0] + w[1]) + (w[2] + w[3]);
        if (HC || HM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t b = f32_bin(z[e], ncR, OR);
            if (HC) atomicAdd(&hc[b], 1u);
            if (HM) {
              atomicAdd(&hm[b], f32_bin_mass(w[e], b));
              exc += __builtin_fmaxf(w[e] - 4.0f, 0.0f);
            }
          }
        }
      }
      f32_round_sum(W1, q, gs);
    }
  };
  f32_stream_rest(rv, ngroups, d0, d1, weigh);
}

// Pass 2 of a row with candidates: each wave's round totals of the elements
// in bins above bstar (z > eb) into W2 (kept for sure), the elements of bin
// bstar (ec < z <= eb)
// gathered into LDS (keys and weights times cscale; their number in
// sh.i32[5], possibly above kCandCap), and per thread the number of sure
// elements and of candidates at or above zt.
__device__ __forceinline__ void f32_gather(const u32x4* rv, int ngroups, float eb, float ec, float zt, float chi,
                                           float clo, float negO, float cscale, const Smem& sm, double* W2,
                                           Shared& sh, uint32_t& cnt, uint32_t& cge) {
  const int tid = threadIdx.x;
  u32x4 d0[kFC], d1[kFC];
  f32_stream(rv, ngroups, d0, d1, [&](const u32x4 (&d)[kFC], int ch) {
#pragma unroll
    for (int r = 0; r < kFC; ++r) {
      const int q = ch * kFC + r;
      float gs = 0.0f;
      if (tid < ngroups - q * kFT) {
        float z[4], s[4];
        unpack4(d[r], z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool sure = z[e] > eb;
          const float w = wexp(z[e], chi, clo, negO);
          s[e] = sure ? w : 0.0f;
          cnt += sure ? 1u : 0u;
          if (z[e] > ec && !sure) {
            cge += z[e] >= zt ? 1u : 0u;
            const int slot = atomicAdd(&sh.i32[5], 1);
            if (slot < kCandCap) {
              sm.ckey[slot] = cand_key(z[e], (int64_t)(q * kFT + tid) * 4 + e);
              sm.cw[slot] = w * cscale;
            }
          }
        }
        gs = (s[0] + s[1]) + (s[2] + s[3]);
      }
      f32_round_sum(W2, q, gs);
    }
  });
}

// The sampled row on the fast path.  Returns false (uniformly) when the row
// needs the general pipeline; nothing is written then.
__device__ __forceinline__ bool f32_sample_row(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                               const RowRng& rng, uint32_t path, unsigned char* smem_raw,
                                               Shared& sh, u32x4 (&d0)[kFC], u32x4 (&d1)[kFC]) {
  const int tid = threadIdx.x;
  const int64_t V = a.V;
  const int ngroups = (int)(V / 4);
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 4);
  const bool kon = P.top_k >= 1 && (int64_t)P.top_k < V;
  const bool pon = P.top_p < 1.0f;
  const bool mon = P.min_p > 0.0f;
  const bool nofilter = !kon && !pon && !mon;
  const bool hist = kon || pon;
  path |= ARCS_PATH_REREAD;
  const Smem sm = carve_f32(smem_raw);
  uint32_t* hc = (uint32_t*)smem_raw;
  uint32_t* hm = (uint32_t*)(smem_raw + kF32OffHmass);
  double* W1 = (double*)(smem_raw + kF32OffW1);
  double* W2 = (double*)(smem_raw + kF32OffW2);
  uint64_t* Wfix = (uint64_t*)(smem_raw + kF32OffWfix);

  // c = log2(e) / T = chi + clo, chi rounded down, clo > 0 (weights and bins
  // never decrease with z)
  const double c = 1.4426950408889634 / (double)P.temperature;
  if (!(c >= 1e-30 && c <= 1e30)) return false;
  float chi = (float)c;
  if ((double)chi >= c) chi = key_value(ord_key(chi) - 1u);
  float clo = (float)(c - (double)chi);
  if (!(clo > 0.0f)) clo = 1e-30f;
  chi = uniform_f32(chi);
  clo = uniform_f32(clo);
  const double tdl = mon ? uniform_f64((double)P.temperature * log((double)P.min_p)) : 0.0;
  double u;
  if (rng.override_on) {
    u = rng.u_override;
  } else {
    const uint64_t x = splitmix64_counter_output(rng.seed, (uint64_t)row, rng.step);
    u = (double)(x >> 11) * 0x1p-53;
  }
  u = uniform_f64(u);

  if (hist)
    for (int i = tid; i < kFB; i += kFT) { hc[i] = 0u; hm[i] = 0u; }
  // ---- pass 1: the origin from chunk 0's maximum, then weights, sums, bins --
  float tmax = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < kFC; ++r) {
    if (tid < ngroups - r * kFT) {
      float z[4];
      unpack4(d0[r], z);
      tmax = max3f(tmax, max2f(z[0], z[1]), max2f(z[2], z[3]));
    }
  }
  const float mA = f32_block_max(tmax, sh.w_negk);
  const double Od = __builtin_floor((double)mA * c) + 1.0;
  if (!(Od > -8388608.0 && Od < 8388608.0)) return false;
  const float negO = uniform_f32((float)-Od);
  const float OR = uniform_f32((float)(Od * (double)kFR));
  const float ncR = uniform_f32(-(float)(c * (double)kFR));
  // top-k <= the row's thread count: every cut lies within the bins down to
  // that of the k-th largest thread maximum (at least k elements are at or
  // above it, so the top-k prefix, and any shorter one, is there); those bins
  // come from the thread maxima alone, and the pass needs no histogram
  const bool kwin = kon && P.top_k <= (ngroups < kFT ? ngroups : kFT);
  const bool hcount = kon && !kwin, hmass = pon && !kwin;
  float exc = 0.0f;
  if (hcount && hmass) f32_pass1<true, true>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc);
  else if (hcount) f32_pass1<true, false>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc);
  else if (hmass) f32_pass1<false, true>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc);
  else f32_pass1<false, false>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc);
  if (kwin && tid < ngroups) atomicAdd(&hc[f32_bin(tmax, ncR, OR)], 1u);
  if (hmass) {
    const double we = dpp_wave_sum_f64((double)exc);
    if ((tid & (kWave - 1)) == 0) sh.w_sum[tid / kWave] = we;
  }
  const float m = f32_block_max(tmax, sh.w_max);
  const double S = f32_slot_total(W1);
  if (!(m > -__builtin_inff() && m < __builtin_inff()) || !(S > 0.0 && S < 1e300)) return false;
  const float tm = wexp(m, chi, clo, negO);  // the maximum's weight (> 1/2 unless m lies above O)
  if (!(tm > 0.0f && tm < 1e30f)) return false;
  int ex = 0;
  if (tm >= 1.0f) (void)__builtin_frexpf(tm, &ex);
  const float cscale = __builtin_ldexpf(1.0f, -ex);    // candidate weights * cscale < 1
  const double fscale = __builtin_ldexp(1.0, ex - 50);  // 2^-50 fixed point back to the O frame

  int32_t mode = nofilter ? kF32NoFilter : (hist ? kF32Cand : kF32Thresh);
  int bstar = -1, bhi = -1;  // candidate rows: the bins gathered, bstar .. bhi
  float zt = -__builtin_inff();
  if (mon) {
    bool ok;
    zt = minp_threshold(m, tdl, ok);
    if (!ok) return false;
  }
  if (mode == kF32Cand) {
    // wave 0: the first bin (from the top) where the top-k count (of elements,
    // or of thread maxima for kwin) or the top-p mass target is reached; lane l
    // sums bins 32l .. 32l + 31
    constexpr int PER = kFB / kWave;
    const int lane = tid & (kWave - 1);
    if (tid < kWave) {
      const double Pm = pon ? (double)P.top_p * S : 0.0;
      uint32_t lc = 0;
      double lm = 0.0, exc0 = 0.0;
      if (hmass) {
#pragma unroll
        for (int w = 0; w < kFW; ++w) exc0 += sh.w_sum[w];
      }
#pragma unroll 8
      for (int j = 0; j < PER; ++j) {
        lc += hc[lane * PER + j];
        lm += f32_bin_mass_value(hm[lane * PER + j], lane * PER + j);
      }
      if (lane == 0) lm += exc0;
      const uint32_t ic = dpp_wave_incl_scan_u32(lc);
      const double im = dpp_wave_incl_scan_f64(lm);
      const uint64_t hk = __ballot(kon && ic >= (uint32_t)P.top_k);
      const uint64_t hp = __ballot(hmass && im >= Pm);
      if (lane == 0) { sh.i32[6] = kFB; sh.i32[7] = kFB; }
      if (hk && lane == __builtin_ctzll(hk)) {
        uint32_t cc = ic - lc;
        int bk = lane * PER + PER - 1;
        for (int j = 0; j < PER; ++j) {
          cc += hc[lane * PER + j];
          if (cc >= (uint32_t)P.top_k) { bk = lane * PER + j; break; }
        }
        sh.i32[6] = bk;
      }
      if (lane == 0) sh.i32[3] = 0;
      if (hp && lane == __builtin_ctzll(hp)) {
        double cm = im - lm + (lane == 0 ? exc0 : 0.0), before = cm;
        int bp = lane * PER + PER - 1;
        for (int j = 0; j < PER; ++j) {
          before = cm;
          cm += f32_bin_mass_value(hm[lane * PER + j], lane * PER + j);
          if (cm >= Pm) { bp = lane * PER + j; break; }
        }
        sh.i32[7] = bp;
        // the target within the masses' rounding of an edge of the bin: the
        // neighbouring bin is gathered too (1: the bin above, 2: below)
        sh.i32[3] = (Pm - before <= 2e-5 * Pm ? 1 : 0) | (cm - Pm <= 2e-5 * Pm ? 2 : 0);
      }
    }
    lds_barrier();
    const int bk = kon ? sh.i32[6] : kFB;
    const int bp = pon ? sh.i32[7] : kFB;
    const int bm = mon ? (int)f32_bin(zt, ncR, OR) : kFB;
    bstar = bk < bp ? bk : bp;
    bstar = bm < bstar ? bm : bstar;
    // no crossing found (top-p alone, its float masses short of the target
    // by rounding)
    if (bstar >= kFB) return false;
    bhi = bstar;
    if (kwin) {
      bstar = 0;  // the whole window is gathered; nothing is kept for sure
    } else if (pon && bstar == bp) {
      const int near = sh.i32[3];
      if ((near & 1) && bstar > 0) bstar -= 1;
      if ((near & 2) && bhi < kFB - 1) bhi += 1;
    }
  }

  // ---- pass 2: sure masses per thread, candidates of bin b* ---------------------
  KeepCut cut;
  cut.th = 0u;
  cut.istar = INT64_MAX;
  float eb = 0.0f, ec = 0.0f;  // value edges of the gathered bins (candidate rows)
  int64_t L = V;
  if (mode != kF32NoFilter) {
    uint32_t cnt = 0;  // elements kept for sure
    uint32_t cge = 0;  // candidates at or above the min-p threshold
    if (mode == kF32Thresh) {
      cut.th = ord_key(zt);
      f32_stream(rv, ngroups, d0, d1, [&](const u32x4 (&d)[kFC], int ch) {
#pragma unroll
        for (int r = 0; r < kFC; ++r) {
          const int q = ch * kFC + r;
          float gs = 0.0f;
          if (tid < ngroups - q * kFT) {
            float z[4], s[4];
            unpack4(d[r], z);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool k = z[e] >= zt;
              s[e] = k ? wexp(z[e], chi, clo, negO) : 0.0f;
              cnt += k ? 1u : 0u;
            }
            gs = (s[0] + s[1]) + (s[2] + s[3]);
          }
          f32_round_sum(W2, q, gs);
        }
      });
      path |= ARCS_PATH_CUTOFF | ARCS_PATH_MINP_FLOOR;
      __syncthreads();
      L = (int64_t)f32_block_sum_u64(cnt, sh.bs.u64);
    } else {
      // The histogram places b* from rounded masses; the exact sums decide.
      // A crossing found one bin off (the target within rounding of a bin
      // edge) moves b* by one bin and gathers again, once.  (Written as a
      // second call rather than a loop: a loop lets the compiler hoist the
      // rounds' load descriptors out of it and spill.)
      path |= ARCS_PATH_CUTOFF;
      const int bm = mon ? (int)f32_bin(zt, ncR, OR) : kFB;
      // returns 0 when the cut is found, -1 / +1 when the crossing lies one
      // bin above / below b*, 2 when the row needs the general pipeline
      auto try_cut = [&]() __attribute__((always_inline)) -> int {
        cnt = 0;
        cge = 0;
        if (tid == 0) sh.i32[5] = 0;
        if (tid < kFS) Wfix[tid] = 0ull;
        lds_barrier();
        bool eok, cok;
        eb = f32_bin_edge(bstar, ncR, OR, eok);
        ec = f32_bin_edge(bhi + 1, ncR, OR, cok);
        if (!eok || !cok) return 2;
        f32_gather(rv, ngroups, eb, ec, zt, chi, clo, negO, cscale, sm, W2, sh, cnt, cge);
        __syncthreads();
        const int nc = sh.i32[5];
        const double A = f32_slot_total(W2);
        const uint64_t sums = f32_block_sum_u64((uint64_t)cnt | ((uint64_t)cge << 32), sh.bs.u64);
        const uint32_t above = (uint32_t)sums;
        L = (int64_t)above;
        if (nc > kCandCap) return 2;
        const bool binding_m = bm >= bstar && bm <= bhi;
        // step: 0 done, -1 the crossing lies above b*, +1 below it
        int step = 0;
        const double need = pon ? ((double)P.top_p * S - A) * (double)cscale : 0.0;
        if (pon && !(need > 0.0)) {
          step = -1;
        } else if (mon && (sums >> 32) == 0) {
          // no candidate reaches the min-p threshold (b* is its bin): the kept
          // set is the sure set, exactly the elements at or above it (top-k
          // and top-p keep at least one candidate more, so min-p binds)
          if (!binding_m) return 2;
          cut.th = ord_key(zt);
          path |= ARCS_PATH_MINP_FLOOR;
        } else if (nc == 0) {
          step = 1;
        } else {
          int64_t Lc = 0;
          double kmass = 0.0;
          if (!large_cut_select<kFT>(sm, sh, nc, 0, kon, kon ? P.top_k - (int)above : 0, pon, need, mon, zt, cut, Lc,
                                kmass, pon)) {
            step = 1;  // only top-p can miss its target here
          } else {
            L += Lc;
            if (cut.istar != INT64_MAX) path |= ARCS_PATH_TIE_SPLIT;
            if (binding_m) path |= ARCS_PATH_MINP_FLOOR;
            // kept candidates' fixed-point weights, summed per wave-round slot
            // (group g = idx / 4 is read in round g / kFT by wave (g % kFT) / 64)
#pragma unroll
            for (int r = 0; r < kCandCap / kFT; ++r) {
              const int i = tid + r * kFT;
              if (i < nc) {
                const uint64_t k = sm.ckey[i];
                const uint32_t idx = (uint32_t)k;
                const float z = key_value(~(uint32_t)(k >> 32));
                const uint32_t g = idx >> 2;
                if (keep_cut(z, (int64_t)idx, cut))
                  atomicAdd((unsigned long long*)&Wfix[(g / kFT) * kFW + (g % kFT) / kWave],
                            (unsigned long long)to_fix50(sm.cw[i]));
              }
            }
          }
        }
        return step;
      };
      int st = try_cut();
      if (st == 1 || st == -1) {
        bstar = st < 0 ? bstar - 1 : bhi + 1;
        bhi = bstar;
        st = 2;
        if (bstar >= 0 && bstar < kFB) {
          __syncthreads();
          st = try_cut();
        }
      }
      if (st != 0) return false;
      lds_barrier();
    }
  } else {
    path |= ARCS_PATH_SORT_SKIP;
  }
  double S_K = 0.0;
  const int64_t id = f32_draw(rv, ngroups, mode == kF32NoFilter ? W1 : W2, mode == kF32Cand ? Wfix : nullptr, u,
                              cut, mode == kF32Cand ? bstar : -1, eb, ec, chi, clo, negO, cscale, fscale, sh, S_K);
  if (id < 0) return false;
  if (tid == 0) {
    a.out_ids[row] = (int32_t)id;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
  }
  // ---- debug outputs ------------------------------------------------------------
  if (a.stats || a.out_probs) {
    const double inv_sk = 1.0 / S_K;
    uint32_t kmin = 0xFFFFFFFFu;
    int64_t kmin_idx = -1;
    int amin = INT_MAX;
    for (int g = tid; g < ngroups; g += kFT) {
      float z[4];
      unpack4(rv[g], z);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t idx = (int64_t)g * 4 + e;
        const bool kept = keep_cut(z[e], idx, cut);
        if (a.out_probs)
          a.out_probs[row * V + idx] = kept ? (float)((double)wexp(z[e], chi, clo, negO) * inv_sk) : 0.0f;
        if (kept) {
          const uint32_t k = ord_key(z[e]);
          if (k < kmin || (k == kmin && idx > kmin_idx)) { kmin = k; kmin_idx = idx; }
        }
        if (z[e] == m && amin == INT_MAX) amin = (int)idx;
      }
    }
    if (a.stats) {
      if (tid == 0) { sh.u64[9] = ~0ull; sh.i32[5] = INT_MAX; }
      __syncthreads();
      const uint64_t packed =
          ((uint64_t)kmin << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(kmin_idx < 0 ? 0 : kmin_idx));
      if (kmin_idx >= 0) atomicMin((unsigned long long*)&sh.u64[9], (unsigned long long)packed);
      if (amin != INT_MAX) atomicMin(&sh.i32[5], amin);
      __syncthreads();
      if (tid == 0) {
        const uint64_t pk = sh.u64[9];
        arcs_row_stats st = {};
        st.id = (int32_t)id; st.argmax = sh.i32[5]; st.kept = (int32_t)L;
        st.cut_index = (int32_t)(0xFFFFFFFFu - (uint32_t)(pk & 0xFFFFFFFFu));
        st.cut_value = key_value((uint32_t)(pk >> 32));
        st.max_logit = m; st.status = 0; st.path = path;
        st.mass_total = S / (double)tm;
        st.mass_kept = S_K / (double)tm;
        st.uniform = u;
        a.stats[row] = st;
      }
    }
  }
  return true;
}

__global__ __launch_bounds__(kFT, 4) void sample_f32_kernel(SampleArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const int ngroups = (int)(a.V / 4);
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 4);
  arcs_row_params P = a.params[row];
  const RowRng rng = load_row_rng(a, row);
  u32x4 d0[kFC], d1[kFC];
  __builtin_amdgcn_sched_barrier(0);
  issue_f32_chunk(rv, ngroups, 0, d0);
  issue_f32_chunk(rv, ngroups, 1, d1);
  __builtin_amdgcn_sched_barrier(0);
  // parameters (rows with history never reach this kernel)
  const int status = row_param_status(P);
  if (status != ARCS_ROW_OK) {
    if (threadIdx.x == 0) {
      a.out_ids[row] = -1;
      if (a.out_status) a.out_status[row] = status;
      if (a.stats) {
        arcs_row_stats st = {};
        st.id = -1; st.argmax = -1; st.status = status;
        a.stats[row] = st;
      }
    }
    if (a.out_probs)
      for (int64_t i = threadIdx.x; i < a.V; i += kFT) a.out_probs[row * a.V + i] = 0.0f;
    return;
  }
  const uint32_t path = 0u;
  if (P.temperature == 0.0f || P.top_k == 1) {
    f32_greedy(a, row, rv, ngroups, d0, d1, sh, path);
    return;
  }
  if (!f32_sample_row(a, row, P, rng, path, smem_raw, sh, d0, d1) && threadIdx.x == 0)
    a.out_ids[row] = kDeferredId;
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
  if (dtype == ARCS_DTYPE_F32 && vec && !pen && a.V <= kF32MaxV && a.V % 4 == 0) {
    static std::atomic<int> f32_done{0};
    if (!f32_done.load(std::memory_order_acquire)) {
      hipError_t e = hipFuncSetAttribute((const void*)sample_f32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)kF32Lds);
      if (e != hipSuccess) return e;
      f32_done.store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL(sample_f32_kernel, dim3((unsigned)B), dim3(kFT), kF32Lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the rows it handed back (a row's block exits at once otherwise)
    SampleArgs g = a;
    g.deferred_only = 1;
    return launch_one(sample_kernel<false, true, false>, false, g, B, sample_lds_bytes(false, false, a.V), stream,
                      done[7]);
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

// The step of a device-held key moves on by one.  Enqueued after the
// sampling kernel on the same stream, so every workgroup has read the old
// value; inside a captured graph each replay advances it.
__global__ void advance_step_kernel(uint64_t* key) {
  if (threadIdx.x == 0 && blockIdx.x == 0) key[1] += 1u;
}

hipError_t launch_advance_step(uint64_t* key, hipStream_t stream) {
  hipLaunchKernelGGL(advance_step_kernel, dim3(1), dim3(64), 0, stream, key);
  return hipGetLastError();
}

}  // namespace arcs
