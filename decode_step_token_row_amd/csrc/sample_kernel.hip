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
// The kernels:
//
// sample_summary_kernel (bf16 rows, 16-byte aligned, V <= 131072, V % 8 == 0;
//   512 threads, 32 rounds of 16 bytes per thread, or 1024 threads and 16
//   rounds in launches with history arrays): the row is read from HBM
//   exactly once, every load issued before any is used (in the penalised
//   kernel a quarter of them before the penalty tables are built, the rest
//   after).  Each thread turns every group of 8 logits
//   (penalised through LDS tables when the row has active penalties) into
//   its maximum and, for rows with top-p, its fp32 weight
//   exp2(z*log2(e)/T - K_t) (K_t an integer reference exponent of the thread,
//   so moving sums between frames is an exact power of two); rows without
//   filters weigh every element in double precision instead and keep each
//   wave's total per round.  After the pass, per-wave records and one wave
//   give the row's maximum, mass and min-p threshold, and then:
//     greedy rows   -> the lowest index of the maximum, from registers;
//     no filter     -> an id-order draw over the double weights (round,
//                      wave, lane, element), from registers;
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
// split_partial_kernel (batches of at most 64 bf16 rows): slices of each
//   row read by many workgroups; the summary kernel then finishes greedy rows
//   and rows without filters from the slice records.
//
// sample_f32_kernel (fp32 rows, V <= 131072): one read from HBM with a
//   histogram of weights, one from cache gathering the crossing bin.
//
// long_history_prep_kernel: penalised logits of rows beyond the LDS penalty
//   tables, written in binary32 to the caller's workspace.
//
// sample_kernel (everything else, and the rows the others hand back): the
//   general streaming pipeline of sample_common.hpp -- pass A for
//   max/argmax, fixed-point softmax mass, radix-select cutoff over
//   order-preserving keys, id-order draw -- with re-walks of the row served
//   from L2 / the Infinity Cache.
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
  if (!row_prologue<kNT, BF16, PEN>(a, row, sm, sh, P, pc, path)) return;
  generic_row<kNT, BF16, VEC>(a, row, P, pc, path, sm, sh);
}

// ---------------------------------------------------------------------------
// summary kernel helpers (independent of the workgroup shape)
// ---------------------------------------------------------------------------
// The summary path of the sampler (bf16 rows kept in registers), written
// once for a workgroup of kSNT threads: the file is included inside a
// namespace that defines kSNT (no include guard on purpose), so that the
// kernel exists in more than one workgroup shape.  See sample_kernel.hip for
// what the path computes.
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


// Element e of the group (e differs from lane to lane) replaced by its
// penalised value for an id seen cnt times.
__device__ __forceinline__ void penalize_elem(float (&z)[8], int e, uint32_t cnt, const PenCtx& pc) {
  float ze = z[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) ze = e == k ? z[k] : ze;
  const float pz = penalize(canon_nan(ze), cnt, pc);
#pragma unroll
  for (int k = 0; k < 8; ++k) z[k] = e == k ? pz : z[k];
}

// The history ids among the 8 elements of the group at g0 (a multiple of 8)
// replaced by their penalised values, from their own logit and their
// occurrence count in the LDS tables (the general path's binary32 sequence):
// one pass of the loop per history id in the group (groups without one cost
// a bitmap read).
__device__ __forceinline__ void penalize8(float (&z)[8], int64_t g0, const PenCtx& pc) {
  const uint32_t w = (uint32_t)(g0 >> 5), s5 = (uint32_t)(g0 & 31);
  const uint32_t word = pc.bitmap[w];
  uint32_t bits = (word >> s5) & 0xFFu;
  if (!bits) return;
  uint32_t r = (uint32_t)pc.wprefix[w] + (uint32_t)__builtin_popcount(word & ((1u << s5) - 1u));
  do {
    const int e = __builtin_ctz(bits);
    bits &= bits - 1u;
    penalize_elem(z, e, pc.pcount[r++], pc);
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


// The row's parameter record as two 16-byte vector loads (into vector
// registers, read back with readfirstlane once needed): issued before the
// row's loads, they return first, and nothing in the issue of the row's loads
// waits for them (a scalar load here would hold the issue until it returns).
__device__ __forceinline__ void issue_params_load(const arcs_row_params* prow, u32x4& p0, u32x4& p1) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)prow, (short)0, 32, 0x00020000);
  p0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0));
  p1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16, 0, 0));
}
__device__ __forceinline__ arcs_row_params params_from(u32x4 p0, u32x4 p1) {
  arcs_row_params P;
  P.temperature = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p0.x));
  P.top_k = __builtin_amdgcn_readfirstlane((int)p0.y);
  P.top_p = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p0.z));
  P.min_p = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p0.w));
  P.presence = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p1.x));
  P.frequency = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p1.y));
  P.repetition = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)p1.z));
  P.flags = __builtin_amdgcn_readfirstlane((int)p1.w);
  return P;
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
// What the pass leaves per thread for the rest of a filter or no-filter row.
struct PassOut {
  float best;         // the thread's largest value (-inf: none)
  int bq;             // the first round whose group holds it (-1: none)
  float second;       // filter rows: the largest maximum of the thread's other groups
  double lsum;        // top-p rows: the thread's weight total in its frame 2^-kfr
  float kfr, negk;    // the frame exponent (-inf before the first finite group) and -kfr
  bool bad, special;  // a frame out of range; a signalling NaN
};

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

// The same values through two unconditional vector loads (a missing array
// reads zeros through an empty buffer resource), issued before the row's
// loads: with no branch around them, a wait for them counts only the loads
// issued before them and never drains the row's loads.
struct RngLoads {
  u32x4 key;
  u32x4 ovr;
};
__device__ __forceinline__ RngLoads issue_rng_loads(const SampleArgs& a, int64_t row) {
  RngLoads l;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.key, (short)0, a.key ? 16 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.uniforms ? a.uniforms + row : nullptr), (short)0, a.uniforms ? 8 : 0, 0x00020000);
  l.key = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 0, 0, 0));
  l.ovr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ru, 0, 0, 0));
  return l;
}
__device__ __forceinline__ RowRng rng_from(const SampleArgs& a, const RngLoads& l) {
  auto u64_of = [](uint32_t lo, uint32_t hi) {
    return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)lo) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)hi) << 32);
  };
  RowRng r;
  r.override_on = a.uniforms != nullptr;
  r.u_override = r.override_on ? __builtin_bit_cast(double, u64_of(l.ovr.x, l.ovr.y)) : 0.0;
  r.seed = a.key ? u64_of(l.key.x, l.key.y) : a.seed;
  r.step = a.key ? u64_of(l.key.z, l.key.w) : a.step;
  return r;
}

// The row's constants for the summary path: the temperature coefficient
// c = log2(e) / T = chi + clo (chi rounded down, clo > 0), T ln(min_p) and the
// uniform.  ok = false for temperatures so extreme that z * c leaves the
// float range (the general pipeline takes the row).  Greedy rows need none.
struct RowConsts {
  float chi, clo;
  double tdl, u;
  bool ok;
};
// c = log2(e) / T as chi + clo (chi rounded down, clo > 0, so weights and
// bins never decrease with z); false when c is out of range.
__device__ __forceinline__ bool temp_coeffs(float T, float& chi, float& clo) {
  const double c = 1.4426950408889634 / (double)T;
  if (!(c >= 1e-30 && c <= 1e30)) return false;
  chi = (float)c;
  if ((double)chi >= c) chi = key_value(ord_key(chi) - 1u);
  clo = (float)(c - (double)chi);
  if (!(clo > 0.0f)) clo = 1e-30f;
  chi = uniform_f32(chi);
  clo = uniform_f32(clo);
  return true;
}
__device__ __forceinline__ RowConsts row_consts(const arcs_row_params& P, const RowRng& rng, int64_t row) {
  RowConsts r;
  r.chi = 0.0f; r.clo = 0.0f; r.tdl = 0.0; r.u = 0.0; r.ok = true;
  if (P.temperature == 0.0f || P.top_k == 1) return r;
  if (!temp_coeffs(P.temperature, r.chi, r.clo)) { r.ok = false; return r; }
  if (P.min_p > 0.0f) r.tdl = uniform_f64((double)P.temperature * log((double)P.min_p));
  double u;
  if (rng.override_on) {
    u = rng.u_override;
  } else {
    const uint64_t x = splitmix64_counter_output(rng.seed, (uint64_t)row, rng.step);
    u = (double)(x >> 11) * 0x1p-53;
  }
  r.u = uniform_f64(u);
  return r;
}

// The penalised summary kernel holds the first kHistRegs * kSNT history ids
// of its row in registers, loaded just before the row's own loads: waiting for
// them then leaves the row's loads in flight (loads complete in issue order).
constexpr int kHistRegs = 4;

// Rows without filters weigh every element in double precision: fp32
// weights carry relative errors near 1e-7, and on rows whose heavy tokens
// precede long tails of tiny ones that moves many CDF boundaries by more
// than the tail tokens' widths.  w = 2^(z c) with c = log2(e) / T and no
// frame (the row maximum keeps |m c| <= kF64Span, else the general path).
// The group's weights are summed in id order; both the pass and the draw
// call this, so the draw sees the pass's values exactly.  The powers come
// from exp2_f64_tab, its table in LDS (fill_exp2_table first).
constexpr double kF64Span = 960.0;
__device__ __forceinline__ double group_weights_f64(const float (&z)[8], bool valid, double c, double (&w)[8],
                                                    const double* T64) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    w[e] = valid ? exp2_f64_tab((double)z[e] * c, T64) : 0.0;
    s += w[e];
  }
  return s;
}
// exp2_f64_tab's table, written by every wave that uses it (the same values
// everywhere, so no workgroup barrier: each wave reads its own writes).
__device__ __forceinline__ void fill_exp2_table(double* T64) {
  const int lane = threadIdx.x & (kWave - 1);
  T64[lane] = exp2_f64((double)lane * 0.015625);
  wave_lds_sync();
}


// ---------------------------------------------------------------------------
// split rows, first half: slice partials.  Grid (P, B), kSplitThreads
// threads; workgroup (s, row) reads groups [s GS, (s + 1) GS) of its row
// (GS = ceil(V / 8 / P)) and writes that slice's maximum, the lowest index
// holding it and, for rows without filters, its double-precision weight
// sum 2^(z c) (no frame).  Rows with filters or bad parameters are left to
// the row's own workgroup (nothing is written for them).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSplitThreads) void split_partial_kernel(SampleArgs a) {
  constexpr int NW = kSplitThreads / kWave;
  __shared__ float s_m[NW];
  __shared__ uint32_t s_arg[NW], s_bad[NW];
  __shared__ double s_sum[NW];
  const int64_t row = blockIdx.y;
  const int sl = blockIdx.x, Pn = a.split_P;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  __shared__ double s_exp2[kWave];
  const arcs_row_params P = a.params[row];
  if (row_param_status(P) != ARCS_ROW_OK) return;
  const bool greedy = P.temperature == 0.0f || P.top_k == 1;
  const bool nofilter = !greedy && !(P.top_k >= 1 && (int64_t)P.top_k < a.V) && !(P.top_p < 1.0f) &&
                        !(P.min_p > 0.0f);
  if (!greedy && !nofilter) return;
  if (nofilter) fill_exp2_table(s_exp2);
  float chi = 0.0f, clo = 0.0f;
  if (nofilter && !temp_coeffs(P.temperature, chi, clo)) return;
  const double c = (double)chi + (double)clo;
  const int ngroups = (int)(a.V / 8);
  const int GS = (ngroups + Pn - 1) / Pn;
  const int g0 = sl * GS, g1 = g0 + GS < ngroups ? g0 + GS : ngroups;
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  float best = -__builtin_inff();
  uint32_t bidx = 0xFFFFFFFFu;
  bool bad = false;
  double sum = 0.0;
  for (int g = g0 + tid; g < g1; g += kSplitThreads) {
    float z[8];
    unpack8(rv[g], z);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (z[e] > best) { best = z[e]; bidx = (uint32_t)(g * 8 + e); }  // ids increase: the first wins
      bad = bad || !(z[e] == z[e]) || z[e] == __builtin_inff();
    }
    if (nofilter) {
      double w8[8];
      sum += group_weights_f64(z, true, c, w8, s_exp2);
    }
  }
  const float wm = dpp_wave_max_f32(best);
  const uint32_t wa = dpp_wave_min_u32(best == wm ? bidx : 0xFFFFFFFFu);
  const double ws = dpp_wave_sum_f64(sum);
  const uint32_t wb = __ballot(bad) != 0 ? 1u : 0u;
  if (lane == 0) { s_m[wid] = wm; s_arg[wid] = wa; s_sum[wid] = ws; s_bad[wid] = wb; }
  __syncthreads();
  if (tid == 0) {
    float m = s_m[0];
    uint32_t anybad = s_bad[0];
    double tot = s_sum[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      m = max2f(m, s_m[w]);
      tot += s_sum[w];
      anybad |= s_bad[w];
    }
    // the lowest index among the waves holding the maximum (a wave's rounds
    // interleave with the others', so any wave may hold the lowest)
    uint32_t arg = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NW; ++w) arg = (s_m[w] == m && s_arg[w] < arg) ? s_arg[w] : arg;
    if (nofilter && !((double)m * c < kF64Span)) anybad = 1u;
    SplitPart r;
    r.m = m;
    r.arg = anybad ? -1 : (int32_t)(arg == 0xFFFFFFFFu ? 0u : arg);
    r.s = tot;
    a.split_parts[row * Pn + sl] = r;
  }
}

// ---------------------------------------------------------------------------
// summary kernel: 512 threads per row (eight waves, two per SIMD, up to 256
// registers each, so the row's loads fill half a thread's registers).  The
// path is written for any workgroup shape kSNT (the file is included inside
// the namespace that sets it).
// ---------------------------------------------------------------------------
namespace sum512 {
constexpr int kSNT = 512;
#include "summary_path.hpp"
}  // namespace sum512
// Rows with active penalties: 1024 threads of 16 rounds each.  Their row is
// latency-bound (history ids, tables, the per-round lookups, the cut), and
// twice the waves halve each thread's share of those steps.
namespace sum1024 {
constexpr int kSNT = 1024;
#include "summary_path.hpp"
}  // namespace sum1024

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
// Rows without filters: the group's weights 2^(z c - O) in double precision
// (fp32 weights carry relative errors near 1e-7, which on rows with heavy
// tokens ahead of long tails of tiny ones moves many CDF boundaries by more
// than the tail tokens' widths).  Pass 1 and the draw both call this.
__device__ __forceinline__ void f32_weights_f64(const float (&z)[4], double c, float negO, double (&w)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = exp2_f64(__builtin_fma((double)z[e], c, (double)negO));
}
__device__ __forceinline__ void f32_round_sum_f64(double* W, int q, double gs) {
  const double s = dpp_wave_sum_f64(gs);
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
// bin bstar.  With `w64` (rows without filters) every weight is the
// double-precision 2^(z c - O) of pass 1.  Returns the id,
// or -1 (uniformly) when the kept mass is not positive.
__device__ __forceinline__ int64_t f32_draw(const u32x4* rv, int ngroups, const double* W, const uint64_t* Wfix,
                                            double u, const KeepCut& cut, int bstar, float eb, float ec, float chi,
                                            float clo, float negO, float cscale, double fscale, bool w64, double c,
                                            Shared& sh, double& S_K) {
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
    double s64[4] = {0.0, 0.0, 0.0, 0.0};
    if (g < ngroups) {
      const u32x4 dd = rv[g];
      float z[4];
      unpack4(dd, z);
      if (w64) {
        f32_weights_f64(z, c, negO, s64);
      } else {
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
    }
    const float gs = (s[0] + s[1]) + (s[2] + s[3]);
    const uint64_t cf = (fx[0] + fx[1]) + (fx[2] + fx[3]);
    const double v = w64 ? ((s64[0] + s64[1]) + (s64[2] + s64[3])) : (double)gs + (double)cf * fscale;
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
        const double we = w64 ? s64[e] : (s[e] > 0.0f ? (double)s[e] : (double)fx[e] * fscale);
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
// above bin 0's per-element limit).  F64 (rows without filters, no
// histogram): the weights in double precision, f32_weights_f64.
template <bool HC, bool HM, bool F64 = false>
__device__ __forceinline__ void f32_pass1(const u32x4* rv, int ngroups, u32x4 (&d0)[kFC], u32x4 (&d1)[kFC],
                                          float chi, float clo, float negO, float ncR, float OR, uint32_t* hc,
                                          uint32_t* hm, double* W1, float& tmax, float& exc, double c = 0.0) {
  static_assert(!F64 || (!HC && !HM), "double weights only for rows without filters");
  const int tid = threadIdx.x;
  auto weigh = [&](const u32x4 (&d)[kFC], int ch) {
#pragma unroll
    for (int r = 0; r < kFC; ++r) {
      const int q = ch * kFC + r;
      if (F64) {
        double g64 = 0.0;
        if (tid < ngroups - q * kFT) {
          float z[4];
          unpack4(d[r], z);
          tmax = max3f(tmax, max2f(z[0], z[1]), max2f(z[2], z[3]));
          double w[4];
          f32_weights_f64(z, c, negO, w);
          g64 = (w[0] + w[1]) + (w[2] + w[3]);
        }
        f32_round_sum_f64(W1, q, g64);
        continue;
      }
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
  // rows under the wide tie rule run on the general pipeline
  if ((P.flags & ARCS_ROW_TIES_WIDE) && (kon || pon)) return false;
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
  else if (nofilter) f32_pass1<false, false, true>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc, c);
  else f32_pass1<false, false>(rv, ngroups, d0, d1, chi, clo, negO, ncR, OR, hc, hm, W1, tmax, exc);
  if (kwin && tid < ngroups) atomicAdd(&hc[f32_bin(tmax, ncR, OR)], 1u);
  if (hmass) {
    const double we = dpp_wave_sum_f64((double)exc);
    if ((tid & (kWave - 1)) == 0) sh.w_sum[tid / kWave] = we;
  }
  const float m = f32_block_max(tmax, sh.w_max);
  const double S = f32_slot_total(W1);
  if (!(m > -__builtin_inff() && m < __builtin_inff()) || !(S > 0.0 && S < 1e300)) return false;
  // double weights: the maximum's within the exponent range (no loss to subnormals)
  if (nofilter && !((double)m * c - Od < 960.0)) return false;
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
          if (!sum512::large_cut_select<kFT>(sm, sh, nc, 0, kon, kon ? P.top_k - (int)above : 0, pon, need, mon, zt, cut, Lc,
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
                              cut, mode == kF32Cand ? bstar : -1, eb, ec, chi, clo, negO, cscale, fscale,
                              mode == kF32NoFilter, c, sh, S_K);
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
hipError_t launch_one(Kern kernel, bool summary, int threads, const SampleArgs& a, int64_t B, size_t lds,
                      hipStream_t stream, std::atomic<int>& attr_done) {
  if (!attr_done.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sample_lds_bytes(summary, true, summary ? kSummaryMaxV : kMaxPenVocab));
    if (e != hipSuccess) return e;
    attr_done.store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)B), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

// Rows the sampling kernel handed over (out_ids marked) in a launch with a
// long-history workspace: their penalties in binary32 in the row's slice of
// the workspace, for the general kernel to sample with no penalties.  The
// slice first counts each id's occurrences in the history (atomics in device
// memory), then every element becomes its penalised value (the same binary32
// sequence as the tables' path) or keeps its raw value; an active DRY record
// then lowers the ids its repeat lengths reach, the lengths gathered per id
// in an LDS hash of the window's ids (at most ARCS_DRY_MAX_WINDOW of them, in
// twice as many slots).  Other rows exit at once.
constexpr int kLongNT = 512;
constexpr int kDryHashSlots = 2 * ARCS_DRY_MAX_WINDOW;
static_assert((kDryHashSlots & (kDryHashSlots - 1)) == 0, "hash slots: a power of two");
template <bool BF16>
__global__ __launch_bounds__(kLongNT) void long_history_prep_kernel(SampleArgs a) {
  __shared__ uint32_t win[ARCS_DRY_MAX_WINDOW];
  __shared__ uint32_t hkey[kDryHashSlots];
  __shared__ uint32_t hlen[kDryHashSlots];
  constexpr uint32_t kEmpty = 0xFFFFFFFFu, kBreak = 0xFFFFFFFFu;
  const int64_t row = blockIdx.x;
  if (a.out_ids[row] != kDeferredId) return;
  const int tid = threadIdx.x;
  const int64_t V = a.V;
  uint32_t* cnt = (uint32_t*)(a.long_ws + row * V);
  float* zc = a.long_ws + row * V;
  const arcs_row_params P = a.params[row];
  PenCtx pc;
  set_penalty_values(pc, P);
  const int64_t h0 = a.hist_offsets[row], h1 = a.hist_offsets[row + 1];
  for (int64_t i = tid; i < V; i += kLongNT) cnt[i] = 0u;
  __syncthreads();
  for (int64_t i = h0 + tid; i < h1; i += kLongNT) {
    const int32_t id = a.hist_ids[i];
    if (id >= 0 && (int64_t)id < V) atomicAdd(&cnt[id], 1u);
  }
  __syncthreads();
  const char* rowp = (const char*)a.logits + row * a.stride * (BF16 ? 2 : 4);
  for (int64_t i = tid; i < V; i += kLongNT) {
    const uint32_t c = cnt[i];
    const float raw = BF16 ? bf16_to_f32(((const uint16_t*)rowp)[i]) : ((const float*)rowp)[i];
    zc[i] = c != 0u ? penalize(canon_nan(raw), c, pc) : raw;
  }
  bool dry_on = false;
  (void)dry_status(a, row, dry_on);  // (the record was validated by the sampling kernel)
  if (!dry_on) return;
  const arcs_dry_params D = a.dry[row];
  int64_t N = h1 - h0;
  if (D.range > 0 && (int64_t)D.range < N) N = D.range;
  if (N > ARCS_DRY_MAX_WINDOW) N = ARCS_DRY_MAX_WINDOW;
  const int64_t s0 = h1 - N;
  for (int64_t i = tid; i < N; i += kLongNT) {
    const int32_t id = a.hist_ids[s0 + i];
    bool brk = id < 0 || (int64_t)id >= V;
    for (int k = 0; k < a.n_breakers && !brk; ++k) brk = a.dry_breakers[k] == id;
    win[i] = brk ? kBreak : (uint32_t)id;
  }
  for (int k = tid; k < kDryHashSlots; k += kLongNT) { hkey[k] = kEmpty; hlen[k] = 0u; }
  __syncthreads();  // also orders the penalised values above before the DRY updates below
  for (int64_t j = 1 + tid; j < N; j += kLongNT) {
    const uint32_t t = win[j];
    if (t == kBreak) continue;
    int64_t n = 0;
    while (n < j) {
      const uint32_t x = win[j - 1 - n];
      if (x == kBreak || x != win[N - 1 - n]) break;
      ++n;
    }
    if (n == 0) continue;
    uint32_t h = (t * 2654435761u) >> 20 & (kDryHashSlots - 1);  // Knuth's multiplicative hash
    for (;;) {
      const uint32_t old = atomicCAS(&hkey[h], kEmpty, t);
      if (old == kEmpty || old == t) {
        atomicMax(&hlen[h], (uint32_t)n);
        break;
      }
      h = (h + 1u) & (kDryHashSlots - 1);
    }
  }
  __syncthreads();
  const float base = D.base, mult = D.multiplier;
  for (int k = tid; k < kDryHashSlots; k += kLongNT) {
    const uint32_t t = hkey[k], n = hlen[k];
    if (t == kEmpty || n < (uint32_t)D.allowed_length) continue;
    float v = 1.0f;
    for (uint32_t i = (uint32_t)D.allowed_length; i < n; ++i) {
      v = v * base;
      if (!__builtin_isfinite(v)) break;
    }
    zc[t] = zc[t] - mult * v;
  }
}

hipError_t launch_sample_rows(const SampleArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream);

hipError_t launch_sample(const SampleArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream) {
  hipError_t e = launch_sample_rows(a, dtype, B, vec, stream);
  if (e != hipSuccess || a.long_ws == nullptr) return e;
  if (dtype == ARCS_DTYPE_BF16) hipLaunchKernelGGL(long_history_prep_kernel<true>, dim3((unsigned)B), dim3(kLongNT), 0, stream, a);
  else hipLaunchKernelGGL(long_history_prep_kernel<false>, dim3((unsigned)B), dim3(kLongNT), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the handed-over rows from their binary32 copies, penalties done
  SampleArgs g = a;
  g.logits = a.long_ws;
  g.stride = a.V;
  g.hist_ids = nullptr;
  g.hist_offsets = nullptr;
  g.dry = nullptr;
  g.pen_tables = 0;
  g.bitmap_words = 0;
  g.split_parts = nullptr;
  g.split_P = 0;
  g.long_ws = nullptr;
  g.deferred_only = 1;
  static std::atomic<int> done[2];
  const size_t lds = sample_lds_bytes(false, false, a.V);
  return a.V % 4 == 0 ? launch_one(sample_kernel<false, true, false>, false, kNT, g, B, lds, stream, done[0])
                      : launch_one(sample_kernel<false, false, false>, false, kNT, g, B, lds, stream, done[1]);
}

hipError_t launch_sample_rows(const SampleArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream) {
  const bool pen = a.pen_tables != 0;
  static std::atomic<int> done[10];
  if (dtype == ARCS_DTYPE_BF16 && vec && a.V <= kSummaryMaxV && a.V % 8 == 0) {
    const size_t lds = sample_lds_bytes(true, pen, a.V);
    if (a.split_parts != nullptr) {
      if (pen || a.split_P < 1 || a.split_P > kSplitMaxP || B > kSplitMaxB) return hipErrorInvalidValue;
      hipLaunchKernelGGL(split_partial_kernel, dim3((unsigned)a.split_P, (unsigned)B), dim3(kSplitThreads), 0,
                         stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return pen ? launch_one(sum1024::sample_summary_kernel<true>, true, sum1024::kSNT, a, B, lds, stream, done[0])
               : launch_one(sum512::sample_summary_kernel<false>, true, sum512::kSNT, a, B, lds, stream, done[1]);
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
    return launch_one(sample_kernel<false, true, false>, false, kNT, g, B, sample_lds_bytes(false, false, a.V), stream,
                      done[7]);
  }
  const size_t lds = sample_lds_bytes(false, pen, a.V);
  if (dtype == ARCS_DTYPE_BF16) {
    if (vec)
      return pen ? launch_one(sample_kernel<true, true, true>, false, kNT, a, B, lds, stream, done[2])
                 : launch_one(sample_kernel<true, true, false>, false, kNT, a, B, lds, stream, done[3]);
    return pen ? launch_one(sample_kernel<true, false, true>, false, kNT, a, B, lds, stream, done[4])
               : launch_one(sample_kernel<true, false, false>, false, kNT, a, B, lds, stream, done[5]);
  }
  if (vec)
    return pen ? launch_one(sample_kernel<false, true, true>, false, kNT, a, B, lds, stream, done[6])
               : launch_one(sample_kernel<false, true, false>, false, kNT, a, B, lds, stream, done[7]);
  return pen ? launch_one(sample_kernel<false, false, true>, false, kNT, a, B, lds, stream, done[8])
             : launch_one(sample_kernel<false, false, false>, false, kNT, a, B, lds, stream, done[9]);
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
