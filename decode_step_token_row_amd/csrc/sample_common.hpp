// Device code shared by the sampling kernels: parameter checks, LDS
// penalty tables, element decoding, fixed-point weights, block primitives and
// the general streaming row pipeline (used on its own for fp32 rows, rows that
// are not 16-byte aligned and vocabularies too large to keep a bf16 row in
// registers, and as the exact fallback of the register-resident path).
#pragma once

#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace arcs {


constexpr int kNT = 1024;
constexpr int kNW = kNT / kWave;
constexpr int kMaxDistinct = ARCS_MAX_HISTORY;  // distinct history ids per row
constexpr int kMaxBins = 2048;
constexpr int kTileUnroll = 4;
constexpr int kCandCap = 4096;                 // LDS candidates of the summary path
constexpr int kMaxGroups = 16384;              // summary path: V <= 8 * kMaxGroups
constexpr int kSmallSort = 64;                 // candidate sets up to this size are handled by one wave
constexpr int kBins = 256;                     // summary path: bound histogram bins
// Start of dynamic LDS ("union area"), used differently by the two paths:
//   general path: radix histograms, counts [kMaxBins] u32 + masses [kMaxBins] u64;
//   summary path: one f32 per group of the row, [kMaxGroups] (group j at
//     j): its maximum (penalised filter rows) or its masked weight sum (min-p
//     rows with many candidates), or for rows without filters each wave's
//     double-precision weight total of each round; candidates (keys u64,
//     weights f32) [kCandCap]; a bound histogram (counts u32, masses f32)
//     [kBins]; a sorted copy of small candidate sets.
constexpr size_t kUnionGeneric = (size_t)kMaxBins * 12;
constexpr size_t kOffTsum = 0;
constexpr size_t kOffCand = kOffTsum + (size_t)kMaxGroups * 4;
constexpr size_t kOffHist = kOffCand + (size_t)kCandCap * 12;
constexpr size_t kOffSort = kOffHist + (size_t)kBins * 8;
constexpr size_t kUnionSummary = kOffSort + (size_t)kSmallSort * 12;
static_assert(kOffCand % 16 == 0 && kOffHist % 16 == 0 && kOffSort % 16 == 0,
              "summary LDS layout");
static_assert((size_t)kCandCap * 12 >= (size_t)kMaxDistinct * 4, "the candidate area also holds the build-time counts");
constexpr int64_t kMaxPenVocab = ARCS_MAX_PENALTY_VOCAB;

// Dynamic LDS layout.
struct Smem {
  uint32_t* hcnt;      // [kMaxBins]               (general path)
  uint64_t* hmass;     // [kMaxBins]               (general path)
  float* tsum;         // [kMaxGroups] group weight sums or maxima (summary path)
  uint64_t* ckey;      // [kCandCap] candidate sort keys   (summary path)
  float* cw;           // [kCandCap] candidate weights     (summary path)
  uint32_t* bcnt;      // [kBins] bound histogram counts   (summary path)
  float* bmass;        // [kBins] bound histogram masses   (summary path)
  uint64_t* skey;      // [kSmallSort] rank-sorted keys    (summary path)
  float* sw;           // [kSmallSort] rank-sorted weights (summary path)
  // penalty tables: history ids as a bitmap over V, the number of set bits
  // before each bitmap word, and per distinct id (in id order) its
  // occurrence count and its penalised logit
  uint32_t* bitmap;    // [bitmap_words]
  uint16_t* wprefix;   // [bitmap_words]
  uint32_t* pcount;    // [kMaxDistinct]
  float* zpen;         // [kMaxDistinct]
};

__host__ __device__ inline size_t pen_prefix_bytes(uint32_t bitmap_words) { return ((size_t)bitmap_words * 2 + 15) / 16 * 16; }

// The penalty tables follow the union area of the kernel's path: the general
// kernel keeps per distinct id its count and its penalised logit; the summary
// kernel keeps only the counts (its pass penalises each history id from its
// own logit and count).
inline size_t sample_lds_bytes(bool summary, bool pen_tables, int64_t V) {
  size_t b = summary ? kUnionSummary : kUnionGeneric;
  if (pen_tables) {
    const uint32_t bw = (uint32_t)((V + 31) / 32);
    b += (size_t)bw * 4 + pen_prefix_bytes(bw) + (size_t)kMaxDistinct * (summary ? 4 : 8);
  }
  return b;
}

struct PenCtx {
  bool on;
  bool rep_on;
  float pres, freq, rep;   // a factor or term that is off holds its neutral value (set_penalty_values)
  const uint32_t* bitmap;
  const uint16_t* wprefix;
  const float* zpen;       // general path: penalised logit per distinct id
  const uint32_t* pcount;  // summary path: occurrence count per distinct id
  uint32_t hmask;          // summary path: bit q set when this thread's group of round q holds a history id
  bool dry_on;             // the row's DRY record is active (its rows run on the general pipeline)
};

// Rank of a history id among the row's distinct history ids (id order).
__device__ __forceinline__ uint32_t pen_rank(uint32_t id, const uint32_t* bitmap, const uint16_t* wprefix) {
  const uint32_t w = id >> 5;
  return (uint32_t)wprefix[w] + (uint32_t)__builtin_popcount(bitmap[w] & ((1u << (id & 31)) - 1u));
}

// The row's penalty values.  One that is off is stored as its neutral value:
// a repetition factor of 1 (z / 1 and z * 1 are z), frequency and presence
// terms of +0 (z - (+0) is z for every binary32 z, -0 and the infinities
// included).  The penalty then runs the same three steps on every row, with
// no branch, and gives the values of the steps it would otherwise skip.
__device__ __forceinline__ void set_penalty_values(PenCtx& pc, const arcs_row_params& P) {
  pc.rep_on = !(P.repetition == 1.0f || P.repetition == 0.0f);
  pc.rep = pc.rep_on ? P.repetition : 1.0f;
  pc.freq = P.frequency != 0.0f ? P.frequency : 0.0f;
  pc.pres = P.presence != 0.0f ? P.presence : 0.0f;
}

// Penalised logit of an id seen c times (z already canonical: no NaN):
// repetition (divide positive logits, multiply the others), then frequency,
// then presence, each an exact binary32 operation (no FMA).
__device__ __forceinline__ float penalize(float z, uint32_t c, const PenCtx& pc) {
  z = (z > 0.0f) ? z / pc.rep : z * pc.rep;
  z = z - pc.freq * (float)c;
  z = z - pc.pres;
  return z;
}

// Penalised values of the history ids in the EPL-aligned group at g0.
template <int EPL>
__device__ __forceinline__ void apply_penalties(float* z, int64_t g0, int n, const PenCtx& pc) {
  const uint32_t w = (uint32_t)(g0 >> 5), sh = (uint32_t)(g0 & 31);
  const uint32_t word = pc.bitmap[w];
  uint32_t bits = (word >> sh) & ((1u << EPL) - 1u);
  if (n < EPL) bits &= (1u << n) - 1u;
  if (bits) {
    const uint32_t base = (uint32_t)pc.wprefix[w] + (uint32_t)__builtin_popcount(word & ((1u << sh) - 1u));
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if ((bits >> e) & 1u) z[e] = pc.zpen[base + (uint32_t)__builtin_popcount(bits & ((1u << e) - 1u))];
  }
}

// Element group of one thread in one tile: EPL consecutive ids starting at a
// multiple of EPL.  Raw load first (so several tiles' loads can be in flight),
// decode later.
template <bool BF16>
struct Group {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int EPL = 16 / ES;
  u32x4 raw;
  int n;  // valid elements (0 when the group lies past V)
};

template <bool BF16, bool VEC>
__device__ __forceinline__ void load_group(const char* rowp, int64_t V, int64_t g0, Group<BF16>& g) {
  constexpr int EPL = Group<BF16>::EPL;
  if (g0 >= V) { g.n = 0; return; }
  int64_t rem = V - g0;
  g.n = rem < EPL ? (int)rem : EPL;
  if (VEC && g.n == EPL) {
    g.raw = *(const u32x4*)(rowp + g0 * Group<BF16>::ES);
  } else {
    u32x4 r = {0u, 0u, 0u, 0u};
    if (BF16) {
      const uint16_t* p = (const uint16_t*)rowp + g0;
      uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int e = 0; e < g.n; ++e) h[e] = p[e];
      r.x = h[0] | (h[1] << 16); r.y = h[2] | (h[3] << 16);
      r.z = h[4] | (h[5] << 16); r.w = h[6] | (h[7] << 16);
    } else {
      const uint32_t* p = (const uint32_t*)rowp + g0;
      uint32_t h[4] = {0, 0, 0, 0};
      for (int e = 0; e < g.n; ++e) h[e] = p[e];
      r.x = h[0]; r.y = h[1]; r.z = h[2]; r.w = h[3];
    }
    g.raw = r;
  }
}

// Decode a group into penalised float32 values z' (NaN -> -inf).
template <bool BF16>
__device__ __forceinline__ void decode_group(const Group<BF16>& g, int64_t g0, const PenCtx& pc,
                                             float (&z)[Group<BF16>::EPL]) {
  if (BF16) {
    z[0] = bf16_lo(g.raw.x); z[1] = bf16_hi(g.raw.x);
    z[2] = bf16_lo(g.raw.y); z[3] = bf16_hi(g.raw.y);
    z[4] = bf16_lo(g.raw.z); z[5] = bf16_hi(g.raw.z);
    z[6] = bf16_lo(g.raw.w); z[7] = bf16_hi(g.raw.w);
  } else {
    z[0] = __uint_as_float(g.raw.x); z[1] = __uint_as_float(g.raw.y);
    z[2] = __uint_as_float(g.raw.z); z[3] = __uint_as_float(g.raw.w);
  }
#pragma unroll
  for (int e = 0; e < Group<BF16>::EPL; ++e) z[e] = canon_nan(z[e]);
  if (pc.on && g.n > 0) apply_penalties<Group<BF16>::EPL>(z, g0, g.n, pc);
}

// Weight of a value relative to the row max m: exp((z-m)/T) as
// exp2(d * log2(e)/T) with the coefficient split in two floats; 1 at the
// max itself (also for +inf rows).
struct WeightCtx {
  float m, chi, clo;
  bool inf_row;
  bool w64;   // rows without filters: weights in double precision
  double c;   // log2(e) / T
};
__device__ __forceinline__ float weight(float z, const WeightCtx& wc) {
  if (wc.inf_row) return z == wc.m ? 1.0f : 0.0f;
  float d = z - wc.m;
  d = d < -FLT_MAX ? -FLT_MAX : d;
  float y = __builtin_fmaf(d, wc.chi, d * wc.clo);
  float w = __builtin_amdgcn_exp2f(y);
  return z == wc.m ? 1.0f : w;
}

// The weight in fixed point 2^-F.  Rows without filters compute it in double
// precision, exp2((z - m) c): fp32 weights carry relative errors near 1e-7,
// which on rows with heavy tokens ahead of long tails of tiny ones moves
// many CDF boundaries by more than the tail tokens' widths.
__device__ __forceinline__ uint64_t weight_fixed(float z, const WeightCtx& wc, float scale) {
  if (!wc.w64 || wc.inf_row) return to_fixed(weight(z, wc), scale);
  const double w = z == wc.m ? 1.0 : exp2_f64(((double)z - (double)wc.m) * wc.c);
  return (uint64_t)(w * (double)scale);
}

// ceil(S * p) for p in (0, 1), exact (128-bit product).
__device__ __forceinline__ uint64_t ceil_mul_frac(uint64_t S, float p) {
  uint32_t b = __float_as_uint(p);
  int e = (int)((b >> 23) & 0xFF);
  uint64_t mant = b & 0x7FFFFF;
  int sh;
  if (e == 0) { sh = 149; } else { mant |= 0x800000; sh = 150 - e; }
  // value = mant * 2^-sh, sh >= 24 here because p < 1
  uint64_t lo = S * mant, hi = __umul64hi(S, mant);
  uint64_t q, rem;
  if (sh >= 128) { q = 0; rem = hi | lo; }
  else if (sh >= 64) { int s2 = sh - 64; q = s2 ? (hi >> s2) : hi; rem = lo | (s2 ? (hi & ((1ull << s2) - 1)) : 0); }
  else { q = (lo >> sh) | (hi << (64 - sh)); rem = lo & ((1ull << sh) - 1); }
  return q + (rem != 0);
}

// ---------------------------------------------------------------------------
// block primitives (kNT threads)
// ---------------------------------------------------------------------------
struct BlockScratch {
  uint64_t u64[kNW];
  float f32[kNW];
  int32_t i32[kNW];
  uint32_t u32[kNW];
};

template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, BlockScratch& bs) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_sum_u64(v);
  __syncthreads();
  if (lane == 0) bs.u64[wid] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < (NT / kWave); ++w) t += bs.u64[w];
  return t;
}

// inclusive block scan; also returns the block total
template <int NT>
__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, BlockScratch& bs, uint64_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_incl_scan_u64(v, lane);
  __syncthreads();
  if (lane == kWave - 1) bs.u64[wid] = v;
  __syncthreads();
  uint64_t off = 0, t = 0;
#pragma unroll
  for (int w = 0; w < (NT / kWave); ++w) {
    uint64_t x = bs.u64[w];
    off += (w < wid) ? x : 0;
    t += x;
  }
  total = t;
  return v + off;
}

// A workgroup barrier that orders LDS only: it waits for the wave's LDS
// operations, not for its outstanding global loads (which __syncthreads
// would drain), so row loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_incl_scan_u32(uint32_t v, BlockScratch& bs, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_incl_scan_u32(v, lane);
  if (LDS_ONLY) lds_barrier(); else __syncthreads();
  if (lane == kWave - 1) bs.u32[wid] = v;
  if (LDS_ONLY) lds_barrier(); else __syncthreads();
  uint32_t off = 0, t = 0;
#pragma unroll
  for (int w = 0; w < (NT / kWave); ++w) {
    uint32_t x = bs.u32[w];
    off += (w < wid) ? x : 0;
    t += x;
  }
  total = t;
  return v + off;
}

// Visit every element of the row once, in tiles: tile t holds ids
// [t*kNT*EPL, (t+1)*kNT*EPL) and thread i the EPL ids starting at
// (t*kNT + i)*EPL.  f(g0, z[], n) is called for this thread's group of each
// tile (n may be 0 past the end; f must then do nothing).
template <int NT, bool BF16, bool VEC, class Fn>
__device__ __forceinline__ void for_each_group(const char* rowp, int64_t V, const PenCtx& pc, Fn&& f) {
  constexpr int EPL = Group<BF16>::EPL;
  const int64_t tile_elems = (int64_t)NT * EPL;
  const int64_t ntiles = (V + tile_elems - 1) / tile_elems;
  for (int64_t t0 = 0; t0 < ntiles; t0 += kTileUnroll) {
    Group<BF16> g[kTileUnroll];
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      int64_t g0 = ((t0 + u) * NT + threadIdx.x) * EPL;
      load_group<BF16, VEC>(rowp, V, g0, g[u]);
    }
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      int64_t g0 = ((t0 + u) * NT + threadIdx.x) * EPL;
      if (g[u].n > 0) {
        float z[EPL];
        decode_group<BF16>(g[u], g0, pc, z);
        f(g0, z, g[u].n);
      }
    }
  }
}

// The kept predicate after the cutoff.
struct KeptCtx {
  int mode;            // 0 all kept, 1 key >= floor, 2 key > theta or (== theta and id <= idx_star)
  uint32_t floor_key;
  uint32_t theta;
  int64_t idx_star;    // INT64_MAX when all ties at theta are kept
};
__device__ __forceinline__ bool is_kept(float z, int64_t idx, const KeptCtx& kc) {
  if (kc.mode == 0) return true;
  uint32_t k = ord_key(z);
  if (kc.mode == 1) return k >= kc.floor_key;
  return k > kc.theta || (k == kc.theta && idx <= kc.idx_star);
}


// Block-shared scalars of one row.  u64 slots: 0-1 pass A, 2 min-p floor,
// 3-6 radix levels, 7 tie split, 8 draw, 9 debug stats, 10-15 resident path.
// Carve the dynamic LDS block: the union area (the general path uses its
// first kUnionGeneric bytes, the summary path up to kUnionSummary), and the
// penalty tables after the union area of the kernel's path.
__device__ __forceinline__ Smem carve_smem(unsigned char* raw, bool summary, uint32_t bitmap_words) {
  Smem sm;
  sm.hcnt = (uint32_t*)raw;
  sm.hmass = (uint64_t*)(raw + (size_t)kMaxBins * 4);
  sm.tsum = (float*)(raw + kOffTsum);
  sm.ckey = (uint64_t*)(raw + kOffCand);
  sm.cw = (float*)(raw + kOffCand + (size_t)kCandCap * 8);
  sm.bcnt = (uint32_t*)(raw + kOffHist);
  sm.bmass = (float*)(raw + kOffHist + (size_t)kBins * 4);
  sm.skey = (uint64_t*)(raw + kOffSort);
  sm.sw = (float*)(raw + kOffSort + (size_t)kSmallSort * 8);
  unsigned char* pen_base = raw + (summary ? kUnionSummary : kUnionGeneric);
  sm.bitmap = (uint32_t*)pen_base;
  sm.wprefix = (uint16_t*)(pen_base + (size_t)bitmap_words * 4);
  unsigned char* after = pen_base + (size_t)bitmap_words * 4 + pen_prefix_bytes(bitmap_words);
  if (summary) {
    // counts kept for the whole row (the pass penalises from them); the
    // penalised logits only for a row handed to the general pipeline, in the
    // candidate area (free then)
    sm.pcount = (uint32_t*)after;
    sm.zpen = (float*)(raw + kOffCand);
  } else {
    sm.pcount = (uint32_t*)after;
    sm.zpen = (float*)(after + (size_t)kMaxDistinct * 4);
  }
  return sm;
}

struct Shared {
  BlockScratch bs;
  int32_t i32[8];
  uint64_t u64[16];
  float f32[8];
  double f64[kNW + 4];
  // summary path, one record per wave: maximum, reference exponent (negated),
  // weight total, kept count (debug outputs), argmax candidate, flags
  float w_max[kNW];
  float w_negk[kNW];
  double w_sum[kNW];
  uint32_t w_cnt[kNW];
  uint32_t w_arg[kNW];
  uint32_t w_flags[kNW];
  double rtot[kNW];      // summary path, no-filter rows: weight per group round
  // summary path: the row's values, computed by one wave and broadcast
  float r_m, r_negks, r_zt, r_zc;
  double r_S, r_Pm;
  int32_t r_mode;
  uint32_t r_arg;
};

// Per-row parameter validation: ARCS_ROW_OK or the row's error code.
__device__ __forceinline__ int row_param_status(const arcs_row_params& P) {
  if (!(P.temperature >= 0.0f)) return ARCS_ROW_BAD_TEMPERATURE;
  if (!(P.top_p > 0.0f)) return ARCS_ROW_BAD_TOP_P;
  if (!(P.min_p >= 0.0f && P.min_p <= 1.0f)) return ARCS_ROW_BAD_MIN_P;
  if (!(__builtin_isfinite(P.presence) && __builtin_isfinite(P.frequency) && __builtin_isfinite(P.repetition)) ||
      P.repetition < 0.0f)
    return ARCS_ROW_BAD_PENALTY;
  if ((P.flags & ~ARCS_ROW_TIES_WIDE) != 0) return ARCS_ROW_BAD_FLAGS;
  return ARCS_ROW_OK;
}

// The row's DRY record (rows with history arrays only): ARCS_ROW_OK or
// ARCS_ROW_BAD_PENALTY; `on` when its multiplier is not 0.
__device__ __forceinline__ int dry_status(const SampleArgs& a, int64_t row, bool& on) {
  on = false;
  if (a.dry == nullptr || a.hist_ids == nullptr) return ARCS_ROW_OK;
  const arcs_dry_params D = a.dry[row];
  if (!(__builtin_isfinite(D.multiplier) && D.multiplier >= 0.0f && __builtin_isfinite(D.base) && D.base > 0.0f) ||
      D.allowed_length < 1 || D.range < 0)
    return ARCS_ROW_BAD_PENALTY;
  on = D.multiplier != 0.0f;
  return ARCS_ROW_OK;
}

// The DRY penalty folded into the penalised logits zpen[rank] (built
// already).  Over the last min(range, ARCS_DRY_MAX_WINDOW) history ids, in
// `win` (ids outside [0, V) and sequence breakers become a marker that
// matches nothing), each position j >= 1 extends the window's tail backwards
// from j - 1 while the ids agree: that length n is a repeat the token at j
// would continue; per distinct id the longest (LDS atomic max into `len`,
// kMaxDistinct entries), then zpen -= multiplier * base^(n - allowed_length)
// for n >= allowed_length.  The power is a product of n - allowed_length
// binary32 multiplications.  All NT threads call it; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void apply_dry(const SampleArgs& a, int64_t row, int64_t h0, int64_t h1, const Smem& sm,
                                          uint32_t* win, uint32_t* len) {
  constexpr uint32_t kBreak = 0xFFFFFFFFu;
  const int tid = threadIdx.x;
  const arcs_dry_params D = a.dry[row];
  int64_t N = h1 - h0;
  if (D.range > 0 && (int64_t)D.range < N) N = D.range;
  if (N > ARCS_DRY_MAX_WINDOW) N = ARCS_DRY_MAX_WINDOW;
  const int64_t s0 = h1 - N;
  for (int64_t i = tid; i < N; i += NT) {
    const int32_t id = a.hist_ids[s0 + i];
    bool brk = id < 0 || (int64_t)id >= a.V;
    for (int k = 0; k < a.n_breakers && !brk; ++k) brk = a.dry_breakers[k] == id;
    win[i] = brk ? kBreak : (uint32_t)id;
  }
  for (int r = tid; r < kMaxDistinct; r += NT) len[r] = 0u;
  __syncthreads();
  for (int64_t j = 1 + tid; j < N; j += NT) {
    const uint32_t t = win[j];
    if (t == kBreak) continue;
    int64_t n = 0;
    while (n < j) {
      const uint32_t x = win[j - 1 - n];
      if (x == kBreak || x != win[N - 1 - n]) break;
      ++n;
    }
    if (n > 0) atomicMax(&len[pen_rank(t, sm.bitmap, sm.wprefix)], (uint32_t)n);
  }
  __syncthreads();
  const float base = D.base, mult = D.multiplier;
  for (int r = tid; r < kMaxDistinct; r += NT) {
    const uint32_t n = len[r];
    if (n >= (uint32_t)D.allowed_length) {
      float v = 1.0f;
      for (uint32_t k = (uint32_t)D.allowed_length; k < n; ++k) {
        v = v * base;
        if (!__builtin_isfinite(v)) break;
      }
      sm.zpen[r] = sm.zpen[r] - mult * v;
    }
  }
  __syncthreads();
}

// A row whose active penalties the LDS tables cannot hold (more distinct
// history ids than kMaxDistinct, or V above the penalty vocabulary) in a
// launch with a long-history workspace: handed to the workspace path (its
// out_ids entry marked, nothing else written), never stored as a status.
constexpr int kStatusDeferLong = -100;

// A row whose parameters or history failed: -1, its status, zeroed debug outputs.
template <int NT>
__device__ __forceinline__ void write_row_failure(const SampleArgs& a, int64_t row, int status) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    a.out_ids[row] = -1;
    if (a.out_status) a.out_status[row] = status;
    if (a.stats) {
      arcs_row_stats st = {};
      st.id = -1; st.argmax = -1; st.status = status;
      a.stats[row] = st;
    }
  }
  if (a.out_probs)
    for (int64_t i = tid; i < a.V; i += NT) a.out_probs[row * a.V + i] = 0.0f;
}

// Parameter validation and penalty tables.  Returns false when the row is
// finished (invalid parameters: out_ids = -1 and the status written).
//
// Penalty tables (only when the row has active penalties and history ids):
// a bitmap of the history ids over [0, V), the number of distinct ids before
// each bitmap word (a block scan of popcounts), and per distinct id its count
// and its penalised logit, computed once here from the raw logit.  Looking
// up an element is then one popcount and one LDS read.
// NOHIST: a launch without history arrays (the caller guarantees
// a.hist_ids == NULL, and with it no DRY record is read): nothing here reads
// device memory, so no wait here can drain row loads already in flight.
template <int NT, bool BF16, bool PEN, bool NOHIST = false>
__device__ __forceinline__ bool row_prologue(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh,
                                             arcs_row_params& P, PenCtx& pc, uint32_t& path) {
  const int tid = threadIdx.x;
  const int64_t V = a.V;
  // ---- 0. parameters (P holds the row's record, loaded by the caller) ------
  int status = row_param_status(P);
  bool dry_on = false;
  if (!NOHIST && status == ARCS_ROW_OK) status = dry_status(a, row, dry_on);

  pc.on = false;
  pc.dry_on = false;
  set_penalty_values(pc, P);
  pc.bitmap = sm.bitmap; pc.wprefix = sm.wprefix; pc.zpen = sm.zpen; pc.pcount = sm.pcount;
  int64_t h0 = 0, h1 = 0;
  if (!NOHIST && status == ARCS_ROW_OK && a.hist_ids != nullptr) {
    const bool active = P.presence != 0.0f || P.frequency != 0.0f || pc.rep_on || dry_on;
    h0 = a.hist_offsets[row];
    h1 = a.hist_offsets[row + 1];
    if (active && h1 > h0) {
      if (!PEN) status = a.long_ws != nullptr ? kStatusDeferLong : ARCS_ROW_VOCAB_TOO_LARGE;
      else { pc.on = true; pc.dry_on = dry_on; }
    }
  }

  if (PEN && pc.on) {
    const uint32_t bw = a.bitmap_words;
    for (uint32_t i = tid; i < bw; i += NT) sm.bitmap[i] = 0u;
    __syncthreads();
    for (int64_t i = h0 + tid; i < h1; i += NT) {
      const int32_t id = a.hist_ids[i];
      if (id >= 0 && (int64_t)id < V) atomicOr(&sm.bitmap[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    // distinct ids before each word: contiguous chunks of words per thread
    const uint32_t per = (bw + NT - 1) / NT;
    const uint32_t w0 = tid * per, w1 = (w0 + per < bw) ? w0 + per : bw;
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; ++w) c += (uint32_t)__builtin_popcount(sm.bitmap[w]);
    uint32_t total;
    const uint32_t incl = block_incl_scan_u32<NT>(c, sh.bs, total);
    if (total <= (uint32_t)kMaxDistinct) {
      uint32_t run = incl - c;
      for (uint32_t w = w0; w < w1; ++w) {
        sm.wprefix[w] = (uint16_t)run;
        run += (uint32_t)__builtin_popcount(sm.bitmap[w]);
      }
      for (uint32_t i = tid; i < total; i += NT) sm.pcount[i] = 0u;
      __syncthreads();
      for (int64_t i = h0 + tid; i < h1; i += NT) {
        const int32_t id = a.hist_ids[i];
        if (id >= 0 && (int64_t)id < V) atomicAdd(&sm.pcount[pen_rank((uint32_t)id, sm.bitmap, sm.wprefix)], 1u);
      }
      __syncthreads();
      // every occurrence of an id writes the same penalised value
      const char* rowp = (const char*)a.logits + row * a.stride * (BF16 ? 2 : 4);
      for (int64_t i = h0 + tid; i < h1; i += NT) {
        const int32_t id = a.hist_ids[i];
        if (id >= 0 && (int64_t)id < V) {
          const uint32_t rk = pen_rank((uint32_t)id, sm.bitmap, sm.wprefix);
          const float raw = BF16 ? bf16_to_f32(((const uint16_t*)rowp)[id]) : ((const float*)rowp)[id];
          sm.zpen[rk] = penalize(canon_nan(raw), sm.pcount[rk], pc);
        }
      }
      __syncthreads();
      // the general pipeline's union area is free until pass A: the window
      // (2048 ids) and the per-id repeat lengths (4096) fit it
      static_assert((size_t)kMaxBins * 4 >= (size_t)ARCS_DRY_MAX_WINDOW * 4 &&
                    (size_t)kMaxBins * 8 >= (size_t)kMaxDistinct * 4, "DRY scratch in the union area");
      if (pc.dry_on) apply_dry<NT>(a, row, h0, h1, sm, sm.hcnt, (uint32_t*)sm.hmass);
    } else {
      status = a.long_ws != nullptr ? kStatusDeferLong : ARCS_ROW_HISTORY_TOO_LONG;
      pc.on = false;
    }
  }

  if (status == kStatusDeferLong) {
    if (tid == 0) a.out_ids[row] = kDeferredId;
    return false;
  }
  if (status != ARCS_ROW_OK) {
    write_row_failure<NT>(a, row, status);
    return false;
  }
  path = pc.on ? ARCS_PATH_PENALTY : 0u;
  return true;
}

// The general row pipeline from pass A on (see the file comment of
// sample_kernel.hip).  All threads of the block call it together.
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ void generic_row(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                         const PenCtx& pc, uint32_t path, const Smem& sm, Shared& sh) {
  constexpr int EPL = Group<BF16>::EPL;
  constexpr int ES = Group<BF16>::ES;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t V = a.V;
  const char* rowp = (const char*)a.logits + row * a.stride * ES;
  // ---- 1. pass A: max and first argmax -------------------------------------
  float best = -__builtin_inff();
  int64_t bidx = INT64_MAX;
  for_each_group<NT, BF16, VEC>(rowp, V, pc, [&](int64_t g0, const float* z, int n) {
    for (int e = 0; e < n; ++e)
      if (z[e] > best) { best = z[e]; bidx = g0 + e; }
  });
  {
    float wm = wave_max_f32(best);
    if (lane == 0) sh.bs.f32[wid] = wm;
    if (tid == 0) sh.u64[0] = (uint64_t)INT64_MAX;
    __syncthreads();
    float m = sh.bs.f32[0];
#pragma unroll
    for (int w = 1; w < (NT / kWave); ++w) m = m > sh.bs.f32[w] ? m : sh.bs.f32[w];
    if (best == m && bidx != INT64_MAX) atomicMin((unsigned long long*)&sh.u64[0], (unsigned long long)bidx);
    __syncthreads();
    if (tid == 0) { sh.f32[0] = m; sh.u64[1] = (m == -__builtin_inff()) ? 0 : sh.u64[0]; }
    __syncthreads();
  }
  const float m = sh.f32[0];
  const int64_t argmax = (int64_t)sh.u64[1];

  const bool greedy = P.temperature == 0.0f || P.top_k == 1;
  if (m == -__builtin_inff() || m == __builtin_inff()) path |= ARCS_PATH_SPECIAL;
  if (greedy || m == -__builtin_inff()) {
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
      for (int64_t i = tid; i < V; i += NT) a.out_probs[row * V + i] = (i == argmax) ? 1.0f : 0.0f;
    return;
  }

  // ---- 2. pass B: total fixed-point mass -----------------------------------
  WeightCtx wc;
  {
    double c = 1.4426950408889634 / (double)P.temperature;
    wc.m = m;
    wc.chi = (float)c;
    wc.clo = (float)(c - (double)wc.chi);
    wc.inf_row = (m == __builtin_inff());
    wc.w64 = !(P.top_k >= 1 && (int64_t)P.top_k < V) && !(P.top_p < 1.0f) && !(P.min_p > 0.0f);
    wc.c = c;
  }
  const float scale = a.scale;
  uint64_t my_mass = 0;
  for_each_group<NT, BF16, VEC>(rowp, V, pc, [&](int64_t, const float* z, int n) {
    for (int e = 0; e < n; ++e) my_mass += weight_fixed(z[e], wc, scale);
  });
  const uint64_t S = block_sum_u64<NT>(my_mass, sh.bs);

  // ---- 3. cutoff -------------------------------------------------------------
  const bool kon = P.top_k >= 1 && (int64_t)P.top_k < V;
  const bool pon = P.top_p < 1.0f;
  const bool mon = P.min_p > 0.0f;
  KeptCtx kc;
  kc.mode = 0; kc.floor_key = 0u; kc.theta = 0u; kc.idx_star = INT64_MAX;
  uint64_t S_K = S;
  int64_t L = V;
  if (!kon && !pon && !mon) {
    path |= ARCS_PATH_SORT_SKIP;
  } else {
    path |= ARCS_PATH_CUTOFF;
    // min-p threshold: the smallest float z with ((double)z - m) / T >= ln(min_p).
    if (tid == 0) {
      float zt;
      if (!mon) {
        zt = -__builtin_inff();
      } else if (wc.inf_row) {
        zt = __builtin_inff();
      } else {
        const double lnmp = log((double)P.min_p), T = (double)P.temperature, md = (double)m;
        auto keep = [&](float z) { return ((double)z - md) / T >= lnmp; };
        zt = (float)(md + T * lnmp);
        if (zt < -FLT_MAX) zt = -FLT_MAX;
        if (keep(zt)) {
          for (int it = 0; it < 64; ++it) {
            float dn = key_value(ord_key(zt) - 1u);
            if (!keep(dn)) break;
            zt = dn;
          }
        } else {
          for (int it = 0; it < 64 && !keep(zt); ++it) zt = key_value(ord_key(zt) + 1u);
        }
        if (zt > m) zt = m;
      }
      sh.u64[2] = mon ? ord_key(zt) : 0u;
    }
    __syncthreads();
    const uint32_t floor_key = (uint32_t)sh.u64[2];
    const uint64_t Lk = kon ? (uint64_t)P.top_k : (uint64_t)V;
    const uint64_t Pm = pon ? ceil_mul_frac(S, P.top_p) : ~0ull;

    const bool key16 = BF16 && !pc.on;
    const int nlev = key16 ? 2 : 3;
    uint32_t prefix = 0;
    uint64_t cnt_above = 0, mass_above = 0, cnt_eq = 0, mass_eq = 0;
    bool floor_hit = false;
    for (int lev = 0; lev < nlev; ++lev) {
      const int shf = key16 ? (lev == 0 ? 24 : 16) : (lev == 0 ? 21 : lev == 1 ? 10 : 0);
      const int bits = key16 ? 8 : (lev == 2 ? 10 : 11);
      const int nb = 1 << bits;
      for (int i = tid; i < nb; i += NT) { sm.hcnt[i] = 0u; sm.hmass[i] = 0ull; }
      __syncthreads();
      for_each_group<NT, BF16, VEC>(rowp, V, pc, [&](int64_t, const float* z, int n) {
        for (int e = 0; e < n; ++e) {
          uint32_t k = ord_key(z[e]);
          if (k < floor_key) continue;
          if (lev > 0 && (k >> (shf + bits)) != prefix) continue;
          uint32_t d = (k >> shf) & (uint32_t)(nb - 1);
          atomicAdd(&sm.hcnt[d], 1u);
          atomicAdd((unsigned long long*)&sm.hmass[d], (unsigned long long)to_fixed(weight(z[e], wc), scale));
        }
      });
      __syncthreads();
      // Wave 0 scans the digits from the top: lane l owns digits
      // [nb - (l+1)*per, nb - l*per), visited in descending order.
      if (wid == 0) {
        const int per = nb / kWave;
        const int hi_d = nb - lane * per - 1;
        uint64_t lc = 0, lm = 0;
        for (int j = 0; j < per; ++j) { lc += sm.hcnt[hi_d - j]; lm += sm.hmass[hi_d - j]; }
        uint64_t ic = wave_incl_scan_u64(lc, lane), im = wave_incl_scan_u64(lm, lane);
        uint64_t ec = ic - lc, em = im - lm;
        bool cross = (cnt_above + ic >= Lk) || (pon && mass_above + im >= Pm);
        uint64_t ball = __ballot(cross);
        if (ball == 0) {
          if (lane == kWave - 1) { sh.i32[0] = -1; sh.u64[3] = ic; sh.u64[4] = im; }
        } else {
          int first = __builtin_ctzll(ball);
          if (lane == first) {
            uint64_t c = cnt_above + ec, ms = mass_above + em;
            int dstar = hi_d - per + 1;
            for (int j = 0; j < per; ++j) {
              int d = hi_d - j;
              uint64_t dc = sm.hcnt[d], dm = sm.hmass[d];
              if (c + dc >= Lk || (pon && ms + dm >= Pm)) { dstar = d; break; }
              c += dc; ms += dm;
            }
            sh.i32[0] = dstar; sh.u64[3] = c; sh.u64[4] = ms;
            sh.u64[5] = sm.hcnt[dstar]; sh.u64[6] = sm.hmass[dstar];
          }
        }
      }
      __syncthreads();
      const int dstar = sh.i32[0];
      if (dstar < 0) {  // neither target reached above the min-p floor
        floor_hit = true;
        cnt_above += sh.u64[3];
        mass_above += sh.u64[4];
        break;
      }
      cnt_above = sh.u64[3];
      mass_above = sh.u64[4];
      cnt_eq = sh.u64[5];
      mass_eq = sh.u64[6];
      prefix = (prefix << bits) | (uint32_t)dstar;
      __syncthreads();
    }
    if (floor_hit) {
      path |= ARCS_PATH_MINP_FLOOR;
      kc.mode = 1;
      kc.floor_key = floor_key;
      S_K = mass_above;
      L = (int64_t)cnt_above;
    } else {
      uint32_t theta = key16 ? ((prefix << 16) | ((prefix & 0x8000u) ? 0u : 0xFFFFu)) : prefix;
      const uint64_t Wt = cnt_eq ? mass_eq / cnt_eq : 0;
      uint64_t r = cnt_eq;
      if (kon && Lk - cnt_above < r) r = Lk - cnt_above;
      if (pon && Wt > 0) {
        uint64_t need = Pm > mass_above ? Pm - mass_above : 0;
        uint64_t rp = (need + Wt - 1) / Wt;
        if (rp < 1) rp = 1;
        if (rp < r) r = rp;
      }
      // the wide tie rule keeps every id tied at the cut value
      if (P.flags & ARCS_ROW_TIES_WIDE) r = cnt_eq;
      kc.mode = 2;
      kc.theta = theta;
      S_K = mass_above + r * Wt;
      L = (int64_t)(cnt_above + r);
      if (r < cnt_eq) {
        path |= ARCS_PATH_TIE_SPLIT;
        // find the id of the r-th element (in id order) whose key is theta
        uint32_t running = 0;
        if (tid == 0) sh.u64[7] = (uint64_t)INT64_MAX;
        const int64_t tile_elems = (int64_t)NT * EPL;
        const int64_t ntiles = (V + tile_elems - 1) / tile_elems;
        for (int64_t t = 0; t < ntiles; ++t) {
          const int64_t g0 = (t * NT + tid) * EPL;
          Group<BF16> g;
          load_group<BF16, VEC>(rowp, V, g0, g);
          float z[EPL];
          uint32_t c = 0;
          if (g.n > 0) {
            decode_group<BF16>(g, g0, pc, z);
            for (int e = 0; e < g.n; ++e) c += ord_key(z[e]) == theta;
          }
          uint32_t tot;
          uint32_t incl = block_incl_scan_u32<NT>(c, sh.bs, tot);
          if ((uint64_t)running + tot >= r) {
            uint32_t excl = running + incl - c;
            if (c > 0 && excl < r && (uint64_t)running + incl >= r) {
              uint32_t need = (uint32_t)r - excl, seen = 0;
              for (int e = 0; e < g.n; ++e) {
                if (ord_key(z[e]) == theta && ++seen == need) { sh.u64[7] = (uint64_t)(g0 + e); break; }
              }
            }
            break;
          }
          running += tot;
        }
        __syncthreads();
        kc.idx_star = (int64_t)sh.u64[7];
      }
    }
  }

  // ---- 4. draw ----------------------------------------------------------------
  uint64_t uf;
  double u;
  if (a.uniforms) {
    u = a.uniforms[row];
    double x = u * 0x1p64;
    uf = (x >= 0x1p64) ? ~0ull : (x <= 0.0 ? 0ull : (uint64_t)x);
  } else {
    uint64_t x = splitmix64_counter_output(a.key ? a.key[0] : a.seed, (uint64_t)row, a.key ? a.key[1] : a.step);
    uf = (x >> 11) << 11;
    u = (double)(x >> 11) * 0x1p-53;
  }
  const uint64_t Tfix = __umul64hi(uf, S_K);  // floor(u * S_K) <= S_K - 1
  {
    uint64_t running = 0;
    if (tid == 0) sh.u64[8] = (uint64_t)INT64_MAX;
    const int64_t tile_elems = (int64_t)NT * EPL;
    const int64_t ntiles = (V + tile_elems - 1) / tile_elems;
    for (int64_t t = 0; t < ntiles; ++t) {
      const int64_t g0 = (t * NT + tid) * EPL;
      Group<BF16> g;
      load_group<BF16, VEC>(rowp, V, g0, g);
      float z[EPL];
      uint64_t wv[EPL];
      uint64_t c = 0;
      if (g.n > 0) {
        decode_group<BF16>(g, g0, pc, z);
        for (int e = 0; e < EPL; ++e) {
          wv[e] = (e < g.n && is_kept(z[e], g0 + e, kc)) ? weight_fixed(z[e], wc, scale) : 0ull;
          c += wv[e];
        }
      }
      uint64_t tot;
      uint64_t incl = block_incl_scan_u64<NT>(c, sh.bs, tot);
      if (running + tot > Tfix) {
        uint64_t acc = running + incl - c;
        if (c > 0 && acc <= Tfix && running + incl > Tfix) {
          for (int e = 0; e < g.n; ++e) {
            acc += wv[e];
            if (wv[e] > 0 && acc > Tfix) { sh.u64[8] = (uint64_t)(g0 + e); break; }
          }
        }
        break;
      }
      running += tot;
    }
    __syncthreads();
  }
  const int64_t id = (int64_t)sh.u64[8];

  if (tid == 0) {
    a.out_ids[row] = (int32_t)id;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
  }

  // ---- debug outputs ------------------------------------------------------------
  if (a.stats || a.out_probs) {
    const double inv_sk = 1.0 / ((double)S_K * (double)(1.0f / scale));
    uint32_t kmin = 0xFFFFFFFFu;
    int64_t kmin_idx = -1;
    for_each_group<NT, BF16, VEC>(rowp, V, pc, [&](int64_t g0, const float* z, int n) {
      for (int e = 0; e < n; ++e) {
        bool kept = is_kept(z[e], g0 + e, kc);
        if (a.out_probs)
          a.out_probs[row * V + g0 + e] = kept ? (float)((double)weight(z[e], wc) * inv_sk) : 0.0f;
        if (kept) {
          uint32_t k = ord_key(z[e]);
          if (k < kmin || (k == kmin && g0 + e > kmin_idx)) { kmin = k; kmin_idx = g0 + e; }
        }
      }
    });
    if (a.stats) {
      if (tid == 0) { sh.u64[9] = ~0ull; }
      __syncthreads();
      // order (key asc, idx desc) packed so that the minimum wins
      uint64_t packed = ((uint64_t)kmin << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(kmin_idx < 0 ? 0 : kmin_idx));
      if (kmin_idx >= 0) atomicMin((unsigned long long*)&sh.u64[9], (unsigned long long)packed);
      __syncthreads();
      if (tid == 0) {
        uint64_t pk = sh.u64[9];
        arcs_row_stats st = {};
        st.id = (int32_t)id; st.argmax = (int32_t)argmax; st.kept = (int32_t)L;
        st.cut_index = (int32_t)(0xFFFFFFFFu - (uint32_t)(pk & 0xFFFFFFFFu));
        st.cut_value = key_value((uint32_t)(pk >> 32));
        st.max_logit = m; st.status = 0; st.path = path;
        st.mass_total = (double)S / (double)scale;
        st.mass_kept = (double)S_K / (double)scale;
        st.uniform = u;
        a.stats[row] = st;
      }
    }
  }
}

}  // namespace arcs
