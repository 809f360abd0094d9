// The summary path of the sampler (bf16 rows kept in registers), written
// once for a workgroup of kSNT threads: the file is included inside a
// namespace that defines kSNT (no include guard on purpose), so that the
// kernel exists in more than one workgroup shape.  See sample_kernel.hip for
// what the path computes.

// ---------------------------------------------------------------------------
// summary kernel
// ---------------------------------------------------------------------------
// One workgroup of kSNT threads per row; thread t owns the groups
// q * kSNT + t, kSQ of them, all held in its registers after one load each.
constexpr int kSNW = kSNT / kWave;
constexpr int kSQ = kMaxGroups / kSNT;  // groups per thread
static_assert(kSQ <= 32, "round masks and round codes hold 32 rounds");

// The row's groups owned by this thread: group j = q * kSNT + tid holds ids
// [8j, 8j + 8), so one load instruction of a wave reads 1 KB of contiguous
// logits.  All rounds go through one buffer resource that covers exactly the
// row, with the byte offset of the group in the per-lane offset (which the
// range check covers), so lanes past the row's end read zeros without
// touching memory (their results are discarded).  All kSQ loads are issued
// before any of them is used.
template <int Q0 = 0, int Q1 = kSQ>
__device__ __forceinline__ void issue_row_loads(const u32x4* rv, int ngroups, u32x4 (&d)[kSQ]) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)rv, (short)0, ngroups * 16, 0x00020000);
  // one offset register stepped from round to round (opaque, so that the
  // compiler neither precomputes every round's offset nor keeps them live for
  // a later re-read)
  int voff = (threadIdx.x + Q0 * kSNT) * 16;
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    asm volatile("" : "+v"(voff));
    d[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2 /* nt */));
    voff += kSNT * 16;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The 16 bytes of round qs when qs is the same in every lane of the wave: a
// scalar branch to one copy instead of a select over every round (each case
// opaque, so that the switch is not folded into an indexed read, which would
// move the row's registers to scratch memory).
__device__ __forceinline__ u32x4 uniform_round(const u32x4 (&d)[kSQ], int qs) {
  const int q = __builtin_amdgcn_readfirstlane(qs);
  u32x4 v = d[0];
  switch (q) {
#define ARCS_UROUND_(i)                                       \
  case i:                                                     \
    v = d[i < kSQ ? i : 0];                                   \
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); \
    break;
    ARCS_UROUND_(1) ARCS_UROUND_(2) ARCS_UROUND_(3) ARCS_UROUND_(4) ARCS_UROUND_(5) ARCS_UROUND_(6)
    ARCS_UROUND_(7) ARCS_UROUND_(8) ARCS_UROUND_(9) ARCS_UROUND_(10) ARCS_UROUND_(11) ARCS_UROUND_(12)
    ARCS_UROUND_(13) ARCS_UROUND_(14) ARCS_UROUND_(15) ARCS_UROUND_(16) ARCS_UROUND_(17) ARCS_UROUND_(18)
    ARCS_UROUND_(19) ARCS_UROUND_(20) ARCS_UROUND_(21) ARCS_UROUND_(22) ARCS_UROUND_(23) ARCS_UROUND_(24)
    ARCS_UROUND_(25) ARCS_UROUND_(26) ARCS_UROUND_(27) ARCS_UROUND_(28) ARCS_UROUND_(29) ARCS_UROUND_(30)
    ARCS_UROUND_(31)
#undef ARCS_UROUND_
    default: break;
  }
  return v;
}

// The 16 bytes of round bq (lanes with `want`; the others get zeros): one
// uniform fetch per distinct round among those lanes, so a wave where few
// lanes want a group pays for few copies.
__device__ __forceinline__ u32x4 rounds_of(const u32x4 (&d)[kSQ], int bq, bool want) {
  u32x4 v = {0u, 0u, 0u, 0u};
  for (uint64_t pend = __ballot(want); pend;) {
    const int qs = __builtin_amdgcn_readlane(bq, __builtin_ctzll(pend));
    const u32x4 vq = uniform_round(d, qs);
    const bool take = want && bq == qs;
    v.x = take ? vq.x : v.x; v.y = take ? vq.y : v.y;
    v.z = take ? vq.z : v.z; v.w = take ? vq.w : v.w;
    pend &= ~__ballot(take);
  }
  return v;
}

// Inverse-CDF draw in id order over sm.tsum (group j's weight at j, in the
// row frame 2^-K*).
// Wave w takes the groups w*64G .. w*64G + 64G - 1 (G = kSQ groups per
// thread), its lane l the G consecutive groups from w*64G + Gl (owned by the
// threads (Gl + i) mod kSNT): the wave totals locate the wave, a wave scan
// the lane, the lane's G sums the group,
// and one re-read of that group the element (entries `cut` drops weigh 0).
// The drawing lane writes the output row.  Returns false (uniformly) when
// the total weight is zero or not finite; else S (the total).  With `sync`
// the id is left in sh.u64[10] for the whole block; otherwise waves other
// than the drawing one return at once.
template <bool PEN>
__device__ __forceinline__ bool tsum_draw(const SampleArgs& a, int64_t row, const u32x4* rv, const PenCtx& pc,
                                          const Smem& sm, Shared& sh, KeepCut cut, float chi,
                                          float clo, float negks, double u, bool sync, double& S) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  constexpr int G = kSQ;  // groups per lane
  static_assert(kSNT % G == 0, "a lane's groups have consecutive owners");
  double v[G];
  const float4* src = (const float4*)(sm.tsum + wid * kWave * G + lane * G);
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const float4 f = src[i];
    v[4 * i] = (double)f.x;
    v[4 * i + 1] = (double)f.y;
    v[4 * i + 2] = (double)f.z;
    v[4 * i + 3] = (double)f.w;
  }
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < G; ++i) part += v[i];
  const double incl = dpp_wave_incl_scan_f64(part);
  if (lane == kWave - 1) sh.rtot[wid] = incl;
  __syncthreads();
  // every thread: the total, in wave order, and the wave the target lies in
  double cum = 0.0, before = 0.0, before_last = 0.0;
  int qs = -1, qlast = 0;
  S = 0.0;
  for (int w = 0; w < kSNW; ++w) S += sh.rtot[w];
  if (!(S > 0.0) || !(S < 1e300)) return false;
  const double t = u * S;
  for (int w = 0; w < kSNW; ++w) {
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
      for (int i = 0; i < G; ++i) {
        const double w = v[i];
        if (v[i] > 0.0) {
          if (is < 0 && bl + w > t) { is = i; bsel = bl; }
          ilast = i;
          blast = bl;
        }
        bl += w;
      }
      if (is < 0) { is = ilast; bsel = blast; }
      const int j = wid * kWave * G + lane * G + is;
      // the group's weights as its owner computed them: the running sum
      // ends at exactly the group's value
      float z[8];
      load_z8<PEN>(rv[j], j, pc, z);
      float acc = 0.0f, prev = 0.0f;
      int pe = -1, last_e = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = keep_cut(z[e], (int64_t)j * 8 + e, cut) ? wexp(z[e], chi, clo, negks) : 0.0f;
        acc = (e == 0) ? w : acc + w;
        const bool pos = acc > prev;
        if (pos) last_e = e;
        if (pe < 0 && pos && bsel + (double)acc > t) pe = e;
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

// The draw for rows without filters over the pass's double weights.  Round
// q's groups are q * kSNT + tid, so id order is (round, wave, lane,
// element): the pass left each wave's total of each round (the last lane of
// an inclusive wave scan) in rw[q * kSNW + w].  Every wave sums the round
// totals and locates the round and then the wave; that wave repeats the
// round's scan from its registers and locates the lane, whose running sum
// locates the element.  Returns false (uniformly) when the total is zero or
// not finite, else S, the total (no frame).  With `sync` the id is left in
// sh.u64[10] for the whole block.
template <bool PEN>
__device__ __forceinline__ bool nofilter_draw(const SampleArgs& a, int64_t row, const u32x4 (&d)[kSQ], int ngroups,
                                              const PenCtx& pc, const Smem& sm, Shared& sh, double c, double u,
                                              bool sync, double& S) {
  static_assert(kSQ <= kWave, "one lane per round");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const double* rw = (const double*)sm.tsum;
  double rt = 0.0;
  if (lane < kSQ) {
#pragma unroll
    for (int w = 0; w < kSNW; ++w) rt += rw[lane * kSNW + w];
  }
  const double rincl = dpp_wave_incl_scan_f64(rt);
  S = readlane63_f64(rincl);
  if (!(S > 0.0) || !(S < 1e300)) return false;
  const double t = u * S;
  const uint64_t nzq = __ballot(rt > 0.0);
  const uint64_t hitq = __ballot(rt > 0.0 && rincl > t);
  const int qs = hitq ? __builtin_ctzll(hitq) : 63 - __builtin_clzll(nzq);  // rounding: the last round with weight
  double cum = qs > 0 ? readlane_f64(rincl, qs - 1) : 0.0;
  int ws = -1, wlast = 0;
  double bw = 0.0, bwlast = 0.0;
  for (int w = 0; w < kSNW; ++w) {
    const double r = rw[qs * kSNW + w];
    if (r > 0.0) {
      if (ws < 0 && cum + r > t) { ws = w; bw = cum; }
      wlast = w;
      bwlast = cum;
    }
    cum += r;
  }
  if (ws < 0) { ws = wlast; bw = bwlast; }
  if (wid == ws) {
    const bool valid = tid < ngroups - qs * kSNT;
    float z[8];
    unpack8(uniform_round(d, qs), z);
    if (PEN && pc.on && valid) penalize8(z, (int64_t)(qs * kSNT + tid) * 8, pc);
    double w8[8];
    const double g = group_weights_f64(z, valid, c, w8, (const double*)sm.skey);
    const double incl = dpp_wave_incl_scan_f64(g);
    const double prev = __shfl_up(incl, 1);
    const uint64_t hit = __ballot(g > 0.0 && bw + incl > t);
    const uint64_t nz = __ballot(g > 0.0);
    const int ls = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
    if (lane == ls) {
      const double bsel = bw + (lane > 0 ? prev : 0.0);
      double acc = 0.0;
      int pe = -1, last_e = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc += w8[e];
        if (w8[e] > 0.0) {
          if (pe < 0 && bsel + acc > t) pe = e;
          last_e = e;
        }
      }
      if (pe < 0) pe = last_e;
      const int32_t id = (qs * kSNT + tid) * 8 + pe;
      a.out_ids[row] = id;
      if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      sh.u64[10] = (uint64_t)id;
    }
  }
  if (sync) __syncthreads();
  return true;
}


// Cut and draw over nc <= kSmallSort candidates, by one wave.  The list is
// sm.ckey / sm.cw[0 .. nc) (keys: ascending = value desc, id asc; weights in
// the row frame).  One pass in which every lane reads the whole list (LDS
// broadcast reads, eight in flight) gives each entry its rank by key, the
// weight of the entries before it in id order, the total and the min-p count.
// When the min-p set is complete and neither top-k nor top-p can cut inside
// it, every entry is kept and the id-order draw follows at once.  Otherwise
// the entries are placed in key order, an fp64 scan gives the prefix masses
// for L = min(L_k, L_p, L_m), and a second pass over the kept prefix gives
// the id-order draw.  Writes the output row and sh.u64[10..12] /
// sh.f64[kSNW+1] (id, L, cut key, S_K).  Returns 1 when drawn, 0 when no
// prefix length is known from the candidates, 2 (nothing written) when
// `lazy_cap` > 0 and the kept mass reaches it.
__device__ __forceinline__ int small_cut_draw(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh, int nc,
                                               bool kon, int top_k, bool pon, double Pm, bool minp_complete, float zt,
                                               double u, double lazy_cap) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int64_t INF = INT64_MAX;
  const bool in = lane < nc;
  const uint64_t key = in ? sm.ckey[lane] : ~0ull;
  const float w = in ? sm.cw[lane] : 0.0f;
  const uint32_t myid = (uint32_t)key;
  const int64_t Lk0 = (kon && (int64_t)top_k <= nc) ? (int64_t)top_k : INF;
  if (minp_complete && Lk0 >= nc && __builtin_popcountll(__ballot(in && key_value(~(uint32_t)(key >> 32)) >= zt)) == nc) {
    // every entry is kept unless top-p cuts inside the min-p set: the total
    // by a wave sum, and only the id-order masses by a pass over the list
    const double tot = dpp_wave_sum_f64(in ? (double)w : 0.0);
    const bool fast = lazy_cap > 0.0 ? tot < lazy_cap : (!pon || tot < Pm);
    if (lazy_cap > 0.0 && !fast) return 2;
    if (fast) {
      // (four partial sums: the weights of a min-p set lie within a factor
      // 1 / min_p of each other, so for min_p above about 1e-7 every sum of
      // up to 64 of them is exact in double precision and the order does not
      // matter; below that the order moves a sum by a double's rounding, far
      // under the binary32 weights' own error)
      double b4[4] = {0.0, 0.0, 0.0, 0.0};
      for (int j0 = 0; j0 < nc; j0 += 8) {
        uint32_t ij[8];
        float wj[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e < nc ? j0 + e : nc - 1;
          ij[e] = ((const uint32_t*)sm.ckey)[2 * j];  // the id half of the key
          wj[e] = sm.cw[j];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j0 + e < nc) b4[e & 3] += ij[e] < myid ? (double)wj[e] : 0.0;
      }
      const double before = (b4[0] + b4[1]) + (b4[2] + b4[3]);
      const double t = u * tot;
      const bool hit = in && w > 0.0f && before + (double)w > t;
      uint32_t pid = dpp_wave_min_u32(hit ? myid : 0xFFFFFFFFu);
      if (pid == 0xFFFFFFFFu) pid = ~dpp_wave_min_u32(in && w > 0.0f ? ~myid : 0xFFFFFFFFu);  // rounding: the last id with weight
      if (lane == 0) {
        a.out_ids[row] = (int32_t)pid;
        if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      }
      // the debug outputs' values: the largest key is the kept set's last entry
      const uint32_t khi = ~dpp_wave_min_u32(in ? ~(uint32_t)(key >> 32) : 0xFFFFFFFFu);
      const uint32_t klo = ~dpp_wave_min_u32(in && (uint32_t)(key >> 32) == khi ? ~(uint32_t)key : 0xFFFFFFFFu);
      if (lane == 0) {
        sh.u64[10] = pid;
        sh.u64[11] = (uint64_t)nc;
        sh.f64[kSNW + 1] = tot;
        sh.u64[12] = ((uint64_t)khi << 32) | klo;
      }
      return 1;
    }
  }
  // the rank of each entry among the keys
  uint32_t r = 0;
  for (int j0 = 0; j0 < nc; j0 += 8) {
    uint64_t kj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kj[e] = sm.ckey[j0 + e < nc ? j0 + e : nc - 1];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < nc) r += kj[e] < key ? 1u : 0u;
  }
  const int64_t Lk = Lk0;
  // the entries in key order, the value-order prefix masses
  wave_lds_sync();
  if (in) { sm.skey[r] = key; sm.sw[r] = w; }
  wave_lds_sync();
  const uint64_t skey = in ? sm.skey[lane] : ~0ull;
  const float sw = in ? sm.sw[lane] : 0.0f;
  const double cum = dpp_wave_incl_scan_f64((double)sw);
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
  // the id-order draw over the kept prefix: each kept entry's running mass in id order
  const bool kept = lane < Lw;
  const uint32_t id2 = (uint32_t)skey;
  double before2 = 0.0;
  for (int j0 = 0; j0 < (int)Lw; j0 += 8) {
    uint64_t kj[8];
    float wj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e < (int)Lw ? j0 + e : (int)Lw - 1;
      kj[e] = sm.skey[j];
      wj[e] = sm.sw[j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < (int)Lw) before2 += (uint32_t)kj[e] < id2 ? (double)wj[e] : 0.0;
  }
  const bool hit = kept && sw > 0.0f && before2 + (double)sw > t;
  uint32_t pid = dpp_wave_min_u32(hit ? id2 : 0xFFFFFFFFu);
  if (pid == 0xFFFFFFFFu) pid = ~dpp_wave_min_u32(kept && sw > 0.0f ? ~id2 : 0xFFFFFFFFu);  // rounding: the last id with weight
  if (lane == 0) {
    sh.u64[10] = pid;
    sh.u64[11] = (uint64_t)Lw;
    sh.f64[kSNW + 1] = sk;
    sh.u64[12] = ck;
    a.out_ids[row] = (int32_t)pid;
    if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
  }
  return 1;
}

template <int NT = kSNT>
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
// order.  Writes the output row, sh.u64[10] (id) and sh.f64[kSNW + 1] (S_K in
// the row frame).  Returns false (uniformly) when the kept mass is zero.
__device__ __forceinline__ bool cand_draw(const SampleArgs& a, int64_t row, const Smem& sm, Shared& sh, int nc,
                                          const KeepCut& cut, uint64_t uf) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  constexpr int ENT = kCandCap / kSNT;
  uint64_t* hm = sm.hmass;
  for (int i = tid; i < 512; i += kSNT) hm[i] = 0ull;
  if (tid == 0) sh.i32[4] = 0;
  __syncthreads();
  uint32_t myid[ENT];
  uint64_t myw[ENT];
#pragma unroll
  for (int q = 0; q < ENT; ++q) {
    const int i = tid + q * kSNT;
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
    sh.f64[kSNW + 1] = (double)sh.u64[7] / kFixScale;
  }
  return true;
}

// The row's exact total weight in the row frame (-negks): every element of
// the row (still in registers) weighed; fp64 per thread, one wave sum and one
// LDS sum.  All threads call it; uniform result.
template <bool PEN>
__device__ __forceinline__ double exact_row_mass(const u32x4 (&dd)[kSQ], const PenCtx& pc, int ngroups, float chi,
                                                 float clo, float negks, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kSQ; ++q) {
    // the round's bound is formed here, not hoisted out of the unrolled
    // loop: live lane masks for every round would crowd out the scalar registers
    int lim = ngroups - q * kSNT;
    asm volatile("" : "+s"(lim));
    const bool valid = tid < lim;
    // opaque copy: the weighing stays where it is called (the compiler would
    // otherwise hoist this loop-invariant work out of the caller's retry loop
    // and run it on every row)
    u32x4 dq = dd[q];
    asm volatile("" : "+v"(dq));
    float z[8];
    unpack8(dq, z);
    if (PEN && pc.on && valid) penalize8(z, (int64_t)(q * kSNT + tid) * 8, pc);
    s += valid ? (double)group_weight(z, chi, clo, negks) : 0.0;
  }
  s = dpp_wave_sum_f64(s);
  __syncthreads();
  if (lane == 0) sh.rtot[wid] = s;
  __syncthreads();
  double S = 0.0;
  for (int w = 0; w < kSNW; ++w) S += sh.rtot[w];
  return S;
}

// The pass over a row whose loads are in flight, one instantiation per kind
// of row so that the unrolled loop carries no per-group branches on the
// row's parameters:
//   W = 0  group maxima only (greedy, min-p and top-k rows, and top-p with
//          top-k, whose mass is bounded from the group maxima afterwards);
//   W = 2  plus every element's weight (top-p rows without top-k).
// Filter rows keep each group's maximum (-inf for groups past the row's end)
// in registers, gm[q], or with penalties (whose arithmetic needs the
// registers) in LDS at sm.tsum[q * kSNT + tid].  NOFILTER rows (W == 3)
// weigh every element in double precision instead and leave each wave's
// total of each round in LDS (as doubles at sm.tsum, [q * kSNW + wave]).
// A lower bound of the row's mass (frame 2^-K*) from every group's maximum,
// for rows whose top-p test the two largest group maxima per thread did not
// settle: the maxima again from the registers (keeping them from the pass
// would hold 32 more registers through the whole tail), binary32 sums of 32
// terms per thread (rounding far inside the 1e-5 margin of the test).
__device__ __forceinline__ double group_max_mass(const u32x4 (&dd)[kSQ], int ngroups, float chi, float clo,
                                                 float negks, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kSQ; ++q) {
    int lim = ngroups - q * kSNT;
    asm volatile("" : "+s"(lim));
    u32x4 dq = dd[q];
    asm volatile("" : "+v"(dq));  // weighed here, not ahead in the caller
    float z[8];
    unpack8(dq, z);
    const float g = group_max(z);
    s += tid < lim && g == g ? wexp(g, chi, clo, negks) : 0.0f;
  }
  const double ws = dpp_wave_sum_f64((double)s);
  __syncthreads();
  if (lane == 0) sh.rtot[wid] = ws;
  __syncthreads();
  double S = 0.0;
  for (int w = 0; w < kSNW; ++w) S += sh.rtot[w];
  return S;
}

template <bool PEN, int W, bool NOFILTER>
__device__ __forceinline__ void row_pass(const u32x4 (&d)[kSQ], int ngroups, const PenCtx& pc, const Smem& sm,
                                         float chi, float clo, PassOut& o, float (&gm)[kSQ]) {
  const int tid = threadIdx.x;
  const double c64 = (double)chi + (double)clo;
  float best = -__builtin_inff(), second = -__builtin_inff();
  int bq = -1;
  double lsum = 0.0;
  float kfr = -__builtin_inff(), negk = 0.0f;
  bool bad = false, special = false;
  // the penalty values in vector registers: the pass's scalar registers are
  // all taken, and scalar copies would be spilled and reloaded every round
  PenCtx pv = pc;
  if (PEN) asm volatile("" : "+v"(pv.pres), "+v"(pv.freq), "+v"(pv.rep));
#pragma unroll
  for (int q = 0; q < kSQ; ++q) {
    // the round's bound is formed here, not hoisted out of the unrolled
    // loop: live lane masks for every round would crowd out the scalar registers
    int lim = ngroups - q * kSNT;
    asm volatile("" : "+s"(lim));
    const bool valid = tid < lim;
    // opaque copy: keeps the compiler from hoisting the widening of all
    // rounds out of the per-kind instantiations (which spills the row)
    u32x4 dq = d[q];
    asm volatile("" : "+v"(dq));
    float z[8];
    unpack8(dq, z);
    if (PEN && ((pc.hmask >> q) & 1u)) penalize8(z, (int64_t)(q * kSNT + tid) * 8, pv);
    float g = group_max(z);
    special = special || !(g == g);
    g = valid && g == g ? g : -__builtin_inff();
    if (!NOFILTER) {
      if (PEN) sm.tsum[q * kSNT + tid] = g;
      else gm[q] = g;
      bq = g > best ? q : bq;
      second = max2f(second, g > best ? best : g);
    }
    best = max2f(best, g);
    if (W == 0) continue;
    if (W == 3) {
      double w8[8];
      const double gw = group_weights_f64(z, valid, c64, w8, (const double*)sm.skey);
      const double incl = dpp_wave_incl_scan_f64(gw);
      if ((tid & (kWave - 1)) == kWave - 1) ((double*)sm.tsum)[q * kSNW + tid / kWave] = incl;
      continue;
    }
    const float x = g * chi;
    if (x > kfr + 64.0f) {
      // the first finite group, or one far above the frame: (re)set it
      if (!(x > -1048576.0f && x < 1048576.0f)) bad = true;
      const float nk = __builtin_floorf(x);
      if (kfr > -__builtin_inff()) {
        const int sh_ = (int)(kfr - nk);
        lsum = __builtin_ldexp(lsum, sh_);
      }
      kfr = nk;
      negk = -nk;
    }
    const float s = group_weight(z, chi, clo, negk);
    lsum += valid ? (double)s : 0.0;
  }
  o.best = best; o.bq = bq; o.second = second; o.lsum = lsum; o.kfr = kfr; o.negk = negk; o.bad = bad; o.special = special;
}

// The lowest index of the maximum wm in the thread's group bq (the first of
// its groups holding its largest value), for lanes whose largest value is wm;
// 0xFFFFFFFF for the others.
template <bool PEN>
__device__ __forceinline__ uint32_t first_index_of(const u32x4 (&d)[kSQ], int bq, float wm, bool look,
                                                   const PenCtx& pc) {
  const int tid = threadIdx.x;
  uint32_t idx = 0xFFFFFFFFu;
  if (!__ballot(look)) return idx;
  const u32x4 v = rounds_of(d, bq, look);
  if (look) {
    float z[8];
    load_z8<PEN>(v, bq * kSNT + tid, pc, z);
#pragma unroll
    for (int e = 7; e >= 0; --e)
      if (z[e] == wm) idx = (uint32_t)(bq * kSNT + tid) * 8u + (uint32_t)e;
  }
  return idx;
}

// Gathers this thread's elements z >= bound (bound finite) into the candidate
// list sm.ckey / sm.cw (with their weights in the row frame -negks when
// WEIGHTS), from the registers.  The group holding the thread's maximum
// (round bq) is taken by a branch-free select; the other groups at or above
// the bound (a mask from the group maxima gm; rare) are visited round by
// round over the set bits of the wave's OR of those masks, each by the same
// select, so rounds no lane needs cost nothing.  Each
// lane counts its entries, one wave scan and one LDS atomic on the block
// count sh.i32[3] place them.  A count above kCandCap means the list is
// incomplete.  Waves with no group at or above the bound return at once.
template <bool PEN, bool WEIGHTS = true>
__device__ __forceinline__ void gather_candidates(const u32x4 (&d)[kSQ], const float (&gm)[kSQ], float best, float second, int bq,
                                                  const PenCtx& pc, const Smem& sm, Shared& sh, float bound,
                                                  float chi, float clo, float negks) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const bool has = best >= bound;
  if (!__ballot(has)) return;
  // the best group, and a mask of the other rounds at or above the bound
  // (looked for only in waves where some thread's second group reaches it)
  const u32x4 v = rounds_of(d, bq, has);
  uint32_t extra = 0;
  if (__ballot(second >= bound)) {
#pragma unroll
    for (int q = 0; q < kSQ; ++q) {
      const float g = PEN ? sm.tsum[q * kSNT + tid] : gm[q];
      extra |= (q != bq && g >= bound) ? (1u << q) : 0u;
    }
  }
  float zb[8];
  load_z8<PEN>(v, bq * kSNT + tid, pc, zb);
  uint32_t mb = 0;
  if (has) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mb |= zb[e] >= bound ? (1u << e) : 0u;
  }
  const uint32_t wex = dpp_wave_or_u32(extra);  // other groups at or above the bound
  // few such rounds: each by a select; many (a low bound): one pass over the
  // rounds with static register names, skipping rounds no lane needs
  const bool few = __builtin_popcount(wex) <= 2;
  uint32_t n = (uint32_t)__builtin_popcount(mb);
  if (few) {
    for (uint32_t m = wex; m; m &= m - 1u) {
      const int qs = __builtin_ctz(m);
      const u32x4 v2 = uniform_round(d, qs);
      if ((extra >> qs) & 1u) {
        float z[8];
        load_z8<PEN>(v2, qs * kSNT + tid, pc, z);
#pragma unroll
        for (int e = 0; e < 8; ++e) n += z[e] >= bound ? 1u : 0u;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < kSQ; ++q) {
      const bool mine = (extra >> q) & 1u;
      if (!__ballot(mine)) continue;
      if (mine) {
        u32x4 dq = d[q];
        asm volatile("" : "+v"(dq));  // not speculated for lanes (or rounds) without candidates
        float z[8];
        load_z8<PEN>(dq, q * kSNT + tid, pc, z);
#pragma unroll
        for (int e = 0; e < 8; ++e) n += z[e] >= bound ? 1u : 0u;
      }
    }
  }
  const uint32_t incl = dpp_wave_incl_scan_u32(n);
  uint32_t base = 0;
  if (lane == kWave - 1) base = (uint32_t)atomicAdd(&sh.i32[3], (int)incl);
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
  uint32_t slot = base + incl - n;
  if (mb) {
    const int64_t i0 = (int64_t)(bq * kSNT + tid) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((mb >> e) & 1u) {
        if (slot < (uint32_t)kCandCap) {
          sm.ckey[slot] = cand_key(zb[e], i0 + e);
          if (WEIGHTS) sm.cw[slot] = wexp(zb[e], chi, clo, negks);
        }
        ++slot;
      }
    }
  }
  if (few) {
    for (uint32_t m = wex; m; m &= m - 1u) {
      const int qs = __builtin_ctz(m);
      const u32x4 v2 = uniform_round(d, qs);
      if ((extra >> qs) & 1u) {
        const int j = qs * kSNT + tid;
        float z[8];
        load_z8<PEN>(v2, j, pc, z);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (z[e] >= bound) {
            if (slot < (uint32_t)kCandCap) {
              sm.ckey[slot] = cand_key(z[e], (int64_t)j * 8 + e);
              if (WEIGHTS) sm.cw[slot] = wexp(z[e], chi, clo, negks);
            }
            ++slot;
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kSQ; ++q) {
    const bool mine = (extra >> q) & 1u;
    if (!__ballot(mine)) continue;
    if (mine) {
      u32x4 dq = d[q];
      asm volatile("" : "+v"(dq));
      const int j = q * kSNT + tid;
      float z[8];
      load_z8<PEN>(dq, j, pc, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (z[e] >= bound) {
          if (slot < (uint32_t)kCandCap) {
            sm.ckey[slot] = cand_key(z[e], (int64_t)j * 8 + e);
            if (WEIGHTS) sm.cw[slot] = wexp(z[e], chi, clo, negks);
          }
          ++slot;
        }
      }
    }
  }
}

template <bool PEN>
__device__ __forceinline__ bool stream_row(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                           const RowConsts& rc, const PenCtx& pc, uint32_t path, const Smem& sm,
                                           Shared& sh, const u32x4 (&d)[kSQ]) {
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
  const bool weights = pon;  // a mass in the wave records (from every weight in the pass, unless lazy)
  // top-p with top-k and min-p: the pass weighs nothing; the weights of each
  // thread's two largest group maxima bound the row's mass from below, and a
  // kept prefix whose mass stays under top_p times that bound is not cut by
  // top-p.  Only when it is not are all group maxima weighed (a tighter
  // bound), and then the exact mass computed (a second pass over the
  // registers).  A prefix cut by both top-k and min-p rarely reaches top_p of
  // the mass; the top-k prefix alone often does (top-p then cuts inside it),
  // and a min-p set without top-k holds most of the mass on exactly the
  // peaked rows where top-p cuts, so those rows weigh every element in the
  // pass.  The penalised kernel always weighs every element: there the
  // second-pass code measured slower than what it saves.
  bool lazy = !PEN && pon && kon && mon;

  if (!rc.ok) return false;
  // rows under the wide tie rule, and rows with an active DRY penalty, run on
  // the general pipeline
  if ((P.flags & ARCS_ROW_TIES_WIDE) && (kon || pon)) return false;
  if (PEN && pc.dry_on) return false;
  const float chi = rc.chi, clo = rc.clo;
  const double tdl = rc.tdl, u = rc.u;

  // ---- the pass over the row (loads already in flight), specialised by mode --------
  // (greedy rows take the group-maxima pass and find the element afterwards)
  PassOut po;
  float gm[kSQ];  // filter rows: the maximum of each of the thread's groups
  if (nofilter) {
    // the power table of the double weights in the small-sort area (unused by
    // rows without filters)
    static_assert((size_t)kSmallSort * 8 >= (size_t)kWave * 8, "the power table fits the small-sort keys");
    fill_exp2_table((double*)sm.skey);
    row_pass<PEN, 3, true>(d, ngroups, pc, sm, chi, clo, po, gm);
  }
  else if (weights && !lazy) row_pass<PEN, 2, false>(d, ngroups, pc, sm, chi, clo, po, gm);
  else row_pass<PEN, 0, false>(d, ngroups, pc, sm, chi, clo, po, gm);
  const float best = po.best;
  const int bq = po.bq;
  double lsum = po.lsum;
  const float kfr = po.kfr, negk = po.negk;
  const bool bad = po.bad, special = po.special;

  // ---- wave records ----------------------------------------------------------------
  {
    const float wm = dpp_wave_max_f32(best);
    const float kw = wm > -__builtin_inff() && weights ? __builtin_floorf(wm * chi) : 0.0f;  // K_w >= K_t
    if (lazy) {
      // the weights of each thread's two largest group maxima, in the wave's
      // frame: a lower bound of the row's mass
      lsum = (double)wexp(best, chi, clo, -kw) + (double)wexp(po.second, chi, clo, -kw);
    } else if (weights) {
      lsum = __builtin_ldexp(lsum, kfr > -__builtin_inff() ? (int)(kfr - kw) : 0);
    }
    const double ws = pon ? dpp_wave_sum_f64(lsum) : 0.0;
    uint32_t warg = 0xFFFFFFFFu;
    if (greedy) warg = dpp_wave_min_u32(first_index_of<PEN>(d, bq, wm, best == wm && wm > -__builtin_inff(), pc));
    const uint32_t wflags = __ballot(bad || special) != 0 ? 1u : 0u;
    if (lane == 0) {
      sh.w_max[wid] = wm; sh.w_negk[wid] = -kw; sh.w_sum[wid] = ws;
      sh.w_arg[wid] = warg; sh.w_flags[wid] = wflags;
    }
    if (!nofilter && !greedy) {
      if (tid < kBins) {
        sm.bcnt[tid] = 0u;
        sm.bmass[tid] = 0.0f;
      }
      if (tid == kSNT - 1) { sh.i32[3] = 0; sh.i32[6] = 0; }
    }
  }
  __syncthreads();

  // ---- the row's values and the mode, in every wave (lane w reads record w) ---------
  // (the same records and the same wave operations give the same values in
  // every wave, so no second barrier broadcasts them)
  const bool rin = lane < kSNW;
  const float rm = rin ? sh.w_max[lane] : -__builtin_inff();
  static_assert(kSNW <= 16, "one record per lane of the first row of 16 lanes");
  constexpr int kRecLanes = kSNW <= 8 ? 8 : 16;
  const float m0 = dpp_octet_max_f32<kRecLanes>(rm);
  int32_t mode = kModeFallback;
  float negks = 0.0f, zt = -__builtin_inff(), zc0 = -FLT_MAX;
  double S = 0.0;  // a lower bound of the row's mass while `lazy`
  double Pm = 0.0;
  uint32_t argmax = 0u;
  if (__builtin_expect(__ballot(rin && sh.w_flags[lane] != 0u) != 0, 0)) {
    mode = kModeFallback;  // a signalling NaN or an out-of-range exponent frame
  } else if (greedy) {
    mode = kModeGreedy;
    argmax = m0 > -__builtin_inff() ? dpp_octet_min_u32<kRecLanes>(rin && rm == m0 ? sh.w_arg[lane] : 0xFFFFFFFFu) : 0u;
  } else if (m0 > -__builtin_inff() && m0 < __builtin_inff() && m0 * chi > -1048576.0f && m0 * chi < 1048576.0f) {
    // (all -inf rows, +inf, or a maximum too large for the exponent frame: general path)
    negks = -__builtin_floorf(m0 * chi);
    if (nofilter) {
      const double mc = (double)m0 * ((double)chi + (double)clo);
      mode = mc > -kF64Span && mc < kF64Span ? kModeNoFilter : kModeFallback;
    } else {
      bool ok = true;
      if (pon) {
        const double x = rin ? __builtin_ldexp(sh.w_sum[lane], (int)(negks - sh.w_negk[lane])) : 0.0;
        S = dpp_octet_sum_f64<kRecLanes>(x);
        ok = S > 0.0 && S < 1e300;
        Pm = (double)P.top_p * S;
      }
      if (mon) {
        bool found;
        zt = minp_threshold(m0, tdl, found);
        ok = ok && found;
        zc0 = zt > -FLT_MAX ? zt : -FLT_MAX;
      }
      // min-p rows gather at the exact threshold; small rows take every
      // element; the others first bound the cut with a histogram
      if (!ok) mode = kModeFallback;
      else mode = (mon || ngroups <= kCandCap / 8) ? kModeCand : kModeHist;
    }
  }
  // wave-uniform: scalar registers, leaving the vector ones to the row
  mode = __builtin_amdgcn_readfirstlane(mode);
  argmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)argmax);
  const float m = uniform_f32(m0);
  negks = uniform_f32(negks); zt = uniform_f32(zt); zc0 = uniform_f32(zc0);
  S = uniform_f64(S); Pm = uniform_f64(Pm);
  if (__builtin_expect(mode == kModeFallback, 0)) return false;

  if (mode == kModeGreedy) {
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
      for (int64_t i = tid; i < V; i += kSNT) a.out_probs[row * V + i] = (i == (int64_t)argmax) ? 1.0f : 0.0f;
    return true;
  }

  // ---- the candidates z >= zc0 from the registers (min-p rows, small rows) ----------
  int nc = -1;
  if (mode == kModeCand) {
    gather_candidates<PEN>(d, gm, best, po.second, bq, pc, sm, sh, zc0, chi, clo, negks);
    __syncthreads();
    nc = sh.i32[3];
    // more than the list holds (min-p rows only): masked sums for min-p alone,
    // else a histogram bound above the threshold
    if (__builtin_expect(nc > kCandCap, 0)) mode = (!kon && !pon) ? kModeMinpStream : kModeHist;
  }

  int64_t id = -1;
  int64_t L = V;
  double S_K = 0.0;
  uint32_t cut_key = 0u;
  int64_t cut_idx = -1;

  if (mode == kModeNoFilter) {
    path |= ARCS_PATH_SORT_SKIP;
    if (!nofilter_draw<PEN>(a, row, d, ngroups, pc, sm, sh, (double)chi + (double)clo, u, debug, S)) return false;
    if (!debug) return true;
    S = __builtin_ldexp(S, (int)negks);  // into the row frame 2^-K* of the other modes
    S_K = S;
    id = (int64_t)sh.u64[10];
  } else if (PEN && mode == kModeMinpStream) {
    // penalised rows with min-p alone over more than 4,096 candidates: the
    // general pipeline (this loop's registers on top of the penalised row's
    // spilled loaded values, each spill waiting for every load in flight)
    return false;
  } else if (__builtin_expect(mode == kModeMinpStream, 0)) {
    // ---- min-p alone over many groups: masked sums and the id-order draw ------------
    path |= ARCS_PATH_CUTOFF | ARCS_PATH_MINP_FLOOR;
    {
#pragma unroll
      for (int q = 0; q < kSQ; ++q) {
        u32x4 dq = d[q];
        asm volatile("" : "+v"(dq));  // only on rows that take this branch
        float z[8];
        unpack8(dq, z);
        if (PEN && pc.on && tid < ngroups - q * kSNT) penalize8(z, (int64_t)(q * kSNT + tid) * 8, pc);
        const KeepCut cut{ord_key(zt), INT64_MAX};
        const int64_t i0 = (int64_t)(q * kSNT + tid) * 8;
        float s = keep_cut(z[0], i0, cut) ? wexp(z[0], chi, clo, negks) : 0.0f;
#pragma unroll
        for (int e = 1; e < 8; ++e) s += keep_cut(z[e], i0 + e, cut) ? wexp(z[e], chi, clo, negks) : 0.0f;
        sm.tsum[q * kSNT + tid] = tid < ngroups - q * kSNT ? s : 0.0f;
      }
    }
    __syncthreads();
    if (!tsum_draw<PEN>(a, row, rv, pc, sm, sh, KeepCut{ord_key(zt), INT64_MAX}, chi, clo, negks, u, debug,
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
      // a histogram of every group's maximum by weight, 8 bins per unit of
      // log2 weight below the row maximum: counts (top-k) and weights (top-p),
      // each a lower bound of what lies above the bin's edge (one element per
      // group).  Groups in the last bin (far below the maximum) are left out:
      // a bound there is no bound.  When the bound lies beyond the last bin (a
      // large k at a low temperature), the histogram is built again with bins
      // 16 times wider.  Rows with a k of at most half the thread count
      // histogram the thread maxima alone, counts only (also one element
      // each; the kept set lies within the top k, so the count bound is enough
      // whatever top-p does): the k-th largest of them lies close to the k-th
      // largest element, and one update per thread replaces one per group.
      const bool thr = kon && P.top_k <= kSNT / 2;
      const bool hmass = pon && !lazy && !thr;
      float c8 = (chi + clo) * 8.0f;
      for (int attempt = 0; attempt < 3; ++attempt, c8 *= 0.0625f) {
        if (attempt > 0) {
          if (tid < kBins) {
            sm.bcnt[tid] = 0u;
            sm.bmass[tid] = 0.0f;
          }
          __syncthreads();
        }
        if (thr) {
          const float x = (m - best) * c8;
          if (best > -__builtin_inff() && x < (float)(kBins - 1)) atomicAdd(&sm.bcnt[(int)x], 1u);
        } else {
#pragma unroll
          for (int q = 0; q < kSQ; ++q) {
            float v = PEN ? sm.tsum[q * kSNT + tid] : gm[q];
            asm volatile("" : "+v"(v));  // round by round: no weights computed ahead and held
            const float x = (m - v) * c8;
            if (v > -__builtin_inff() && x < (float)(kBins - 1)) {
              const int bin = (int)x;
              atomicAdd(&sm.bcnt[bin], 1u);
              if (hmass) atomicAdd(&sm.bmass[bin], wexp(v, chi, clo, negks));
            }
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
          const double p_need = hmass ? Pm * (1.0 + 1e-4) : __builtin_inf();
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
      gather_candidates<PEN>(d, gm, best, po.second, bq, pc, sm, sh, zc, chi, clo, negks);
      __syncthreads();
      nc = sh.i32[3];
    }
    const bool minp_complete = mon && !(zc > zt);
    if (minp_complete) path |= ARCS_PATH_MINP_FLOOR;
    if (__builtin_expect(nc > kCandCap || nc <= 0, 0)) return false;
    if (__builtin_expect(nc <= kSmallSort, 1)) {
      bool wider_bound = false;
      for (;;) {
        if (wid == 0) {
          const double cap = lazy ? (double)P.top_p * S * (1.0 - 1e-5) : 0.0;
          const int rc = small_cut_draw(a, row, sm, sh, nc, kon, P.top_k, pon && !lazy, Pm, minp_complete, zt, u, cap);
          if (lane == 0) sh.i32[6] = rc == 1 ? 0 : (rc == 2 ? 1 : -1);
        }
        __syncthreads();
        if (!lazy || sh.i32[6] != 1) break;
        // top-p may cut inside the prefix: a tighter bound (every group's
        // maximum), then the exact mass, each followed by the cut again
        if (!wider_bound) {
          wider_bound = true;
          S = group_max_mass(d, ngroups, chi, clo, negks, sh);
          continue;
        }
        S = exact_row_mass<PEN>(d, pc, ngroups, chi, clo, negks, sh);
        Pm = (double)P.top_p * S;
        lazy = false;
      }
      if (__builtin_expect(sh.i32[6] < 0, 0)) return false;
      if (!debug) return true;
      id = (int64_t)sh.u64[10];
      L = (int64_t)sh.u64[11];
      S_K = sh.f64[kSNW + 1];
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
        // top-p may cut inside the prefix: a tighter bound (every group's
        // maximum), then the exact mass and the cut again
        S = group_max_mass(d, ngroups, chi, clo, negks, sh);
        if (!(kept_mass < (double)P.top_p * S * (1.0 - 1e-5))) {
          S = exact_row_mass<PEN>(d, pc, ngroups, chi, clo, negks, sh);
          Pm = (double)P.top_p * S;
          lazy = false;
          if (!large_cut_select(sm, sh, nc, lowbit, kon, P.top_k, true, Pm, minp_complete, zt, cut, L, kept_mass,
                                true))
            return false;
        }
      }
      const double ux = u * 0x1p64;  // the uniform as a 64-bit fraction
      const uint64_t uf = ux >= 0x1p64 ? ~0ull : (ux <= 0.0 ? 0ull : (uint64_t)ux);
      if (!cand_draw(a, row, sm, sh, nc, cut, uf)) return false;
      if (!debug) return true;
      __syncthreads();
      id = (int64_t)sh.u64[10];
      S_K = sh.f64[kSNW + 1];
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
    for (int j = tid; j < ngroups; j += kSNT) {
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
        for (int w = 0; w < kSNW; ++w) { a0 += sh.rtot[w]; a1 += sh.w_cnt[w]; }
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
struct RowHist {
  int64_t h0, h1;
  int nreg;               // ids held in registers: id[k] is valid for k * kSNT + tid < nreg
  int32_t id[kHistRegs];  // raw loads (not waited on until the tables are built)
};

// Parameter status, history bounds and the history ids, issued before the
// row's loads.  Returns the row's status.
__device__ __forceinline__ int load_row_history(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                                PenCtx& pc, RowHist& hs) {
  const int tid = threadIdx.x;
  // the history bounds are read together with the parameter record (not
  // after it), so the history ids wait for one load latency only
  int64_t h0 = 0, h1 = 0;
  if (a.hist_ids != nullptr) {
    h0 = a.hist_offsets[row];
    h1 = a.hist_offsets[row + 1];
  }
  int status = row_param_status(P);
  bool dry_on = false;
  if (status == ARCS_ROW_OK) status = dry_status(a, row, dry_on);
  pc.on = false;
  pc.dry_on = false;
  set_penalty_values(pc, P);
  pc.zpen = nullptr; pc.pcount = nullptr;
  hs.h0 = 0; hs.h1 = 0;
  if (status == ARCS_ROW_OK && a.hist_ids != nullptr) {
    const bool active = P.presence != 0.0f || P.frequency != 0.0f || pc.rep_on || dry_on;
    hs.h0 = h0;
    hs.h1 = h1;
    pc.on = active && hs.h1 > hs.h0;
    pc.dry_on = dry_on && pc.on;
  }
  // branch-free: buffer loads past a resource's size return 0 without a
  // memory access (rows without active penalties get an empty resource; ids
  // outside [0, V) read past the row's resource and are skipped later)
  const int64_t n = pc.on ? hs.h1 - hs.h0 : 0;
  const int64_t nreg = n < (int64_t)kHistRegs * kSNT ? n : (int64_t)kHistRegs * kSNT;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pc.on ? a.hist_ids + hs.h0 : a.hist_ids), (short)0, (int)(nreg * 4), 0x00020000);
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k)
    hs.id[k] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(hr, (k * kSNT + tid) * 4, 0, 0);
  hs.nreg = (int)nreg;
  return status;
}

// Visits the row's history ids in [0, V), with their raw logits (read from
// memory) when WITH_RAW: those held in registers, then any beyond them (or,
// FROM_MEMORY, all of them read again).
template <bool WITH_RAW, bool FROM_MEMORY = false, class Fn>
__device__ __forceinline__ void for_each_hist_id(const SampleArgs& a, int64_t row, const RowHist& hs, Fn&& f) {
  const uint16_t* rowp = (const uint16_t*)((const char*)a.logits + row * a.stride * 2);
  if (!FROM_MEMORY) {
#pragma unroll
    for (int k = 0; k < kHistRegs; ++k)
      if (k * kSNT + (int)threadIdx.x < hs.nreg && hs.id[k] >= 0 && (int64_t)hs.id[k] < a.V)
        f((uint32_t)hs.id[k], WITH_RAW ? bf16_to_f32(rowp[hs.id[k]]) : 0.0f);
  }
  for (int64_t i = hs.h0 + (FROM_MEMORY ? 0 : (int64_t)kHistRegs * kSNT) + threadIdx.x; i < hs.h1; i += kSNT) {
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
  pc.hmask = 0u;
  // per thread, the rounds whose group holds a history id (kept in the group
  // value area, where the pass writes each thread's entry of round 0 only
  // after reading it): the pass looks up the
  // tables only in those rounds
  static_assert((size_t)kMaxGroups >= (size_t)kSNT && kSQ <= 32, "a history round mask per thread");
  uint32_t* hm = (uint32_t*)sm.tsum;
  if (status == ARCS_ROW_OK && pc.on) {
    const uint32_t bw = a.bitmap_words;
    for (uint32_t i = tid; i < bw; i += kSNT) sm.bitmap[i] = 0u;
    hm[tid] = 0u;
    lds_barrier();
    for_each_hist_id<false>(a, row, hs, [&](uint32_t id, float) {
      atomicOr(&sm.bitmap[id >> 5], 1u << (id & 31));
      const uint32_t g = id >> 3;
      atomicOr(&hm[g & (kSNT - 1)], 1u << (g / kSNT));
    });
    lds_barrier();
    pc.hmask = hm[tid];
    const uint32_t per = (bw + kSNT - 1) / kSNT;
    const uint32_t w0 = tid * per, w1 = (w0 + per < bw) ? w0 + per : bw;
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; ++w) c += (uint32_t)__builtin_popcount(sm.bitmap[w]);
    uint32_t total;
    const uint32_t incl = block_incl_scan_u32<kSNT, true>(c, sh.bs, total);
    if (total <= (uint32_t)kMaxDistinct) {
      uint32_t run = incl - c;
      for (uint32_t w = w0; w < w1; ++w) {
        sm.wprefix[w] = (uint16_t)run;
        run += (uint32_t)__builtin_popcount(sm.bitmap[w]);
      }
      for (uint32_t i = tid; i < total; i += kSNT) sm.pcount[i] = 0u;
      lds_barrier();
      for_each_hist_id<false>(a, row, hs, [&](uint32_t id, float) {
        atomicAdd(&sm.pcount[pen_rank(id, sm.bitmap, sm.wprefix)], 1u);
      });
      lds_barrier();
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
    write_row_failure<kSNT>(a, row, status);
    return false;
  }
  path = pc.on ? ARCS_PATH_PENALTY : 0u;
  return true;
}


// Split rows, second half (the row's own workgroup): the partials of the
// row's P slices give the maximum, the lowest index holding it and the
// row's weight; the draw finds the slice (slices are in id order), then one
// read of that slice, with the same double weights, the element.  Returns
// false (uniformly) when a slice saw NaN or +inf, or the weights' exponent
// range does not hold the row: the row then takes the whole-row path.
// The row's slice partials for the first wave (lane l: slices 2l and 2l + 1,
// P <= 128), loaded at the kernel's start together with the parameter record:
// the record's wait then does not delay them.  Rows whose slices wrote
// nothing (rows with filters) load stale records and never read them.
struct SplitPre {
  SplitPart p0, p1;
};
__device__ __forceinline__ SplitPre issue_split_loads(const SampleArgs& a, int64_t row) {
  SplitPre s;
  s.p0 = SplitPart{-__builtin_inff(), 0x7FFFFFFF, 0.0};
  s.p1 = s.p0;
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    const SplitPart* parts = a.split_parts + row * a.split_P;
    if (2 * lane < a.split_P) s.p0 = parts[2 * lane];
    if (2 * lane + 1 < a.split_P) s.p1 = parts[2 * lane + 1];
  }
  return s;
}

__device__ __forceinline__ bool split_finish(const SampleArgs& a, int64_t row, const arcs_row_params& P,
                                             const RowConsts& rc, const Smem& sm, Shared& sh, const SplitPre& pre) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int Pn = a.split_P;
  const int64_t V = a.V;
  const int ngroups = (int)(V / 8);
  const int GS = (ngroups + Pn - 1) / Pn;
  const bool greedy = P.temperature == 0.0f || P.top_k == 1;
  const double c = (double)rc.chi + (double)rc.clo;
  if (wid == 0) {
    // lane l holds slices 2l and 2l + 1 (P <= 128)
    const float m0 = pre.p0.m, m1 = pre.p1.m;
    const int32_t a0 = pre.p0.arg, a1 = pre.p1.arg;
    const double s0 = pre.p0.s, s1 = pre.p1.s;
    const bool bad = __ballot(a0 < 0 || a1 < 0) != 0;
    const float M = dpp_wave_max_f32(max2f(m0, m1));
    const uint32_t c0 = m0 == M ? (uint32_t)a0 : 0xFFFFFFFFu, c1 = m1 == M ? (uint32_t)a1 : 0xFFFFFFFFu;
    const uint32_t argmax = M > -__builtin_inff() ? dpp_wave_min_u32(c0 < c1 ? c0 : c1) : 0u;
    int32_t mode = 0;  // 0: whole-row path, 1: done, 2: draw in slice sh.i32[1]
    int sstar = 0;
    double base = 0.0, t = 0.0;
    if (bad) {
      mode = 0;
    } else if (greedy) {
      mode = 1;
      if (lane == 0) {
        a.out_ids[row] = (int32_t)argmax;
        if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      }
    } else if (M > -__builtin_inff() && (double)M * c > -kF64Span) {
      const double ls = s0 + s1;
      const double incl = dpp_wave_incl_scan_f64(ls);
      const double S = readlane63_f64(incl);
      if (S > 0.0 && S < 1e300) {
        t = rc.u * S;
        const uint64_t hit = __ballot(ls > 0.0 && incl > t);
        const uint64_t nz = __ballot(ls > 0.0);
        const int kl = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(nz);  // rounding: the last with weight
        const double ex = incl - ls;
        // in that lane: slice 2l if its weight passes t, else 2l + 1
        const bool first = s0 > 0.0 && (ex + s0 > t || !(s1 > 0.0));
        sstar = __builtin_amdgcn_readlane(2 * lane + (first ? 0 : 1), kl);
        base = readlane_f64(first ? ex : ex + s0, kl);
        mode = 2;
      }
    }
    if (lane == 0) {
      sh.i32[0] = mode;
      sh.i32[1] = sstar;
      sh.f64[0] = base;
      sh.f64[1] = t;
      sh.i32[2] = -1;  // the last group with weight seen (rounding fallback)
      sh.u64[10] = ~0ull;
    }
  }
  __syncthreads();
  const int32_t mode = sh.i32[0];
  if (mode != 2) return mode == 1;
  fill_exp2_table((double*)sm.skey);  // the slice's double weights, as in the slice kernel
  const int sstar = sh.i32[1];
  double base = sh.f64[0];
  const double t = sh.f64[1];
  const int g0 = sstar * GS, g1 = g0 + GS < ngroups ? g0 + GS : ngroups;
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  for (int r0 = g0; r0 < g1; r0 += kSNT) {
    const int g = r0 + tid;
    const bool valid = g < g1;
    float z[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) unpack8(rv[g], z);
    double w8[8];
    const double gw = group_weights_f64(z, valid, c, w8, (const double*)sm.skey);
    const double incl = dpp_wave_incl_scan_f64(gw);
    if (lane == kWave - 1) sh.rtot[wid] = incl;
    if (gw > 0.0) atomicMax(&sh.i32[2], g);
    __syncthreads();
    double wb = base;  // the total before this thread's wave
    for (int w = 0; w < wid; ++w) wb += sh.rtot[w];
    double rt = base;
    for (int w = 0; w < kSNW; ++w) rt += sh.rtot[w];
    const uint64_t hit = __ballot(gw > 0.0 && wb + incl > t);
    if (hit && lane == __builtin_ctzll(hit)) atomicMin((unsigned long long*)&sh.u64[10], (unsigned long long)g);
    __syncthreads();
    const uint64_t gsel = sh.u64[10];
    if (gsel != ~0ull || r0 + kSNT >= g1) {
      // the group (or, past every boundary by rounding, the last with weight):
      // its thread walks its elements
      const int gg = gsel != ~0ull ? (int)gsel : sh.i32[2];
      if (g == gg) {
        double acc = wb + (incl - gw);
        int pe = -1, last_e = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc += w8[e];
          if (w8[e] > 0.0) {
            if (pe < 0 && acc > t) pe = e;
            last_e = e;
          }
        }
        if (pe < 0) pe = last_e;
        a.out_ids[row] = g * 8 + pe;
        if (a.out_status) a.out_status[row] = ARCS_ROW_OK;
      }
      return true;
    }
    base = rt;
    __syncthreads();  // sh.rtot is written again by the next round
  }
  return true;
}

template <bool PEN>
__global__ __launch_bounds__(kSNT) void sample_summary_kernel(SampleArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const Smem sm = carve_smem(smem_raw, true, a.bitmap_words);
  const int ngroups = (int)(a.V / 8);
  const u32x4* rv = (const u32x4*)((const char*)a.logits + row * a.stride * 2);
  u32x4 d[kSQ];
  PenCtx pc;
  uint32_t path;
  if (!PEN) {
    // the parameter record's loads, then the row's: nothing in the issue
    // waits for a load, and the record returns first
    u32x4 p0, p1;
    issue_params_load(a.params + row, p0, p1);
    const RngLoads rl = issue_rng_loads(a, row);
    if (a.split_parts != nullptr) {
      // split launch: greedy rows and rows without filters finish from the
      // slice partials (this waits for the parameter record first)
      const SplitPre pre = issue_split_loads(a, row);
      const arcs_row_params P = params_from(p0, p1);
      const bool greedy = P.temperature == 0.0f || P.top_k == 1;
      const bool nofilter = !greedy && !(P.top_k >= 1 && (int64_t)P.top_k < a.V) && !(P.top_p < 1.0f) &&
                            !(P.min_p > 0.0f);
      if (row_param_status(P) == ARCS_ROW_OK && (greedy || nofilter)) {
        const RowConsts rc = row_consts(P, rng_from(a, rl), row);
        if (rc.ok && split_finish(a, row, P, rc, sm, sh, pre)) return;
        __syncthreads();
      }
    }
    issue_row_loads(rv, ngroups, d);
    arcs_row_params P = params_from(p0, p1);
    const RowRng rng = rng_from(a, rl);
    // this kernel runs only in launches without history arrays (those take
    // the penalised kernel)
    if (!row_prologue<kSNT, true, false, true>(a, row, sm, sh, P, pc, path)) return;
    const RowConsts rc = row_consts(P, rng, row);  // while the loads are in flight
    if (__builtin_expect(!stream_row<false>(a, row, P, rc, pc, path, sm, sh, d), 0)) {
      __syncthreads();
      generic_row<kSNT, true, true>(a, row, P, pc, path, sm, sh);
    }
  } else {
    // history ids first, then the row's loads; the tables are built while
    // those are in flight
    arcs_row_params P = a.params[row];
    const RowRng rng = load_row_rng(a, row);
    RowHist hs;
    const int status = load_row_history(a, row, P, pc, hs);
    // the row's constants before its loads: with the penalty tables' state
    // live, computing them while the row is in registers would spill it
    const RowConsts rc = row_consts(P, rng, row);
    // a quarter of the row's loads go out before the tables are built, the
    // rest after: those in flight during the build already cover the load
    // latency, and the build's waits and LDS traffic then compete with fewer
    // (measured: a quarter before is about 1.5 % faster on a batch of
    // penalised rows than a half, an eighth, none or the whole row)
    __builtin_amdgcn_sched_barrier(0);
    issue_row_loads<0, kSQ / 4>(rv, ngroups, d);
    if (!summary_pen_tables(a, row, sm, sh, status, pc, hs, path)) return;
    issue_row_loads<kSQ / 4, kSQ>(rv, ngroups, d);
    if (!stream_row<true>(a, row, P, rc, pc, path, sm, sh, d)) {
      __syncthreads();
      if (pc.on) {
        // the general pipeline reads penalised logits per distinct id: built
        // here from the counts and the raw logits (every occurrence of an id
        // writes the same value)
        RowHist hm = hs;
        hm.nreg = 0;  // the ids again from memory: keeping the registers that long spilled the row
        for_each_hist_id<true, true>(a, row, hm, [&](uint32_t id, float raw) {
          const uint32_t rk = pen_rank(id, sm.bitmap, sm.wprefix);
          sm.zpen[rk] = penalize(canon_nan(raw), sm.pcount[rk], pc);
        });
        __syncthreads();
        if (pc.dry_on) {
          // the window and the repeat lengths after the penalised logits, in
          // the candidate area (free on this path)
          uint32_t* win = (uint32_t*)(sm.zpen + kMaxDistinct);
          static_assert((size_t)kCandCap * 12 >= (size_t)kMaxDistinct * 8 + (size_t)ARCS_DRY_MAX_WINDOW * 4,
                        "DRY scratch in the candidate area");
          apply_dry<kSNT>(a, row, hs.h0, hs.h1, sm, win, win + ARCS_DRY_MAX_WINDOW);
        }
      }
      generic_row<kSNT, true, true>(a, row, P, pc, path, sm, sh);
    }
  }
}


