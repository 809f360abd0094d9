// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "arcs.h"

namespace arcs {

// Everything one sampling launch needs, passed by value as the kernel argument.
struct SampleArgs {
  const void* logits;
  int64_t V;
  int64_t stride;
  const arcs_row_params* params;
  const int32_t* hist_ids;
  const int64_t* hist_offsets;
  uint64_t seed;
  uint64_t step;
  const uint64_t* key;  // device {seed, step} read at run time instead of seed / step, or NULL
  int32_t* out_ids;
  int32_t* out_status;
  const double* uniforms;
  float* out_probs;
  arcs_row_stats* stats;
  int F;               // fixed-point fraction bits: V * 2^F < 2^63
  float scale;         // 2^F
  int pen_tables;      // LDS penalty tables present in this launch
  uint32_t bitmap_words;
  int deferred_only;   // general kernel: only rows whose out_ids holds kDeferredId
  struct SplitPart* split_parts;  // split launch: [B][split_P] slice partials, or NULL
  int split_P;                    // slices per row of a split launch
  const arcs_dry_params* dry;     // [B] DRY records, or NULL
  float* long_ws;                 // [B][V] binary32: penalised copies of rows whose penalties the LDS
                                  // tables cannot hold (caller workspace), or NULL
  const int32_t* dry_breakers;    // [n_breakers]
  int n_breakers;
};

// Small batches of bf16 rows (B <= kSplitMaxB): greedy rows and rows without
// filters are read by P slices per row, one workgroup each, whose partials
// (slice maximum, the lowest index holding it, the slice's weight in double
// precision) go to the caller's workspace; the row's own workgroup then
// combines them and draws, reading one slice again.
struct SplitPart {
  float m;      // slice maximum (-inf for a slice of -inf values)
  int32_t arg;  // lowest index of the maximum; -1: the slice holds NaN or +inf, or
                // its maximum is out of the double weights' exponent range
  double s;     // sum over the slice of 2^(z c), c = log2(e) / T (rows without filters)
};
static_assert(sizeof(SplitPart) == 16, "split partial record");
constexpr int64_t kSplitMaxB = 64;     // batches up to this many rows are split
constexpr int64_t kSplitMinV = 8192;   // and rows of at least this many tokens
constexpr int kSplitMaxP = 128;        // slices per row
constexpr int kSplitThreads = 256;     // threads per slice workgroup
// P = 512 / B slices (at least 8, at most kSplitMaxP): about 512 workgroups
constexpr int split_slices(int64_t B) {
  const int64_t p = (512 + B - 1) / B;
  return (int)(p < 8 ? 8 : (p > kSplitMaxP ? kSplitMaxP : p));
}
// The largest split workspace of any batch size.
constexpr size_t split_max_workspace() {
  size_t m = 0;
  for (int64_t b = 1; b <= kSplitMaxB; ++b) {
    const size_t w = (size_t)b * (size_t)split_slices(b) * sizeof(SplitPart);
    m = w > m ? w : m;
  }
  return m;
}
// Whether a launch of this shape and element type takes the split path (the
// kernel also needs 16-byte aligned rows, no history and no debug outputs).
inline bool split_shape(int64_t B, int64_t V, int dtype) {
  return dtype == ARCS_DTYPE_BF16 && B >= 1 && B <= kSplitMaxB && V >= kSplitMinV && V <= 131072 && V % 8 == 0;
}

// out_ids value the fp32 kernel leaves for a row it hands to the general
// kernel launched after it on the same stream (never a valid id or status).
constexpr int32_t kDeferredId = INT32_MIN;

// One launch of the baseline hybrid nucleus selector (arcs_sample_hybrid_nucleus).
struct HybridArgs {
  const void* logits;        // bf16
  int64_t V;
  int64_t stride;
  const float* temperature;  // [B]
  const float* top_p;        // [B]
  int budget;                // ids enumerated before bisection takes over
  uint64_t seed;
  uint64_t step;
  int32_t* out_ids;          // [B]
  int32_t* out_kept;         // [B] or NULL
  int32_t* out_status;       // [B] or NULL
};
hipError_t launch_hybrid_nucleus(const HybridArgs& a, int64_t B, hipStream_t stream);

// One top-logprobs launch (arcs_top_logprobs).
struct LogprobArgs {
  const void* logits;
  int64_t V;
  int64_t stride;
  const float* temperature;  // [B] or NULL (T = 1)
  int n;
  int32_t* out_ids;          // [B * n]
  float* out_logprobs;       // [B * n]
  int32_t* out_status;       // [B] or NULL
};

hipError_t launch_argmax(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                         bool vec, int32_t* out, hipStream_t stream);
hipError_t launch_sample(const SampleArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream);
hipError_t launch_advance_step(uint64_t* key, hipStream_t stream);
hipError_t launch_top_logprobs(const LogprobArgs& a, int dtype, int64_t B, bool vec, hipStream_t stream);

}  // namespace arcs
