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
};

// out_ids value the fp32 kernel leaves for a row it hands to the general
// kernel launched after it on the same stream (never a valid id or status).
constexpr int32_t kDeferredId = INT32_MIN;

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
