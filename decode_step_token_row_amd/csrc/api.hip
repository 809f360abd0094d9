// C ABI of libarcs (declared in include/arcs.h): argument validation, launch
// configuration and nothing else.  No allocation, no synchronisation, no
// host reads of device memory: every call only enqueues kernels on the
// caller's stream (Arc PR #217, "What this does" and "Layering": the
// sampling step must not put a host round trip between decode steps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "arcs.h"
#include "launch.hpp"

// Device scratch of arcs_sample_noalloc: one copy per GPU, held until the
// process ends, at its own address on each device.  Host code never uses the
// symbol itself (on the host it is only a stand-in): the address comes from
// hipGetSymbolAddress with that device current, cached per device.
static __device__ __align__(256) unsigned char scratch[ARCS_NOALLOC_SCRATCH_BYTES];
static_assert(arcs::split_max_workspace() <= ARCS_NOALLOC_SCRATCH_BYTES, "the scratch holds every split workspace");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on the first call there).
// Two threads racing on a first call store the same address.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ARCS_ERR_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return ARCS_ERR_LAUNCH;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  *out = p;
  return ARCS_OK;
}

constexpr int64_t kMaxDim = 2147483647;

int check_common(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                 const void* out_ids) {
  if (logits == nullptr || out_ids == nullptr) return ARCS_ERR_NULL_POINTER;
  if (dtype != ARCS_DTYPE_BF16 && dtype != ARCS_DTYPE_F32) return ARCS_ERR_BAD_DTYPE;
  if (B <= 0 || B > kMaxDim) return ARCS_ERR_BAD_BATCH;
  if (V <= 0 || V > kMaxDim) return ARCS_ERR_BAD_VOCAB;
  if (row_stride < V) return ARCS_ERR_BAD_STRIDE;
  const int64_t es = dtype == ARCS_DTYPE_BF16 ? 2 : 4;
  if (((uintptr_t)logits) % (uintptr_t)es != 0) return ARCS_ERR_MISALIGNED;
  return ARCS_OK;
}

// Rows start on a 16-byte boundary: the vector-load path applies.
bool rows_16b_aligned(const void* logits, int dtype, int64_t row_stride) {
  const int64_t es = dtype == ARCS_DTYPE_BF16 ? 2 : 4;
  return ((uintptr_t)logits % 16u) == 0 && ((row_stride * es) % 16) == 0;
}

// Fixed-point fraction bits: V * 2^F < 2^63 so any sum of weights in [0, 1]
// fits an unsigned 64-bit integer.
int fixed_bits(int64_t V) {
  int lg = 0;
  while ((int64_t(1) << (lg + 1)) <= V) ++lg;  // floor(log2 V)
  int F = 62 - lg;
  return F > 62 ? 62 : F;
}

int sample_impl(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                uint64_t seed, uint64_t step, const uint64_t* key, int32_t* out_ids, int32_t* out_status,
                void* workspace, size_t workspace_bytes, const double* uniforms, float* out_probs,
                arcs_row_stats* out_stats, void* stream, const arcs_dry_params* dry = nullptr,
                const int32_t* breakers = nullptr, int n_breakers = 0) {
  int st = check_common(logits, dtype, B, V, row_stride, out_ids);
  if (st != ARCS_OK) return st;
  if (n_breakers < 0 || n_breakers > ARCS_DRY_MAX_BREAKERS || (n_breakers > 0 && breakers == nullptr))
    return ARCS_ERR_BAD_DRY;
  if (((uintptr_t)dry) % 4u != 0 || ((uintptr_t)breakers) % 4u != 0) return ARCS_ERR_MISALIGNED;
  if (params == nullptr) return ARCS_ERR_NULL_POINTER;
  if ((hist_ids == nullptr) != (hist_offsets == nullptr)) return ARCS_ERR_BAD_HISTORY;
  const size_t ws_need = arcs_sample_workspace_bytes(B, V, dtype);
  if (workspace_bytes < ws_need) return ARCS_ERR_WORKSPACE_TOO_SMALL;
  if (ws_need > 0 && workspace == nullptr) return ARCS_ERR_NULL_POINTER;
  if (ws_need > 0 && ((uintptr_t)workspace & 15u) != 0) return ARCS_ERR_MISALIGNED;
  arcs::SampleArgs a;
  a.logits = logits;
  a.V = V;
  a.stride = row_stride;
  a.params = params;
  a.hist_ids = hist_ids;
  a.hist_offsets = hist_offsets;
  a.seed = seed;
  a.step = step;
  a.key = key;
  a.out_ids = out_ids;
  a.out_status = out_status;
  a.uniforms = uniforms;
  a.out_probs = out_probs;
  a.stats = out_stats;
  a.F = fixed_bits(V);
  a.scale = (float)((double)(int64_t(1) << a.F));
  a.pen_tables = (hist_ids != nullptr && V <= ARCS_MAX_PENALTY_VOCAB) ? 1 : 0;
  a.bitmap_words = a.pen_tables ? (uint32_t)((V + 31) / 32) : 0u;
  a.deferred_only = 0;
  a.dry = dry;
  a.dry_breakers = breakers;
  a.n_breakers = n_breakers;
  // penalised launches: a workspace of arcs_long_history_workspace_bytes()
  // takes the rows whose penalties the LDS tables cannot hold
  const size_t long_need = arcs_long_history_workspace_bytes(B, V);
  a.long_ws = (hist_ids != nullptr && workspace != nullptr && workspace_bytes >= long_need &&
               ((uintptr_t)workspace & 15u) == 0)
                  ? (float*)workspace
                  : nullptr;
  const bool vec = rows_16b_aligned(logits, dtype, row_stride);
  // small batches: greedy rows and rows without filters are read by many
  // workgroups per row (not with debug outputs, which read the row whole)
  const bool split = ws_need > 0 && arcs::split_shape(B, V, dtype) && vec && !a.pen_tables &&
                     out_stats == nullptr && out_probs == nullptr;
  a.split_parts = split ? (arcs::SplitPart*)workspace : nullptr;
  a.split_P = split ? arcs::split_slices(B) : 0;
  hipError_t e = arcs::launch_sample(a, dtype, B, vec, (hipStream_t)stream);
  return e == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int arcs_argmax(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                int32_t* out_ids, void* stream) {
  int st = check_common(logits, dtype, B, V, row_stride, out_ids);
  if (st != ARCS_OK) return st;
  hipError_t e = arcs::launch_argmax(logits, dtype, B, V, row_stride,
                                     rows_16b_aligned(logits, dtype, row_stride), out_ids,
                                     (hipStream_t)stream);
  return e == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}

int arcs_sample(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                uint64_t seed, uint64_t step, int32_t* out_ids, int32_t* out_status,
                void* workspace, size_t workspace_bytes, void* stream) {
  return sample_impl(logits, dtype, B, V, row_stride, params, hist_ids, hist_offsets, seed, step,
                     nullptr, out_ids, out_status, workspace, workspace_bytes, nullptr, nullptr, nullptr,
                     stream);
}

int arcs_sample_dry(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                    const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                    const arcs_dry_params* dry, const int32_t* breakers, int n_breakers, uint64_t seed,
                    uint64_t step, int32_t* out_ids, int32_t* out_status, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return sample_impl(logits, dtype, B, V, row_stride, params, hist_ids, hist_offsets, seed, step, nullptr,
                     out_ids, out_status, workspace, workspace_bytes, nullptr, nullptr, nullptr, stream, dry,
                     breakers, n_breakers);
}

int arcs_sample_noalloc(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                        const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                        uint64_t seed, uint64_t step, int32_t* out_ids, int32_t* out_status, void* stream) {
  int st = check_common(logits, dtype, B, V, row_stride, out_ids);
  if (st != ARCS_OK) return st;
  const size_t need = arcs_sample_workspace_bytes(B, V, dtype);
  if (need > (size_t)ARCS_NOALLOC_SCRATCH_BYTES) return ARCS_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    st = noalloc_scratch(&ws);
    if (st != ARCS_OK) return st;
  }
  return sample_impl(logits, dtype, B, V, row_stride, params, hist_ids, hist_offsets, seed, step, nullptr,
                     out_ids, out_status, ws, need, nullptr, nullptr, nullptr, stream);
}

int arcs_sample_keyed(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const arcs_row_params* params, const int32_t* hist_ids,
                      const int64_t* hist_offsets, uint64_t* key, int advance, int32_t* out_ids,
                      int32_t* out_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (key == nullptr) return ARCS_ERR_NULL_POINTER;
  if (((uintptr_t)key) % 8u != 0) return ARCS_ERR_MISALIGNED;
  int st = sample_impl(logits, dtype, B, V, row_stride, params, hist_ids, hist_offsets, 0, 0, key,
                       out_ids, out_status, workspace, workspace_bytes, nullptr, nullptr, nullptr, stream);
  if (st != ARCS_OK || !advance) return st;
  return arcs::launch_advance_step(key, (hipStream_t)stream) == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}

int arcs_sample_debug(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const arcs_row_params* params, const int32_t* hist_ids,
                      const int64_t* hist_offsets, uint64_t seed, uint64_t step,
                      int32_t* out_ids, int32_t* out_status, void* workspace,
                      size_t workspace_bytes, const double* uniforms, float* out_probs,
                      arcs_row_stats* out_stats, void* stream) {
  return sample_impl(logits, dtype, B, V, row_stride, params, hist_ids, hist_offsets, seed, step,
                     nullptr, out_ids, out_status, workspace, workspace_bytes, uniforms, out_probs,
                     out_stats, stream);
}

int arcs_sample_hybrid_nucleus(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                               const float* temperature, const float* top_p, int budget, uint64_t seed,
                               uint64_t step, int32_t* out_ids, int32_t* out_kept, int32_t* out_status,
                               void* stream) {
  int st = check_common(logits, dtype, B, V, row_stride, out_ids);
  if (st != ARCS_OK) return st;
  if (temperature == nullptr || top_p == nullptr) return ARCS_ERR_NULL_POINTER;
  if (dtype != ARCS_DTYPE_BF16) return ARCS_ERR_BAD_DTYPE;
  if (V % 8 != 0 || V > 131072) return ARCS_ERR_BAD_VOCAB;
  if (!rows_16b_aligned(logits, dtype, row_stride)) return ARCS_ERR_MISALIGNED;
  if (((uintptr_t)temperature) % 4u != 0 || ((uintptr_t)top_p) % 4u != 0) return ARCS_ERR_MISALIGNED;
  if (budget < 0 || budget > 4096) return ARCS_ERR_BAD_BUDGET;
  arcs::HybridArgs a;
  a.logits = logits;
  a.V = V;
  a.stride = row_stride;
  a.temperature = temperature;
  a.top_p = top_p;
  a.budget = budget;
  a.seed = seed;
  a.step = step;
  a.out_ids = out_ids;
  a.out_kept = out_kept;
  a.out_status = out_status;
  return arcs::launch_hybrid_nucleus(a, B, (hipStream_t)stream) == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}

int arcs_top_logprobs(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const float* temperature, int n, int32_t* out_ids, float* out_logprobs,
                      int32_t* out_status, void* stream) {
  int st = check_common(logits, dtype, B, V, row_stride, out_ids);
  if (st != ARCS_OK) return st;
  if (out_logprobs == nullptr) return ARCS_ERR_NULL_POINTER;
  if (n < 1 || n > ARCS_MAX_TOP_LOGPROBS) return ARCS_ERR_BAD_TOP_N;
  if (V > ARCS_TOP_LOGPROBS_MAX_VOCAB) return ARCS_ERR_BAD_VOCAB;
  if (((uintptr_t)temperature) % 4u != 0) return ARCS_ERR_MISALIGNED;
  arcs::LogprobArgs a;
  a.logits = logits;
  a.V = V;
  a.stride = row_stride;
  a.temperature = temperature;
  a.n = n;
  a.out_ids = out_ids;
  a.out_logprobs = out_logprobs;
  a.out_status = out_status;
  hipError_t e = arcs::launch_top_logprobs(a, dtype, B, rows_16b_aligned(logits, dtype, row_stride),
                                           (hipStream_t)stream);
  return e == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}

size_t arcs_long_history_workspace_bytes(int64_t B, int64_t V) {
  if (B <= 0 || V <= 0) return 0;
  const unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)V * 4u;
  return n > (unsigned __int128)SIZE_MAX ? SIZE_MAX : (size_t)n;
}

size_t arcs_sample_workspace_bytes(int64_t B, int64_t V, int dtype) {
  if (!arcs::split_shape(B, V, dtype)) return 0;
  return (size_t)B * (size_t)arcs::split_slices(B) * sizeof(arcs::SplitPart);
}

const char* arcs_status_string(int code) {
  switch (code) {
    case ARCS_OK: return "ok";
    case ARCS_ERR_NULL_POINTER: return "a required pointer is NULL";
    case ARCS_ERR_BAD_BATCH: return "batch size B must be in [1, 2^31-1]";
    case ARCS_ERR_BAD_VOCAB: return "vocabulary size V must be in [1, 2^31-1]";
    case ARCS_ERR_BAD_STRIDE: return "row_stride must be >= V";
    case ARCS_ERR_BAD_DTYPE: return "dtype must be ARCS_DTYPE_BF16 or ARCS_DTYPE_F32";
    case ARCS_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than arcs_sample_workspace_bytes()";
    case ARCS_ERR_BAD_BUDGET: return "budget outside [0, 4096]";
    case ARCS_ERR_BAD_DRY: return "DRY breakers: NULL with n_breakers > 0, or n_breakers outside [0, 64]";
    case ARCS_ERR_SCRATCH_TOO_SMALL:
      return "the shape needs more workspace than arcs_sample_noalloc's scratch (ARCS_NOALLOC_SCRATCH_BYTES)";
    case ARCS_ERR_LAUNCH: return "kernel launch failed";
    case ARCS_ERR_MISALIGNED: return "logits pointer not aligned to its element size";
    case ARCS_ERR_BAD_HISTORY: return "hist_ids and hist_offsets must both be NULL or both be set";
    case ARCS_ERR_BAD_TOP_N: return "n must be in [1, ARCS_MAX_TOP_LOGPROBS]";
    case ARCS_ERR_BAD_CAPACITY: return "ring capacity must be >= 1 and capacity * B must fit int64";
    case ARCS_ROW_BAD_TEMPERATURE: return "row: temperature is NaN or negative";
    case ARCS_ROW_BAD_TOP_P: return "row: top_p is NaN or <= 0";
    case ARCS_ROW_BAD_MIN_P: return "row: min_p is NaN or outside [0, 1]";
    case ARCS_ROW_BAD_PENALTY: return "row: a penalty is not finite or repetition < 0";
    case ARCS_ROW_BAD_FLAGS: return "row: flags must be 0";
    case ARCS_ROW_HISTORY_TOO_LONG: return "row: penalties need at most ARCS_MAX_HISTORY distinct history ids";
    case ARCS_ROW_VOCAB_TOO_LARGE: return "row: penalties need V <= ARCS_MAX_PENALTY_VOCAB";
    default: return "unknown status";
  }
}

int arcs_version(void) { return 100; }

}  // extern "C"
