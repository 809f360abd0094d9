// Token commit into a host-mapped ring, with a sticky fault word.
//
// In the Arc engine's device decode loop (Arc PR #217, "What this does",
// step 3, and the fault handling after it) the step after the draw scatters
// the token into the input buffer of the next step, bumps a device position
// and publishes the token into a pinned, mapped host ring that the host
// drains with plain loads, without any stream synchronisation.  A fault is
// reported without a blocking call through a pinned word the commit kernel
// latches after range-checking the token and the position, before it writes
// anything.
//
// One workgroup.  Every check happens before the first write, so a refused
// step leaves the ring, the next-step inputs and the position as they were.
// Only this kernel writes the fault word and launches on one stream run in
// order, so a plain read-then-store latches it (no atomics to host memory).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arcs.h"

namespace arcs {

constexpr int kCommitNT = 256;

__global__ __launch_bounds__(kCommitNT) void commit_tokens_kernel(const int32_t* ids, int64_t B, int64_t V,
                                                                  int32_t* next_input, uint64_t* position,
                                                                  int32_t* ring, uint64_t capacity,
                                                                  volatile uint64_t* published,
                                                                  const volatile uint64_t* drained,
                                                                  volatile uint32_t* fault) {
  __shared__ int s_bad, s_go;
  __shared__ uint64_t s_p;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  for (int64_t b = tid; b < B; b += kCommitNT) {
    const int32_t t = ids[b];
    // -1 marks a row the sampler refused (its status says why): published as
    // is, so one request's bad parameters do not stop the whole batch
    bad |= ((t < 0 && t != -1) || (int64_t)t >= V) ? 1 : 0;
  }
  if (bad) s_bad = 1;  // any writer stores the same value
  __syncthreads();
  // one thread reads the host-written words (the host may change them at any
  // time) and decides for the workgroup
  if (tid == 0) {
    const uint64_t p = *position;
    const uint32_t latched = *fault;
    uint32_t code = ARCS_FAULT_NONE;
    if (s_bad) code = ARCS_FAULT_TOKEN_RANGE;
    else if (p - *drained >= capacity) code = ARCS_FAULT_RING_OVERRUN;
    if (latched == ARCS_FAULT_NONE && code != ARCS_FAULT_NONE) *fault = code;
    s_go = latched == ARCS_FAULT_NONE && code == ARCS_FAULT_NONE;
    s_p = p;
  }
  __syncthreads();
  if (!s_go) return;
  const uint64_t p = s_p;
  int32_t* slot = ring + (int64_t)(p % capacity) * B;
  for (int64_t b = tid; b < B; b += kCommitNT) {
    const int32_t t = ids[b];
    if (next_input) next_input[b] = t;
    slot[b] = t;
  }
  __threadfence_system();  // the ring entries before the count that publishes them
  __syncthreads();
  if (tid == 0) {
    *published = p + 1;
    *position = p + 1;
  }
}

}  // namespace arcs

extern "C" int arcs_commit_tokens(const int32_t* ids, int64_t B, int64_t V, int32_t* next_input,
                                  uint64_t* position, int32_t* ring, uint64_t capacity, uint64_t* published,
                                  const uint64_t* drained, uint32_t* fault, void* stream) {
  if (ids == nullptr || position == nullptr || ring == nullptr || published == nullptr || drained == nullptr ||
      fault == nullptr)
    return ARCS_ERR_NULL_POINTER;
  if (B <= 0 || B > INT32_MAX) return ARCS_ERR_BAD_BATCH;
  if (V <= 0 || V > INT32_MAX) return ARCS_ERR_BAD_VOCAB;
  if (capacity == 0 || capacity > (uint64_t)INT64_MAX / (uint64_t)B) return ARCS_ERR_BAD_CAPACITY;
  if (((uintptr_t)position | (uintptr_t)published | (uintptr_t)drained) % 8u != 0 ||
      ((uintptr_t)ids | (uintptr_t)ring | (uintptr_t)next_input | (uintptr_t)fault) % 4u != 0)
    return ARCS_ERR_MISALIGNED;
  hipLaunchKernelGGL(arcs::commit_tokens_kernel, dim3(1), dim3(arcs::kCommitNT), 0, (hipStream_t)stream, ids, B,
                     V, next_input, position, ring, capacity, published, drained, fault);
  return hipGetLastError() == hipSuccess ? ARCS_OK : ARCS_ERR_LAUNCH;
}
