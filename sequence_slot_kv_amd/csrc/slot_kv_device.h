// slot_kv_device.h -- device helpers shared by the decode and prefill / verify
// kernels: the coherent stores, loads and epoch-tagged counters through
// which a launch's workgroups hand split partials to the one that merges
// them.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "slot_kv_internal.h"

namespace slotkv {

// Agent-scope (all XCDs) coherent store / load of one float: split partials
// that another workgroup merges within the same launch.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Increment of an epoch-tagged queue or counter word (see kEpochShift): with
// `raise`, the word is first lifted to this launch's epoch, which restarts
// its count at zero if an older launch left it; returns the word as it was
// before the increment, whose count epoch_count() gives.  Both atomics come
// from one lane in program order, so they reach the word in that order.  The
// caller takes the count where it needs it: the wait for the atomic's return
// is placed at the first use of the result, and returns are counted in order
// with the loads, so a use right here would also wait for every load the
// wave has in flight.
__device__ __forceinline__ uint64_t epoch_increment(uint64_t* word, uint64_t epoch_tag,
                                                    bool raise) {
  if (raise) (void)__hip_atomic_fetch_max(word, epoch_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __hip_atomic_fetch_add(word, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t epoch_count(uint64_t word) {
  return static_cast<uint32_t>(word & kCountMask);
}

}  // namespace slotkv
