// Hand-offs between the workgroups of one launch on MI355X: each XCD has its
// own write-back L2, and the agent-scope release/acquire fences that keep
// plain stores coherent across XCDs are L2 write-backs and invalidates, far
// too costly per hand-off.  Every value one workgroup hands to another is
// written with agent-scope (write-through) stores and read with device-scope
// buffer loads (sc1), and every wait for such a value is bounded in time.
// Used by the fused one-token decode kernel and the fused small-batch route.
#pragma once

#include "kernels.hpp"

namespace moe {

__device__ __forceinline__ uint32_t ld_cnt(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_dev(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's earlier memory operations have completed (stores at the
// coherence point).
__device__ __forceinline__ void stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Bounded wait: gives up once `budget` ticks of the 100 MHz wall clock have
// passed (checked at every unsuccessful poll: a scalar clock read, no memory
// access), or soon after another wave of the call gave up (the error word is
// read every 64 polls); it then records the call's tag in the error word (the
// first wave of the call to do so also counts the call in the
// timed-out-calls word) and returns.  Indices read from shared state are
// clamped by their users and every result the waits guard is read from LDS
// tables built from the call's own (clamped) selections or through buffer
// resources bounded by their arrays, so a timed-out wait yields wrong
// numbers, never an out-of-bounds access, and the grid always drains.
template <typename Ready>
__device__ __forceinline__ void wait_until(Ready ready, uint32_t* ctl, uint32_t tag, unsigned long long budget) {
  if (!ready()) {
    uint32_t* err = ctl + kCtlError;
    const unsigned long long t0 = wall_clock64();
    uint32_t n = 0;
    while (!ready()) {
      // A short back-off: every workgroup polls the same few lines, and
      // tighter polling only queues more requests in front of the writes.
      __builtin_amdgcn_s_sleep(4);
      if (wall_clock64() - t0 > budget || ((++n & 63u) == 0u && ld_cnt(err) == tag)) {
        if (__hip_atomic_exchange(err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag)
          __hip_atomic_fetch_add(ctl + kCtlTimeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace moe
