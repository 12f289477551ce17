// atlas_mem_group.h -- synchronisation of the workgroups that share one
// sequence (device code).
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

// Monotonic arrival counter per group; barrier number `k` (1, 2, ...) waits
// for G*k arrivals.  The members of a group share one XCD and its L2, so no
// device-wide cache write-back or L2 invalidation is needed: every wave waits
// until its own stores are complete (they write through the CU's L1), the
// counter is a device-scope atomic, and after the wait every wave invalidates
// its CU's L1 (vector cache) so that later loads read the partners' data from
// L2.  Bounded: about 2^24 polls, then the call's error word is set and every
// later wait returns at once.
__device__ __forceinline__ void group_barrier(unsigned* ctr, unsigned target, unsigned* err) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(ctr, 1u);
    unsigned polls = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
      if (++polls > (1u << 24)) {
        atomicOr(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  asm volatile("buffer_inv sc0" ::: "memory");
}

}  // namespace atlas
