// atlas_mem_group.h -- synchronisation of the workgroups that share one
// sequence (device code).
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

// The XCD (HW_REG_XCC_ID[3:0]) the calling wave runs on.  The members of a
// group report it into a mask word (one bit per XCD) before their first
// barrier and check after it that one bit is set: a placement that breaks the
// barrier's one-L2 assumption sets bit 1 of the error word instead of going
// unnoticed.
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u; }
__device__ __forceinline__ void report_xcc(unsigned* mask) { atomicOr(mask, 1u << xcc_id()); }
__device__ __forceinline__ void check_xcc(const unsigned* mask, unsigned* err) {
  const unsigned m = __hip_atomic_load(mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__builtin_popcount(m) != 1) atomicOr(err, 2u);
}

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
