// atlas_mem_group_split.h -- the group barrier of atlas_mem_group.h in two
// halves (device code), for kernels that overlap work with the wait.
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

// The group barrier (atlas_mem_group.h) in two halves, so that work that
// needs neither the partners' data nor their arrival runs between them:
// group_arrive publishes this workgroup's stores and its arrival,
// group_wait waits for the others (bounded; see group_barrier).
__device__ __forceinline__ void group_arrive(unsigned* ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(ctr, 1u);
}
__device__ __forceinline__ void group_wait(unsigned* ctr, unsigned target, unsigned* err) {
  if (threadIdx.x == 0) {
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
