// atlas_mem_lds_sync.h -- a workgroup barrier that orders LDS accesses only.
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {

// Every wave's LDS reads and writes issued before the barrier are complete,
// and visible to every wave, after it.  Global loads and stores stay in
// flight across it: __syncthreads also waits for all of them (its fences
// cover every address space), which exposes the latency of a prefetch issued
// before the barrier.  Loads that write LDS directly are global loads: wait
// for them (vmcnt) before this barrier.  Global data handed between the waves
// of one workgroup needs __syncthreads.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace atlas
