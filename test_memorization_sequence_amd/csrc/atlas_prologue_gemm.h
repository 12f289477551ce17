// atlas_prologue_gemm.h -- host entry of the prologue's projection GEMM
// (atlas_prologue_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "atlas_mem_internal.h"

namespace atlas {
namespace prologue {

// C[M][N] = A[M][K] . B[N][K]^T on `st`: bf16 operands, fp32 accumulation,
// bf16 result; K a multiple of 32, N a multiple of 4, device pointers
// 16-byte aligned.  Returns hipErrorInvalidValue for shapes outside that.
hipError_t gemm_nt_bf16(const bf16* A, const bf16* B, bf16* C, int M, int N, int K, hipStream_t st);

}  // namespace prologue
}  // namespace atlas
