// atlas_prologue_gemm.h -- host entry of the prologue's projection GEMM
// (atlas_prologue_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "atlas_mem_internal.h"

namespace atlas {
namespace prologue {

// C[M][N] = A[M][K] . B[N][K]^T on `st`: bf16 operands, fp32 accumulation,
// bf16 result; K a multiple of 8, N a multiple of 4, device pointers
// 16-byte aligned.  Returns hipErrorInvalidValue for shapes outside that.
hipError_t gemm_nt_bf16(const bf16* A, const bf16* B, bf16* C, int M, int N, int K, hipStream_t st);

// The whole prologue (include/atlas_prologue.h) in one kernel, the
// projection tile kept on chip; the same bits as the GEMM followed by
// prologue_kernel.  The caller fills every field above tps.
struct FusedParams {
  const bf16* x;        // [B][N][dm]
  const bf16* w;        // [ncol][dm]
  const float* w_conv;  // [3 H D][K]
  const float* gv;      // [4][H][r]
  const float* gb;      // [4][H]
  bf16* q;
  bf16* k;
  bf16* v;
  float* gate[4];
  int B, N, dm, H, K, r, ncol;
  int tps, tiles_m, tiles_n;   // set by fused_prologue
};
// Whether the fused kernel serves this shape: d_head 64, 128 or 256, the
// gate columns in a column tile of their own (3 H d a multiple of 256),
// one sequence's rows below 1 GiB.
bool fused_supported(int d_head, int heads, int gate_rank, int seq_len, int d_model);
hipError_t fused_prologue(const FusedParams& p, int d_head, hipStream_t st);

}  // namespace prologue
}  // namespace atlas
