// atlas_prologue_math.h -- per-token arithmetic of the prologue shared by
// the kernel that reads the projections from memory (atlas_prologue.hip) and
// the GEMM kernel that applies it to its own output tile
// (atlas_prologue_gemm.hip), so that both give the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace atlas {
namespace prologue {

// Cross-lane sums by DPP moves (full-rate vector ops, no LDS round trip):
// xor 1 and xor 2 within quads, then the half-row and row mirrors, leave the
// sum of each aligned group of 2, 4, 8 or 16 lanes in all of its lanes.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += dppf<0xB1>(v);    // quad_perm [1,0,3,2]
  if (width >= 4) v += dppf<0x4E>(v);    // quad_perm [2,3,0,1]
  if (width >= 8) v += dppf<0x141>(v);   // row_half_mirror
  if (width >= 16) v += dppf<0x140>(v);  // row_mirror
  return v;
}
// the sum over all 64 lanes, the same in every lane
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum(v, 16);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// SiLU and the logistic with the hardware reciprocal (about 1 ulp in fp32;
// the outputs are bf16): z -> -inf gives rcp(inf) = 0, z -> +inf gives 1
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
__device__ __forceinline__ float sigm(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

}  // namespace prologue
}  // namespace atlas
