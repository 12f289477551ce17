// atlas_mem_frag.h -- MFMA operand helpers of the MLP kernels (device code).
//
// gfx950 v_mfma_f32_16x16x32_bf16: for both operands lane l supplies row
// (l & 15) and the eight k values 8*(l >> 4) .. +7; the 16x16 fp32 result
// gives lane l the column (l & 15) and rows 4*(l >> 4) + r, r = 0..3.
//
// "perm32" k order.  Two result tiles stacked along a 32-wide block of a
// contraction dimension hold, for lane group g = l >> 4, the indices
// {4g..4g+3} U {16+4g..16+4g+3}.  Used as an operand in that permuted k order
// they need no data movement; the other operand is then read in the same
// order (ld_perm, ld_tr_perm).
#pragma once

#include <hip/hip_runtime.h>

#include "atlas_mem_internal.h"
#include "atlas_mem_gelu.h"

namespace atlas {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// The value x, opaque to the optimiser: index arithmetic derived from it is
// recomputed where it is used instead of being hoisted out of loops (where
// the compiler would keep it live, or spill it, for the whole loop).
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Raw buffer access (gfx9 descriptor: base, no stride, byte size; the third
// config dword 0x00020000 is the plain 32-bit raw-buffer format of gfx9
// parts).  Out-of-range accesses return zero / are dropped by the hardware.
// A per-lane byte offset in a VGPR plus a wave-uniform one in an SGPR keeps
// the address arithmetic off the vector ALU.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store4(const f32x4& v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 0);
}

// Buffer load that writes LDS directly (no registers): lane l's BYTES (4 or
// 16) go to LDS at dst + l * BYTES, dst wave-uniform.  A voff beyond the
// buffer's size reads zeros.  Completion is counted by vmcnt like any load:
// wait for it (s_waitcnt vmcnt) before a barrier after which other waves read.
template <int BYTES>
__device__ __forceinline__ void buf_load_lds(__amdgpu_buffer_rsrc_t r, void* dst, int voff) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 4, voff, 0, 0, 0);
}
// wait for every vector-memory access of this wave (loads to LDS included)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0) only
constexpr int kZeroOffset = 0x7FFFFF00;   // beyond every buffer the kernels address
// Copy of NR rows into LDS by direct loads: row r lands at dst + r * LP
// (bytes), its first RB bytes read from byte src(r) of buffer rs (src < 0:
// zeros), the padding bytes LP - RB zeroed.  The region is cut into
// 64 * GR-byte blocks, one load per block, spread over the NW waves.
template <int GR, int NR, int RB, int LP, int NW, class Src>
__device__ __forceinline__ void rows_to_lds(__amdgpu_buffer_rsrc_t rs, char* dst, int wave_s, int lane, Src src) {
  static_assert((GR == 4 || GR == 16) && LP % GR == 0 && RB % GR == 0 && RB <= LP, "granules");
  constexpr int TOTAL = NR * LP, BLK = 64 * GR, NB = (TOTAL + BLK - 1) / BLK;
#pragma unroll
  for (int b0 = 0; b0 < NB; b0 += NW) {
    const int b = b0 + wave_s;
    if (b < NB) {
      const int off = b * BLK + lane * GR, row = off / LP, cb = off - row * LP;
      const int so = src(row);
      const int voff = cb < RB && so >= 0 ? so + cb : kZeroOffset;
      if (TOTAL % BLK == 0 || off < TOTAL) buf_load_lds<GR>(rs, dst + b * BLK, voff);
    }
  }
}

// Row-major operand (k contiguous), natural k order: lane reads k0+8g .. +7 of row row0 + (l & 15).
__device__ __forceinline__ bf16x8 ld_nat(const bf16* base, int ld, int row0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// Row-major operand, perm32 k order: k0+4g .. +3, then k0+16+4g .. +3.
__device__ __forceinline__ bf16x8 ld_perm(const bf16* base, int ld, int row0, int k0, int lane) {
  const bf16* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Natural order, element i scaled by s[k0 + 8g + i].
__device__ __forceinline__ bf16x8 ld_nat_scaled(const bf16* base, int ld, int row0, int k0, int lane, const float* s) {
  const bf16x8 v = ld_nat(base, ld, row0, k0, lane);
  const float* sc = s + k0 + 8 * (lane >> 4);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)v[i] * sc[i]);
  return r;
}
// Element i scaled by sc[i] (sc already offset to the lane's first k).
__device__ __forceinline__ bf16x8 scaled_k(const bf16x8& v, const float* sc) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)v[i] * sc[i]);
  return r;
}
// Every element scaled by one factor.
__device__ __forceinline__ bf16x8 scaled(const bf16x8& v, float s) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)v[i] * s);
  return r;
}
// Two stacked result tiles -> perm32 operand.
__device__ __forceinline__ bf16x8 tiles_to_frag(const f32x4& lo, const f32x4& hi) {
  return bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3], (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}

// Transposed reads from LDS (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane s addresses row (s >> 2) and columns 4*(s & 3) .. +3 of a 4x16
// block of a k-major matrix M[k][n]; the instruction returns to lane s the
// column n = s, rows 0..3.  Two such reads give the operand of row
// n0 + (l & 15) of the transposed matrix, so M needs no transposed copy.
__device__ __forceinline__ i16x4 tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
// M[k][n] (n contiguous, row stride ld): operand row n0 + (l & 15), natural k order.
__device__ __forceinline__ bf16x8 ld_tr_nat(const bf16* M, int ld, int n0, int k0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const bf16* p = M + (k0 + 8 * g + (s >> 2)) * ld + n0 + 4 * (s & 3);
  return join(tr4(p), tr4(p + 4 * ld));
}
// Same, perm32 k order.
__device__ __forceinline__ bf16x8 ld_tr_perm(const bf16* M, int ld, int n0, int k0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const bf16* p = M + (k0 + 4 * g + (s >> 2)) * ld + n0 + 4 * (s & 3);
  return join(tr4(p), tr4(p + 16 * ld));
}

}  // namespace mfma
}  // namespace atlas
