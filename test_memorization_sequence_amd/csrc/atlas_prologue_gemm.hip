// atlas_prologue_gemm.hip -- the prologue's projection GEMM on gfx950:
// C[M][N] (bf16) = A[M][K] . B[N][K]^T with fp32 accumulation, A and B both
// k-contiguous (x rows and projection-weight rows).
//
// Tiling: a 256 x 256 output tile per workgroup of 4 waves, each wave a
// 128 x 128 quarter held as 8 x 8 MFMA result tiles (v_mfma_f32_16x16x32_bf16,
// accumulators in the accumulation registers).  K advances in LDS
// stages of 64 (two buffers of 2 x 32 KB): each row of a stage is one whole
// 128-byte cache line, written into LDS by buffer loads that target LDS
// directly (1 KB = 8 rows per wave instruction).  Granule g (16 bytes) of
// row r is stored in slot g ^ ((r >> 1) & 7), so the 16 rows an operand
// fragment read touches fall into distinct banks.
//
// Pipeline, per sub-stage of 32 k (two per LDS stage): the wave multiplies
// the first half of its 64 products from fragments already in registers;
// at the end of an LDS stage it waits for the next stage's loads and meets
// the other waves at a barrier; then the second half of the products runs
// with the next sub-stage's fragment reads and (after a barrier) the refill
// of the consumed buffer threaded between them -- one wave per SIMD, so a
// burst of memory instructions would hold back the products behind it.
//
// The output tile is computed transposed (B rows as the MFMA's first
// operand), so each lane holds four adjacent output columns of one row and
// stores them as one 8-byte write.
//
// Tile order: the hardware deals workgroups to the 8 XCDs round robin; the
// tile index is remapped so that each XCD walks its own contiguous range of
// tiles in bands of GM row tiles, and the workgroups resident on one XCD at
// a time share A row tiles and B column tiles in that XCD's L2.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "atlas_mem_internal.h"
#include "atlas_prologue_gemm.h"

namespace atlas {
namespace prologue {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#ifndef GEMM_GM
#define GEMM_GM 4
#endif
constexpr int BM = 256, BN = 256, BK = 64, GM = GEMM_GM;
constexpr int ROWB = BK * 2;   // bytes per LDS row: one cache line
constexpr int TILE_A = BM * ROWB, TILE_B = BN * ROWB, STAGE = TILE_A + TILE_B;
constexpr int LDS_BYTES = 2 * STAGE;   // 128 KB
constexpr int kFar = 0x40000000;       // a scalar offset past every operand descriptor
constexpr int kZeroOffset = 0x7FFFFF00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// lane l's 16 bytes at byte voff + soff of r land in LDS at dst + 16 l
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* dst, int voff, int soff) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_lgkm0_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// acc += a . b^T (one 16 x 16 x 32 product)
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Keeps all of a sub-stage's fragments live until the end of its step, so
// that the next sub-stage's LDS reads land in registers of their own rather
// than in ones an MFMA issued just before may still be reading.
__device__ __forceinline__ void hold(const bf16x8 (&a)[8], const bf16x8 (&b)[8]) {
  asm volatile("" ::"v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
  asm volatile("" ::"v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]));
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_nt_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B, bf16* __restrict__ C, int M, int N, int K,
               int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // tile of this workgroup: XCD x = blockIdx.x % 8 walks tiles [x T8, (x+1) T8)
  const int T = tiles_m * tiles_n, T8 = (T + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * T8 + (int)(blockIdx.x >> 3);
  if (t >= T) return;
  const int band = t / (GM * tiles_n), in = t - band * GM * tiles_n;
  const int gm = min(GM, tiles_m - band * GM);
  const int tm = band * GM + in % gm, tn = in / gm;
  const int m0 = tm * BM, n0 = tn * BN;
  // operand tiles through descriptors sized to their rows: rows past M or N
  // read zeros
  const __amdgpu_buffer_rsrc_t ra = rsrc(A + (size_t)m0 * K, (unsigned)(min(BM, M - m0) * K * 2));
  const __amdgpu_buffer_rsrc_t rb = rsrc(B + (size_t)n0 * K, (unsigned)(min(BN, N - n0) * K * 2));
  // One 1-KB load instruction covers rows r0 .. r0 + 7 (r0 a multiple of 8):
  // lane l fills slot l & 7 of row r0 + (l >> 3) with the granule whose
  // swizzled slot that is; (r >> 1) & 7 = 4 ((r0 >> 3) & 1) + (l >> 4), so
  // two lane offsets serve every instruction.
  // With K not a multiple of 64 the last stage's granules at and past K
  // (K is a multiple of 8) are sent out of range and read zeros.
  const int nk = (K + BK - 1) / BK;   // >= 1
  const int ktail = K - (nk - 1) * BK;
  int voff[2], voff_last[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int g = (lane & 7) ^ (4 * p + (lane >> 4));
    voff[p] = (lane >> 3) * K * 2 + (g << 4);
    voff_last[p] = 8 * g < ktail ? voff[p] : kZeroOffset;
  }
  // instruction q (0..15) of this wave's share of stage s: q < 8 fills A rows
  // 64 wave + 8 q, q >= 8 the same rows of B; a stage past the last reads
  // zeros, so the count of loads in flight is the same every stage
  auto dma = [&](int q, int s) {
    const int row = 64 * wave + 8 * (q & 7);
    const int kofs = s < nk ? s * ROWB : kFar;
    char* dst = smem + (s & 1) * STAGE + (q < 8 ? 0 : TILE_A) + row * ROWB;
    load_lds16(q < 8 ? ra : rb, dst, s == nk - 1 ? voff_last[q & 1] : voff[q & 1], row * K * 2 + kofs);
  };
  // fragment reads of sub-stage kk: row (l & 15) of a 16-row block,
  // granule 4 kk + (l >> 4)
  int fo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) fo[kk] = (lane & 15) * ROWB + (((4 * kk + (lane >> 4)) ^ ((lane & 15) >> 1)) << 4);
  const int wm = wave >> 1, wn = wave & 1;
  // read r (0..15) of sub-stage u, in the order its first products use them:
  // b0, a0..a3, b1, a4..a7, b2..b7
  auto rd = [&](bf16x8 (&an)[8], bf16x8 (&bn)[8], int r, int u) {
    const char* st = smem + ((u >> 1) & 1) * STAGE + fo[u & 1];
    if (r == 0) bn[0] = *reinterpret_cast<const bf16x8*>(st + TILE_A + (128 * wn) * ROWB);
    else if (r <= 4) an[r - 1] = *reinterpret_cast<const bf16x8*>(st + (128 * wm + 16 * (r - 1)) * ROWB);
    else if (r == 5) bn[1] = *reinterpret_cast<const bf16x8*>(st + TILE_A + (128 * wn + 16) * ROWB);
    else if (r <= 9) an[r - 2] = *reinterpret_cast<const bf16x8*>(st + (128 * wm + 16 * (r - 2)) * ROWB);
    else bn[r - 8] = *reinterpret_cast<const bf16x8*>(st + TILE_A + (128 * wn + 16 * (r - 8)) * ROWB);
  };
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Sub-stage u (k 32 u .. +31) of LDS stage t = u >> 1.  The last one of a
  // stage (odd u), after its first half, waits for stage t + 1's loads and
  // this wave's reads and meets the other waves at the barrier: stage t's
  // buffer is then free, and the first half of its refill (stage t + 2)
  // goes out during the second half; the other half goes out during the
  // first half of the next sub-stage, so the loads do not come in one burst.
  auto step = [&](const bf16x8 (&a)[8], const bf16x8 (&b)[8], bf16x8 (&an)[8], bf16x8 (&bn)[8], int u, auto last) {
    constexpr bool LAST = decltype(last)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_acc(acc[i][j], b[i], a[j]);
      if constexpr (!LAST) {
        if (u > 0) dma(8 + i, (u >> 1) + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LAST) {
      wait_lgkm0_vm<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mfma_acc(acc[q][4], b[q], a[4]);
      mfma_acc(acc[q][5], b[q], a[5]);
      rd(an, bn, 2 * q, u + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(acc[q][6], b[q], a[6]);
      mfma_acc(acc[q][7], b[q], a[7]);
      rd(an, bn, 2 * q + 1, u + 1);
      if constexpr (LAST) dma(q, (u >> 1) + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    hold(a, b);
  };
  using no = std::integral_constant<bool, false>;
  using yes = std::integral_constant<bool, true>;
  bf16x8 a0[8], b0[8], a1[8], b1[8];
#pragma unroll
  for (int q = 0; q < 16; ++q) dma(q, 0);
#pragma unroll
  for (int q = 0; q < 16; ++q) dma(q, 1);
  wait_lgkm0_vm<16>();   // stage 0 landed (stage 1 may be in flight)
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int r = 0; r < 16; ++r) rd(a0, b0, r, 0);
  for (int s = 0; s + 1 < nk; ++s) {
    step(a0, b0, a1, b1, 2 * s, no{});
    step(a1, b1, a0, b0, 2 * s + 1, yes{});
  }
  step(a0, b0, a1, b1, 2 * nk - 2, no{});
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) mfma_acc(acc[i][j], b1[i], a1[j]);
  wait_lgkm0_vm<0>();   // no load may still write this workgroup's LDS when it ends
  // acc[i][j]: lane holds columns n0 + 128 wn + 16 i + 4 (l >> 4) + e of row
  // m0 + 128 wm + 16 j + (l & 15); rows past M are outside the descriptor,
  // columns past N (N is a multiple of 4) are sent out of range
  const __amdgpu_buffer_rsrc_t rc = rsrc(C + (size_t)m0 * N, (unsigned)(min(BM, M - m0) * N * 2));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int col = n0 + 128 * wn + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 128 * wm + 16 * j + (lane & 15);
      const bf16x4 v{(bf16)acc[i][j][0], (bf16)acc[i][j][1], (bf16)acc[i][j][2], (bf16)acc[i][j][3]};
      const int vo = col < N ? (row * N + col) * 2 : kZeroOffset;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rc, vo, 0, 0);
    }
  }
}

}  // namespace

hipError_t gemm_nt_bf16(const bf16* A, const bf16* B, bf16* C, int M, int N, int K, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 8 || N % 4 || (long)BM * K * 2 >= (1L << 29) || (long)BM * N * 2 >= (1L << 31))
    return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_nt_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const long T = (long)tiles_m * tiles_n;
  const unsigned blocks = (unsigned)((T + 7) / 8 * 8);
  hipLaunchKernelGGL(gemm_nt_kernel, dim3(blocks), dim3(256), LDS_BYTES, st, A, B, C, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace prologue
}  // namespace atlas
