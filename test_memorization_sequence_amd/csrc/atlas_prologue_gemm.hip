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
#include "atlas_prologue_math.h"

namespace atlas {
namespace prologue {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// The workgroup's tile: the hardware deals workgroups to the 8 XCDs round
// robin, so XCD x = blockIdx.x % 8 walks tiles [x T8, (x + 1) T8), in bands
// of GM row tiles, column by column.  False past the last tile.
__device__ __forceinline__ bool tile_of(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n, T8 = (T + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * T8 + (int)(blockIdx.x >> 3);
  if (t >= T) return false;
  const int band = t / (GM * tiles_n), in = t - band * GM * tiles_n;
  const int gm = min(GM, tiles_m - band * GM);
  tm = band * GM + in % gm;
  tn = in / gm;
  return true;
}

// acc = A_tile . B_tile^T over K for one 256 x 256 tile.  Row r of the A
// tile is at byte sa0 + r K 2 of ra, row r of the B tile at r K 2 of rb;
// rows and granules outside the descriptors read zeros.  Ends with no load
// in flight and every wave past its last LDS read of its own, but other
// waves may still read LDS: synchronise before reusing it.
__device__ __forceinline__ void tile_mma(char* smem, __amdgpu_buffer_rsrc_t ra, unsigned sa0, __amdgpu_buffer_rsrc_t rb,
                                         int K, int wave, int lane, f32x4 (&acc)[8][8]) {
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
    const unsigned so = (q < 8 ? sa0 : 0u) + (unsigned)(row * K * 2 + kofs);
    load_lds16(q < 8 ? ra : rb, dst, s == nk - 1 ? voff_last[q & 1] : voff[q & 1], (int)so);
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
  wait_lgkm0_vm<0>();   // no load may still write LDS after this
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_nt_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B, bf16* __restrict__ C, int M, int N, int K,
               int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  if (!tile_of(tiles_m, tiles_n, tm, tn)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  // operand tiles through descriptors sized to their rows: rows past M or N
  // read zeros
  const __amdgpu_buffer_rsrc_t ra = rsrc(A + (size_t)m0 * K, (unsigned)(min(BM, M - m0) * K * 2));
  const __amdgpu_buffer_rsrc_t rb = rsrc(B + (size_t)n0 * K, (unsigned)(min(BN, N - n0) * K * 2));
  f32x4 acc[8][8];
  tile_mma(smem, ra, 0u, rb, K, wave, lane, acc);
  const int wm = wave >> 1, wn = wave & 1;
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


// ---------------------------------------------------------------------------
// The whole prologue in one kernel: the projection tile stays on chip.
//
// Row tiles run along one sequence: tile tt of sequence b holds rows
// row0 = tt (256 - (K - 1)) .. + 255 of it, and writes the outputs of rows
// [K - 1, 256) (all 256 for tt = 0): the first K - 1 rows are the
// convolution's window, recomputed rather than fetched from the previous
// tile.  Rows past the sequence read zeros and are not written.  After the
// K loop the tile's projections go to LDS as bf16 (the values the two-kernel
// path writes to memory): 512-byte rows, 16-byte granule c of row t in slot
// c ^ (t & 15).
//
// q, k, v column tiles: each wave takes one head of the tile and a run of
// rows; lane l owns D / 64 adjacent channels, keeps their taps and a window
// of KP >= K rows in registers (the first KP - K taps zero: adding exact
// zeros first leaves every sum as it is) and walks the rows: convolution,
// SiLU, the lane's part of the row's sum of squares.  For q and k the parts
// of TB rows go to LDS; TB lanes each sum one row's 64 parts in the order of
// the two-kernel path's lane reduction (so both paths give the same bits)
// and hand back the row's scale 1 / max(|x|, 1e-12).
//
// The gate column tile (the 4 r columns after 3 H D): one thread per row,
// V_g (U_g x) as a pairwise sum in the order of the two-kernel path's lane
// butterfly, then the logistic; V and b staged in LDS.
constexpr int EPI_TB = 16;                               // rows per norm batch
constexpr int EPI_WAVE_FLOATS = EPI_TB * 64 + EPI_TB;    // parts and scales of one wave
constexpr int FUSED_LDS_BYTES = LDS_BYTES + 4 * EPI_WAVE_FLOATS * 4;
constexpr int GATE_PARAM_FLOATS = 4 * EPI_WAVE_FLOATS;   // the same block holds V and b for the gate tile

__device__ __forceinline__ const char* ptile(const char* P, int t, int c16) {
  return P + t * 512 + ((c16 ^ (t & 15)) << 4);
}

template <int R>
__device__ __forceinline__ void gate_rows(const FusedParams& p, const char* P, const float* prm, int b, int row0, int t,
                                          int nvalid) {
  // the products stay separate roundings, as in the lane butterfly (no
  // contraction into fused multiply-adds)
#pragma clang fp contract(off)
  if (t >= nvalid) return;
  float xg[4 * R];
#pragma unroll
  for (int c = 0; c < 4 * R; c += 4) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(ptile(P, t, c >> 3) + (c & 4) * 2);
    const bf16x4 v = __builtin_bit_cast(bf16x4, w);
#pragma unroll
    for (int e = 0; e < 4 && c + e < 4 * R; ++e) xg[c + e] = (float)v[e];
  }
  const size_t n = (size_t)row0 + t;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    for (int h = 0; h < p.H; ++h) {
      float u[R];
#pragma unroll
      for (int j = 0; j < R; ++j) u[j] = xg[g * R + j] * prm[(g * p.H + h) * R + j];
#pragma unroll
      for (int w = 1; w < R; w *= 2)
#pragma unroll
        for (int j = 0; j < R; j += 2 * w) u[j] = u[j] + u[j + w];
      p.gate[g][((size_t)b * p.H + h) * p.N + n] = sigm(u[0] + prm[4 * p.H * R + g * p.H + h]);
    }
}

template <int D, int KP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fused_prologue_kernel(FusedParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int DPL = D / 64, HPT = BN / D, WPH = 4 / HPT, TB = EPI_TB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  if (!tile_of(p.tiles_m, p.tiles_n, tm, tn)) return;
  const int b = tm / p.tps, tt = tm - b * p.tps;
  const int K = p.K, halo = K - 1;
  const int row0 = tt * (BM - halo), n0 = tn * BN;
  const int dm = p.dm;
  const int HD = p.H * D;
  const bool gate_tile = n0 >= 3 * HD;
  float* blk = reinterpret_cast<float*>(smem + LDS_BYTES);   // norm parts, or the gate parameters
  if (gate_tile) {
    const int nv = 4 * p.H * p.r;
    for (int i = tid; i < nv + 4 * p.H; i += 256) blk[i] = i < nv ? p.gv[i] : p.gb[i - nv];
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.x + (size_t)b * p.N * dm, (unsigned)p.N * dm * 2);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.w + (size_t)n0 * dm, (unsigned)(min(BN, p.ncol - n0) * dm * 2));
  f32x4 acc[8][8];
  tile_mma(smem, ra, (unsigned)row0 * dm * 2, rb, dm, wave, lane, acc);
  __syncthreads();   // every wave past its reads of the operand stages
  {
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // four columns 4 cg .. +3 of row t: half cg & 1 of granule cg >> 1
        const int t = 128 * wm + 16 * j + (lane & 15), cg = 32 * wn + 4 * i + (lane >> 4);
        const bf16x4 v{(bf16)acc[i][j][0], (bf16)acc[i][j][1], (bf16)acc[i][j][2], (bf16)acc[i][j][3]};
        *reinterpret_cast<u32x2*>(const_cast<char*>(ptile(smem, t, cg >> 1)) + (cg & 1) * 8) = __builtin_bit_cast(u32x2, v);
      }
  }
  __syncthreads();
  const int nvalid = min(BM, p.N - row0);
  const int out_lo = tt == 0 ? 0 : halo;
  if (gate_tile) {
    const int t = out_lo + tid;
    switch (p.r) {
      case 1: gate_rows<1>(p, smem, blk, b, row0, t, nvalid); break;
      case 2: gate_rows<2>(p, smem, blk, b, row0, t, nvalid); break;
      case 4: gate_rows<4>(p, smem, blk, b, row0, t, nvalid); break;
      case 8: gate_rows<8>(p, smem, blk, b, row0, t, nvalid); break;
      default: gate_rows<16>(p, smem, blk, b, row0, t, nvalid); break;
    }
    return;
  }
  // this wave's head and run of rows
  const int hh = wave / WPH, part = wave - hh * WPH;
  const int c0 = n0 + hh * D;   // the head's first projection column
  const int m = c0 / HD, h = (c0 - m * HD) / D;
  const int len = nvalid - out_lo;
  const int t_beg = out_lo + (part * len) / WPH, t_end = out_lo + ((part + 1) * len) / WPH;
  const int col = hh * D + lane * DPL;   // tile column of this lane's first channel
  float tz[DPL][KP], win[DPL][KP];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const float* wc = p.w_conv + (size_t)(c0 + lane * DPL + i) * K;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int jj = j - (KP - K);
      tz[i][j] = jj >= 0 ? wc[jj] : 0.f;
    }
  }
  // the lane's byte within a row before the swizzle (granule col >> 3, byte
  // (col & 7) 2): the slot is the granule ^ (t & 15), one xor-add per row
  const int lb = ((col >> 3) << 4) | ((col & 7) * 2);
  auto ld = [&](int t, float (&x)[DPL]) {
    const char* a = smem + ((lb ^ ((t & 15) << 4)) + t * 512);
    if constexpr (DPL == 1) {
      x[0] = (float)*reinterpret_cast<const bf16*>(a);
    } else if constexpr (DPL == 2) {
      const bf16x2 v = *reinterpret_cast<const bf16x2*>(a);
      x[0] = (float)v[0];
      x[1] = (float)v[1];
    } else {
      const bf16x4 v = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(a));
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (float)v[i];
    }
  };
  // the window before the first row: rows t_beg - KP + 1 .. t_beg - 1 in
  // entries 1 .. KP - 1 (rows before the sequence: zero; rows before the
  // tile meet only zero taps)
#pragma unroll
  for (int j = 1; j < KP; ++j) {
    const int t = t_beg - KP + j;
    float x[DPL];
    ld(max(t, 0), x);
#pragma unroll
    for (int i = 0; i < DPL; ++i) win[i][j] = t >= 0 ? x[i] : 0.f;
  }
  float* parts = blk + wave * EPI_WAVE_FLOATS;   // [TB][64] parts, then TB scales
  // this head's output rows through a descriptor: the row offset is the
  // same for every lane (a scalar offset), the lane's channels a fixed one
  const __amdgpu_buffer_rsrc_t ro =
      rsrc((m == 0 ? p.q : m == 1 ? p.k : p.v) + ((size_t)b * p.H + h) * p.N * D, (unsigned)(p.N * D * 2));
  const int ovoff = lane * DPL * 2;
  for (int tb = t_beg; tb < t_end; tb += TB) {
    float x[TB][DPL], o[TB][DPL];
#pragma unroll
    for (int u = 0; u < TB; ++u) ld(min(tb + u, t_end - 1), x[u]);
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
#pragma unroll
        for (int j = 0; j + 1 < KP; ++j) win[i][j] = win[i][j + 1];
        win[i][KP - 1] = x[u][i];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < KP; ++j) a = fmaf(tz[i][j], win[i][j], a);
        o[u][i] = silu(a);
        q = fmaf(o[u][i], o[u][i], q);
      }
      parts[u * 64 + lane] = q;
    }
    float scale[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) scale[u] = 1.f;
    if (m < 2) {
      // lane 4 u + g: group g of row tb + u's 64 parts, summed as
      // group_sum(16) leaves it in lane 0 of that row; then the four groups'
      // totals meet as (g0 + g1) + (g2 + g3) by quad moves
      asm volatile("" ::: "memory");
      {
        static_assert(TB == 16, "four lanes per row of the batch");
        const int u = lane >> 2, g = lane & 3;
        const float* v = parts + u * 64 + 16 * g;
        const float4 p0 = *reinterpret_cast<const float4*>(v);
        const float4 p1 = *reinterpret_cast<const float4*>(v + 4);
        const float4 p2 = *reinterpret_cast<const float4*>(v + 8);
        const float4 p3 = *reinterpret_cast<const float4*>(v + 12);
        const float rg = (((p0.x + p0.y) + (p0.z + p0.w)) + ((p1.x + p1.y) + (p1.z + p1.w))) +
                         (((p2.x + p2.y) + (p2.z + p2.w)) + ((p3.x + p3.y) + (p3.z + p3.w)));
        const float pair = rg + dppf<0xB1>(rg);      // g0 + g1 in lane g = 0, g2 + g3 in lane g = 2
        const float ss = pair + dppf<0x4E>(pair);    // (g0 + g1) + (g2 + g3) in lane g = 0
        if (g == 0) parts[TB * 64 + u] = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(|x|, 1e-12)
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < TB; u += 4) {
        const float4 sc = *reinterpret_cast<const float4*>(parts + TB * 64 + u);
        scale[u] = sc.x;
        scale[u + 1] = sc.y;
        scale[u + 2] = sc.z;
        scale[u + 3] = sc.w;
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tb + u;
      if (t >= t_end) break;
      const int so = (row0 + t) * D * 2;
      if constexpr (DPL == 1) {
        const bf16 y = (bf16)(o[u][0] * scale[u]);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, y), ro, ovoff, so, 0);
      } else if constexpr (DPL == 2) {
        const bf16x2 y{(bf16)(o[u][0] * scale[u]), (bf16)(o[u][1] * scale[u])};
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, y), ro, ovoff, so, 0);
      } else {
        const bf16x4 y{(bf16)(o[u][0] * scale[u]), (bf16)(o[u][1] * scale[u]), (bf16)(o[u][2] * scale[u]),
                       (bf16)(o[u][3] * scale[u])};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), ro, ovoff, so, 0);
      }
    }
    asm volatile("" ::: "memory");   // this batch's reads of the parts before the next batch's writes
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


bool fused_supported(int d_head, int heads, int gate_rank, int seq_len, int d_model) {
  if (d_head != 64 && d_head != 128 && d_head != 256) return false;
  if ((3L * heads * d_head) % BN != 0 || 4 * gate_rank > BN) return false;
  if (4L * heads * (gate_rank + 1) > GATE_PARAM_FLOATS) return false;   // the gate tile's V and b in LDS
  // one sequence's rows through a 32-bit descriptor, with room for the
  // scalar offsets that send loads past it
  // (and one head's output rows through another)
  return (long)seq_len * d_model * 2 < (1L << 30) && (long)BM * d_model * 2 < (1L << 29) &&
         (long)seq_len * d_head * 2 < (1L << 31);
}

hipError_t fused_prologue(const FusedParams& p0, int d_head, hipStream_t st) {
  if (p0.B <= 0 || p0.N <= 0) return hipSuccess;
  FusedParams p = p0;
  const int halo = p.K - 1;
  p.tps = 1 + (p.N > BM ? (p.N - BM + (BM - halo) - 1) / (BM - halo) : 0);
  p.tiles_m = p.B * p.tps;
  p.tiles_n = (p.ncol + BN - 1) / BN;
  const long T = (long)p.tiles_m * p.tiles_n;
  const unsigned blocks = (unsigned)((T + 7) / 8 * 8);
  const bool k8 = p.K > 4;
#define ATLAS_FUSED(DD, KK)                                                                                      \
  if (d_head == DD && (KK == 8) == k8) {                                                                        \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_prologue_kernel<DD, KK>),             \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, FUSED_LDS_BYTES);              \
    if (e != hipSuccess) return e;                                                                               \
    hipLaunchKernelGGL((fused_prologue_kernel<DD, KK>), dim3(blocks), dim3(256), FUSED_LDS_BYTES, st, p);         \
  }
  ATLAS_FUSED(64, 4)
  ATLAS_FUSED(64, 8)
  ATLAS_FUSED(128, 4)
  ATLAS_FUSED(128, 8)
  ATLAS_FUSED(256, 4)
  ATLAS_FUSED(256, 8)
#undef ATLAS_FUSED
  return hipGetLastError();
}

}  // namespace prologue
}  // namespace atlas
