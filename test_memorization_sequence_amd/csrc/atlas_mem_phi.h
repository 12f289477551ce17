// atlas_mem_phi.h -- the feature map phi of every key and query, and Q1, for
// the kernels that take phi precomputed per call (device code, included by
// the MLP and the linear recurrences of that family).
//
// phi (ATLAS review sec. 3.1 "Polynomial Feature Mapping"): the identity,
// [k, upper-tri(k k^T)] or [k, poly2(k[:p])], each feature from the raw bf16
// key as an fp32 product, stored bf16.  Q1 = C .* (phi(Q) phi(K)^T) of every
// chunk, C the coefficient block's fp32 band (Titans review sec. 3.1,
// "Retrieving a Memory": the per-token weights applied to a query).
//
// A shape S provides DK, PD, PHI, D, DP (features padded to a multiple of
// 64), BC, WP, rows_k, oXR, oXT, oXQ (byte offsets of the key rows, the
// feature-major key copy and the query rows in a sequence's workspace) and
// xMask (a word the phi kernel clears before the recurrence starts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atlas_mem_internal.h"
#include "atlas_mem_frag.h"

namespace atlas {
namespace grouped {

using namespace mfma;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// v_mfma_f32_16x16x16_bf16: lane l supplies row (l & 15) and k = 4 (l >> 4) .. +3
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0,
                                                   0);
}
// K16 operand of row n0 + (l & 15) of the transpose of a k-major LDS matrix M[k][n]
__device__ __forceinline__ bf16x4 ld_tr16(const bf16* M, int ld, int n0, int k0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  return __builtin_bit_cast(bf16x4, tr4(M + (k0 + 4 * g + (s >> 2)) * ld + n0 + 4 * (s & 3)));
}
__device__ __forceinline__ bf16x8 gload8(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ float gload1(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void gstore1(float v, __amdgpu_buffer_rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, 0, 0);
}


// ----------------------------------------------------------------------------- phi kernel
// Degree-2 block: pair index p -> (a, b), a <= b < P, row-major upper triangle
// (row a starts at off(a) = a P - a (a - 1) / 2): the root of the quadratic,
// then a correction of the float estimate by one row either way.
template <int P>
__device__ __forceinline__ void pair_of(int p, int& a, int& b) {
  constexpr float B2 = 2.f * P + 1.f;
  int aa = (int)((B2 - sqrtf(B2 * B2 - 8.f * (float)p)) * 0.5f);
  aa = max(0, min(P - 1, aa));
  auto off = [](int x) { return x * P - x * (x - 1) / 2; };
  if (off(aa) > p) --aa;
  else if (aa + 1 < P && off(aa + 1) <= p) ++aa;
  a = aa;
  b = aa + p - off(aa);
}

// Where feature f of phi comes from: zero (kind 0), raw component a (kind 1)
// or the product of raw components a and b (kind 2).
struct FeatureSrc { int kind, a, b; };
template <class S>
__device__ __forceinline__ FeatureSrc feature_src(int f) {
  if (f < S::DK) return {1, f, 0};
  if constexpr (S::PHI == PHI_POLY2) {
    if (f < S::D) { FeatureSrc r{2, 0, 0}; pair_of<S::DK>(f - S::DK, r.a, r.b); return r; }
  } else if constexpr (S::PHI == PHI_RAW_POLY2) {
    if (f < S::DK + S::PD) return {1, f - S::DK, 0};
    if (f < S::D) { FeatureSrc r{2, 0, 0}; pair_of<S::PD>(f - S::DK - S::PD, r.a, r.b); return r; }
  }
  return {0, 0, 0};
}
// The value of one feature from a raw row in LDS (products in fp32).
__device__ __forceinline__ float feature_val(const float* row, const FeatureSrc& fs) {
  if (fs.kind == 0) return 0.f;
  const float x = row[fs.a];
  return fs.kind == 1 ? x : x * row[fs.b];
}

// Blocks of 32 tokens: per sequence rows_k(nch) / 32 key blocks (key row i is
// token i - (c - 1): the input for tokens of the call, the state's halo for
// earlier tokens the sequence has seen, else zero), then 2 nch query blocks.
// The raw rows go to LDS as floats; each thread then writes 16 bytes at a
// time: 8 consecutive features of one row, or (keys) 8 consecutive tokens of
// one feature of the feature-major copy.
template <class S>
__global__ void __launch_bounds__(256) phi_kernel(GroupedParams p) {
  constexpr int DK = S::DK, DP = S::DP, F8 = DP / 8, RB = 32;
  __shared__ float raw[RB][DK + 1];
  const int nch = p.nchunks, NR = (int)S::rows_k(nch), kb = NR / RB, per_seq = kb + 2 * nch;
  const int seq = (int)(blockIdx.x / (unsigned)per_seq), blk = (int)(blockIdx.x % (unsigned)per_seq);
  const bool keys = blk < kb;
  const int r0 = RB * (keys ? blk : blk - kb);
  const int N = p.N, c1 = p.c - 1;
  const char* st = p.state + (size_t)seq * p.seq_stride;
  const int64_t cnt = *reinterpret_cast<const int64_t*>(st + p.off_count);
  const int halo_valid = (int)min<int64_t>(cnt, (int64_t)c1);
  const float* hk = reinterpret_cast<const float*>(st + p.off_halo_k);
  const bf16* src = reinterpret_cast<const bf16*>(keys ? p.k : p.q) + (size_t)seq * N * DK;
  char* ws = p.gws + (size_t)seq * p.gseq_bytes;
  if (blk == 0 && threadIdx.x == 0)   // before the recurrence starts: no member has reported yet
    *reinterpret_cast<unsigned*>(ws + S::xMask) = 0u;
  for (int e = threadIdx.x; e < RB * (DK / 8); e += 256) {
    const int r = e / (DK / 8), d8 = (e % (DK / 8)) * 8;
    const int tok = keys ? r0 + r - c1 : r0 + r;
    float x[8];
    if (tok >= 0 && tok < N) {
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(src + (size_t)tok * DK + d8);
#pragma unroll
      for (int z = 0; z < 8; ++z) x[z] = (float)v8[z];
    } else {
      const bool h = keys && tok < 0 && tok >= -halo_valid;
#pragma unroll
      for (int z = 0; z < 8; ++z) x[z] = h ? (float)(bf16)hk[(c1 + tok) * DK + d8 + z] : 0.f;
    }
#pragma unroll
    for (int z = 0; z < 8; ++z) raw[r][d8 + z] = x[z];
  }
  __syncthreads();
  bf16* rows = reinterpret_cast<bf16*>(ws + (keys ? S::oXR(nch) : S::oXQ(nch)));
  for (int e = threadIdx.x; e < RB * F8; e += 256) {
    const int r = e / F8, f0 = (e % F8) * 8;
    bf16x8 v;
#pragma unroll
    for (int z = 0; z < 8; ++z) v[z] = (bf16)feature_val(raw[r], feature_src<S>(f0 + z));
    *reinterpret_cast<bf16x8*>(rows + (size_t)(r0 + r) * DP + f0) = v;
  }
  if (keys) {
    bf16* cols = reinterpret_cast<bf16*>(ws + S::oXT(nch));
    for (int e = threadIdx.x; e < DP * (RB / 8); e += 256) {
      const int f = e / (RB / 8), t8 = (e % (RB / 8)) * 8;
      const FeatureSrc fs = feature_src<S>(f);
      bf16x8 v;
#pragma unroll
      for (int z = 0; z < 8; ++z) v[z] = (bf16)feature_val(raw[t8 + z], fs);
      *reinterpret_cast<bf16x8*>(cols + (size_t)f * NR + r0 + t8) = v;
    }
  }
}

// ----------------------------------------------------------------------------- Q1 kernel
// One workgroup per (sequence, chunk): Q1[t][w] = C[t][w] (phi(q_t) . phi(k_w))
// for window row w, bf16 after the fp32 C of the coefficient block.
template <class S>
__global__ void __launch_bounds__(256) q1_phi_kernel(GroupedParams p) {
  constexpr int DP = S::DP, BC = S::BC, WP = S::WP;
  const int ch = (int)(blockIdx.x % (unsigned)p.nchunks), seq = (int)(blockIdx.x / (unsigned)p.nchunks);
  const int nch = p.nchunks, t0 = ch * BC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const char* ws = p.gws + (size_t)seq * p.gseq_bytes;
  const __amdgpu_buffer_rsrc_t rk = buffer_of(ws + S::oXR(nch), (unsigned)(S::rows_k(nch) * DP * 2));
  const __amdgpu_buffer_rsrc_t rq = buffer_of(ws + S::oXQ(nch), (unsigned)((size_t)nch * BC * DP * 2));
  float* coef = p.coef + ((size_t)seq * nch + ch) * p.coef_stride;
  const float* C = coef + 2 * BC + 4 + 2 * WP;
  bf16* Q1 = reinterpret_cast<bf16*>(coef + 2 * BC + 4 + 2 * WP + BC * WP);
  // wave: query tile `wave`, all 8 window tiles
  f32x4 acc[WP / 16];
#pragma unroll
  for (int n = 0; n < WP / 16; ++n) acc[n] = zero4();
  const int qrow = t0 + 16 * wave + c16;
#pragma unroll 2
  for (int s = 0; s < DP / 32; ++s) {
    const bf16x8 a = gload8(rq, (qrow * DP + 32 * s + 8 * g) * 2);
#pragma unroll
    for (int n = 0; n < WP / 16; ++n)
      acc[n] = mma(a, gload8(rk, ((t0 + 16 * n + c16) * DP + 32 * s + 8 * g) * 2), acc[n]);
  }
#pragma unroll
  for (int n = 0; n < WP / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * wave + 4 * g + r, col = 16 * n + c16;
      Q1[row * WP + col] = (bf16)(C[row * WP + col] * acc[n][r]);
    }
}

}  // namespace grouped
}  // namespace atlas
