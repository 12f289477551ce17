// atlas_mem_coeff.h -- gate-coefficient kernel (device code), included by
// every translation unit that launches a chunk kernel.
#pragma once

#include <hip/hip_runtime.h>

#include "atlas_mem_internal.h"

namespace atlas {

// ----------------------------------------------------------------------------- coefficients
// One workgroup per (sequence, chunk), flattened on x.  256 threads; chunk <= 64.
// QD > 0: also compute Q1 = C .* (Xq X^T) for an identity feature map of
// width QD (window keys X, chunk queries Xq), stored as bf16 after C with
// row pitch q1_pitch(WP, CB16).  CB16: then also C itself as bf16.
template <int BC, int WP, int QD = 0, bool CB16 = false>
__global__ void __launch_bounds__(256) coeff_kernel(CoeffParams p) {
  const int chunk = (int)(blockIdx.x % (unsigned)p.nchunks), seq = (int)(blockIdx.x / (unsigned)p.nchunks);
  const int t0 = chunk * BC;
  const int te = min(p.N, t0 + BC) - 1;
  const int nb = te - t0 + 1;
  const int c = p.c;
  const size_t g0 = (size_t)seq * p.N;
  const int64_t cnt = *reinterpret_cast<const int64_t*>(p.state + (size_t)seq * p.seq_stride + p.off_count);
  const int halo_valid = (int)min<int64_t>(cnt, (int64_t)(c - 1));

  __shared__ float al[BC], et[BC], th[BC];
  // F[t][n] = K_{t,n} theta_n, turned into row prefix sums over n (fp64), so
  // that every window sum of C, cM, cS is one difference
  __shared__ double F[BC][BC + 1];
  __shared__ double G[BC + 1];      // prefix sums of e_{n->te} theta_n
  if (p.ctrl != nullptr && chunk == 0 && threadIdx.x == 0) {
    p.ctrl[1 + seq] = 0u;            // group barrier counter of this sequence
    p.ctrl[1 + gridDim.x / (unsigned)p.nchunks + seq] = 0u;   // XCDs its members ran on
    if (seq == 0) p.ctrl[0] = 0u;    // error word of the call
  }
  float* out = p.coef + ((size_t)seq * p.nchunks + chunk) * p.coef_stride;
  float* oA = out;
  float* oB = out + BC;
  float* oP = out + 2 * BC;
  float* ocM = out + 2 * BC + 4;
  float* ocS = ocM + WP;
  float* oC = ocS + WP;             // [BC][WP]

  // Q1's operands (keys of the window, queries of the chunk; bf16, 8 at a
  // time) are loaded into registers here, so that their latency passes while
  // the recurrences below run; they go to LDS one block of KB columns at a
  // time further down
  typedef __bf16 bx8 __attribute__((ext_vector_type(8)));
  constexpr int KB = 32, NKB = QD > 0 ? QD / KB : 1;
  // (256 threads: the launch size of this kernel)
  constexpr int NXE = (WP * (KB / 8) + 255) / 256, NQE = (BC * (KB / 8) + 255) / 256;   // per thread and block
  bx8 xr[NKB][NXE], qr[NKB][NQE];
  if constexpr (QD > 0) {
    static_assert(QD % KB == 0, "whole column blocks");
    const __bf16* kk = reinterpret_cast<const __bf16*>(p.k) + (size_t)seq * p.N * QD;
    const __bf16* qq = reinterpret_cast<const __bf16*>(p.q) + (size_t)seq * p.N * QD;
    const float* hk = reinterpret_cast<const float*>(p.state + (size_t)seq * p.seq_stride + p.off_halo_k);
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
#pragma unroll
      for (int j = 0; j < NXE; ++j) {
        const int e = (int)threadIdx.x + 256 * j;
        const int w = e / (KB / 8), d = b * KB + (e % (KB / 8)) * 8, i = t0 - (c - 1) + w;
        bx8 x;
        for (int z = 0; z < 8; ++z) x[z] = (__bf16)0.f;
        if (e < WP * (KB / 8) && w < BC + c - 1 && i >= -halo_valid && i <= te) {
          if (i >= 0) x = *reinterpret_cast<const bx8*>(kk + (size_t)i * QD + d);
          else
            for (int z = 0; z < 8; ++z) x[z] = (__bf16)hk[(c - 1 + i) * QD + d + z];
        }
        xr[b][j] = x;
      }
#pragma unroll
      for (int j = 0; j < NQE; ++j) {
        const int e = (int)threadIdx.x + 256 * j;
        const int n = e / (KB / 8), d = b * KB + (e % (KB / 8)) * 8;
        bx8 x;
        for (int z = 0; z < 8; ++z) x[z] = (__bf16)0.f;
        if (e < BC * (KB / 8) && n < nb) x = *reinterpret_cast<const bx8*>(qq + (size_t)(t0 + n) * QD + d);
        qr[b][j] = x;
      }
    }
  }

  for (int n = threadIdx.x; n < BC; n += blockDim.x) {
    const bool ok = n < nb;
    al[n] = ok ? p.alpha[g0 + t0 + n] : 0.f;
    et[n] = (ok && p.momentum) ? p.eta[g0 + t0 + n] : 0.f;
    th[n] = ok ? p.theta[g0 + t0 + n] : 0.f;
  }
  __syncthreads();
  __shared__ float Gv[BC];
  if (threadIdx.x < BC) {
    const int n = threadIdx.x;
    for (int t = 0; t < BC; ++t) F[t][n] = 0.0;
    if (n < nb) {
      float K = 1.f, e = 1.f;
      F[n][n] = th[n];
#pragma unroll 8
      for (int t = n + 1; t < nb; ++t) {
        e *= et[t];
        K = (1.f - al[t]) * K + e;
        F[t][n] = K * th[n];
      }
      Gv[n] = e * th[n];
    } else {
      Gv[n] = 0.f;
    }
  }
  if (threadIdx.x == 64) {
    float a = 1.f, b = 0.f, e0 = 1.f;
#pragma unroll 8
    for (int t = 0; t < BC; ++t) {
      if (t < nb) {
        a *= 1.f - al[t];
        e0 *= et[t];
        b = (1.f - al[t]) * b + e0;
        oA[t] = a;
        oB[t] = b;
      } else {
        oA[t] = 0.f;
        oB[t] = 0.f;
      }
    }
    oP[0] = e0;
  }
  __syncthreads();
  // row prefix sums: F[t][n] <- sum_{m <= n} F[t][m];  G[n + 1] = sum_{m <= n} Gv[m]
  if (threadIdx.x < BC) {
    const int t = threadIdx.x;
    double acc = 0.0;
#pragma unroll 8
    for (int n = 0; n < BC; ++n) {
      acc += F[t][n];
      F[t][n] = acc;
    }
  } else if (threadIdx.x == BC) {
    double acc = 0.0;
    G[0] = 0.0;
#pragma unroll 8
    for (int n = 0; n < BC; ++n) {
      acc += (double)Gv[n];
      G[n + 1] = acc;
    }
  }
  __syncthreads();
  // window row w <-> token i = t0 - (c-1) + w (relative to the call start):
  // C_{tt,w} = sum of F[tt][n] over n in [max(t0, i), min(t0 + tt, i + c - 1)]
  auto cval = [&](int tt, int w) -> float {
    const int i = t0 - (c - 1) + w;
    float s = 0.f;
    if (tt < nb && w < BC + c - 1 && i >= -halo_valid && i <= t0 + tt) {
      const int lo = max(t0, i) - t0, hi = min(t0 + tt, i + c - 1) - t0;
      s = (float)(F[tt][hi] - (lo > 0 ? F[tt][lo - 1] : 0.0));
    }
    return s;
  };
  // the fp32 C; its only reader with a bf16 copy (CB16) is this kernel, which
  // then takes every value straight from the prefix sums instead
  if constexpr (!CB16)
    for (int idx = threadIdx.x; idx < BC * WP; idx += blockDim.x) oC[idx] = cval(idx / WP, idx % WP);
  __syncthreads();
  if constexpr (QD > 0) {
    // Q1 = C .* (Xq X^T): bf16 MFMA, fp32 accumulation, 4 waves x 16x16
    // tiles.  Keys and queries pass through LDS one block of KB columns at a
    // time (a small footprint: three workgroups fit a CU instead of two), the
    // tile accumulators staying in registers across the blocks.
    typedef float fx4 __attribute__((ext_vector_type(4)));
    constexpr int L = KB + 8;
    __shared__ __attribute__((aligned(16))) __bf16 Xs[WP * L];
    __shared__ __attribute__((aligned(16))) __bf16 Qs[BC * L];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
    constexpr int NTL = (BC / 16) * (WP / 16), TPW = (NTL + 3) / 4;   // tiles, per wave
    fx4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = fx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < NKB; ++blk) {
      if (blk) __syncthreads();   // every wave is done with the previous block
#pragma unroll
      for (int jj = 0; jj < NXE; ++jj) {
        const int e = (int)threadIdx.x + 256 * jj;
        if (e < WP * (KB / 8)) *reinterpret_cast<bx8*>(Xs + (e / (KB / 8)) * L + (e % (KB / 8)) * 8) = xr[blk][jj];
      }
#pragma unroll
      for (int jj = 0; jj < NQE; ++jj) {
        const int e = (int)threadIdx.x + 256 * jj;
        if (e < BC * (KB / 8)) *reinterpret_cast<bx8*>(Qs + (e / (KB / 8)) * L + (e % (KB / 8)) * 8) = qr[blk][jj];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int t = wave + 4 * u;
        if (t >= NTL) break;
        const int m0 = 16 * (t / (WP / 16)), n0 = 16 * (t % (WP / 16));
        const bx8 a = *reinterpret_cast<const bx8*>(Qs + (m0 + c16) * L + 8 * g);
        const bx8 b = *reinterpret_cast<const bx8*>(Xs + (n0 + c16) * L + 8 * g);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[u], 0, 0, 0);
      }
    }
    __bf16* oQ = reinterpret_cast<__bf16*>(oC + BC * WP);
    constexpr int QP = q1_pitch(WP, CB16);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + 4 * u;
      if (t >= NTL) break;
      const int m0 = 16 * (t / (WP / 16)), n0 = 16 * (t % (WP / 16));
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 4 * g + r, col = n0 + c16;
        oQ[row * QP + col] = (__bf16)((CB16 ? cval(row, col) : oC[row * WP + col]) * acc[u][r]);
      }
    }
  }
  if constexpr (CB16) {
    __bf16* oCb = reinterpret_cast<__bf16*>(oC + BC * WP) + BC * q1_pitch(WP, CB16);
    for (int idx = threadIdx.x; idx < BC * WP; idx += blockDim.x) oCb[idx] = (__bf16)cval(idx / WP, idx % WP);
  }
  for (int w = threadIdx.x; w < WP; w += blockDim.x) {
    const int i = t0 - (c - 1) + w;
    float sm = 0.f, ss = 0.f;
    if (w < BC + c - 1 && i >= -halo_valid && i <= te) {
      const int lo = max(t0, i) - t0, hi = min(te, i + c - 1) - t0;
      sm = (float)(F[nb - 1][hi] - (lo > 0 ? F[nb - 1][lo - 1] : 0.0));
      ss = (float)(G[hi + 1] - G[lo]);
    }
    ocM[w] = sm;
    ocS[w] = ss;
  }
}

}  // namespace atlas
