// atlas_mem_linear.hip -- the linear memory M [DV][D] on phi precomputed per
// call (the phi and Q1 kernels of atlas_mem_phi.h), one workgroup per
// sequence for the chunk chain and one per (sequence, chunk) for the
// retrieval.  Method as in atlas_mem_kernels.hip (the linear case): per chunk
// of BC tokens, the gradient of the Omega-rule window loss (ATLAS review
// sec. 3.2-3.3) at the chunk-start weights, folded into momentum and decay
// (Titans review sec. 3.1) through the gate coefficients A_t, B_t, C_{t,i},
// cM_i, cS_i, P; retrieval y_t = M_t phi(q_t) with the per-token weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atlas_mem_internal.h"
#include "atlas_mem_coeff.h"
#include "atlas_mem_frag.h"
#include "atlas_mem_phi.h"
#include "atlas_mem_linear.h"

namespace atlas {
namespace grouped {

using namespace mfma;

// ----------------------------------------------------------------------------- linear memory
// Linear memory M [DV][D] (Titans review sec. 3.1: matrix memory; ATLAS review
// sec. 3.1 for the feature map) on the same phi buffers and Q1 blocks.  The
// recurrence needs per chunk only the window forward, D and the update, so it
// runs on one workgroup per sequence with M and S fp32 in registers; it leaves
// the chunk-start images of M and S (bf16) and D of every chunk behind, and
// the retrieval then runs for all chunks at once:
//   linear_rec_kernel  Y = X M^T over the window rows at the chunk-start
//                      state, D = s gamma (Y - V) (dot bias: -s gamma V),
//                      M <- A_te M + B_te S - (cM .* D)^T X,
//                      S <- P S - (cS .* D)^T X;
//   linear_ret_kernel  y_t = A_t M0 phi(q_t) + B_t S0 phi(q_t) - sum_w Q1[t][w] D_w
//                      (M0, S0 the chunk-start state), one workgroup per
//                      (sequence, chunk).
template <int PHI_, int DK_, int PD_, int DV_, int WP_>
struct LShape {
  static constexpr int PHI = PHI_, DK = DK_, PD = PD_, DV = DV_, WP = WP_;
  static constexpr int D = feature_dim(PHI_, DK_, PD_);
  static constexpr int DP = (D + 63) / 64 * 64;   // features, padded to 4 waves x 16-row tiles
  static constexpr int BC = 64;
  static constexpr int NOT = DV / 16, NFT = DP / 16, NWT = WP / 16;
  static constexpr int YPW = NOT * NWT / 4;       // window-forward tiles per wave
  static constexpr int FPW = NFT / 4;             // update feature tiles per wave
  static_assert(DV % 16 == 0 && (NOT * NWT) % 4 == 0, "value tiles");
  static_assert(WP % 32 == 0 && WP >= BC && WP <= 128, "window rows");
  static_assert(DK % 8 == 0, "phi rows");
  static_assert(FPW * NOT <= 18, "state registers: 8 FPW NOT per lane");
  // LDS (bf16 pitches: multiples of 8, 16-byte rows)
  static constexpr int LF = DP + 8, LV = DV + 8;
  static constexpr size_t oMi = 0;                                  // M image [DV][LF]
  static constexpr size_t oD2 = oMi + align_up(DV * LF * 2, 256);   // D [WP][LV]
  // two coefficient sets by chunk parity, each the head of the coefficient
  // block as the coefficient kernel writes it: A[BC] B[BC] P (+3) cM[WP] cS[WP]
  static constexpr size_t oF = oD2 + align_up(WP * LV * 2, 256);
  static constexpr int NCF = 2 * BC + 2 * WP + 4;
  // the window's feature-major rows X^T [DP][WP] for the update, when they fit
  static constexpr size_t oXTl = oF + align_up(2 * NCF * 4, 256);
  static constexpr bool XT_LDS = oXTl + (size_t)DP * WP * 2 <= 163840;
  static constexpr size_t lds = XT_LDS ? oXTl + (size_t)DP * WP * 2 : oF + 2 * NCF * 4;
  static_assert(lds <= 163840, "LDS budget of one CU");
  // workspace per sequence (bytes): a word the phi kernel clears (unused
  // here), the chunk-start images [nch][2][DV][DP] (M, then S), D of every
  // chunk [nch][WP][DV], then the phi buffers as in the MLP shapes
  static constexpr size_t xMask = 0;
  // element (o, f) of a chunk-start image (M or S, DV x DP bf16): feature
  // quad f / 4 major, then o % 16, then the value tile o / 16, then f % 4
  static_assert(NOT % 2 == 0, "images are stored 8 values at a time");
  __host__ __device__ static size_t img_pos(int o, int f) {
    return ((size_t)(f >> 2) * 16 + (o & 15)) * (4 * NOT) + (o >> 4) * 4 + (f & 3);
  }
  __host__ __device__ static size_t rows_k(int nch) { return (size_t)nch * BC + BC; }
  __host__ __device__ static size_t oImg(int) { return 256; }
  __host__ __device__ static size_t oDg(int nch) { return align_up(oImg(nch) + (size_t)nch * 2 * DV * DP * 2, 256); }
  __host__ __device__ static size_t oXR(int nch) { return align_up(oDg(nch) + (size_t)nch * WP * DV * 2, 256); }
  __host__ __device__ static size_t oXT(int nch) { return align_up(oXR(nch) + rows_k(nch) * DP * 2, 256); }
  __host__ __device__ static size_t oXQ(int nch) { return align_up(oXT(nch) + rows_k(nch) * DP * 2, 256); }
  __host__ __device__ static size_t seq_bytes(int nch) { return align_up(oXQ(nch) + (size_t)nch * BC * DP * 2, 256); }
};

// Buffer load of 16 bytes per lane that writes LDS directly (lane l's bytes
// to dst + 16 l, dst wave-uniform), at byte offset voff + soff (soff
// wave-uniform); completion is counted by vmcnt like any load.
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, void* dst, int voff, int soff) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

// X^T rows [DP][WP] of one window into LDS (row-major, pitch WP) by direct
// loads of 1 KB per wave instruction.  J instructions cover exactly R rows, so
// each lane's J byte offsets are fixed for the call and only a wave-uniform
// offset moves with the super block and the window.
template <class S>
struct XtStage {
  static constexpr int RB = S::WP * 2;   // bytes per row
  static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
  static constexpr int J = RB / gcd(RB, 1024);   // lcm(RB, 1024) / 1024
  static constexpr int R = J * 1024 / RB;
  static constexpr int NSB = S::DP / R;
  static_assert(S::DP % R == 0 && NSB % 4 == 0, "whole super blocks, the same count per wave");
};

template <class S>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
linear_rec_kernel(GroupedParams p) {
  constexpr int DK = S::DK, DV = S::DV, D = S::D, DP = S::DP, BC = S::BC, WP = S::WP;
  constexpr int NOT = S::NOT, YPW = S::YPW, FPW = S::FPW, LF = S::LF, LV = S::LV, NCF = S::NCF;
  extern __shared__ __attribute__((aligned(256))) char smem[];
  const int seq = (int)blockIdx.x;
  if (seq >= p.n_seq) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int N = p.N, c = p.c, W = BC + c - 1, nch = p.nchunks;
  const bool mom = p.momentum != 0, dot = p.bias == BIAS_DOT;
  const float s_grad = p.grad_scale;

  char* st = p.state + (size_t)seq * p.seq_stride;
  float* Wt = reinterpret_cast<float*>(st + p.off_weights);
  float* Mo = reinterpret_cast<float*>(st + p.off_momentum);
  float* hk = reinterpret_cast<float*>(st + p.off_halo_k);
  float* hv = reinterpret_cast<float*>(st + p.off_halo_v);
  float* hg = reinterpret_cast<float*>(st + p.off_halo_g);
  int64_t* cnt = reinterpret_cast<int64_t*>(st + p.off_count);
  const int halo_valid = (int)min<int64_t>(*cnt, (int64_t)(c - 1));
  const bf16* k = reinterpret_cast<const bf16*>(p.k) + (size_t)seq * N * DK;
  const bf16* v = reinterpret_cast<const bf16*>(p.v) + (size_t)seq * N * DV;
  const float* gam_in = p.gamma + (size_t)seq * N;

  char* ws = p.gws + (size_t)seq * p.gseq_bytes;
  const size_t NR = S::rows_k(nch);
  const __amdgpu_buffer_rsrc_t rxr = buffer_of(ws + S::oXR(nch), (unsigned)(NR * DP * 2));
  const __amdgpu_buffer_rsrc_t rxt = buffer_of(ws + S::oXT(nch), (unsigned)(NR * DP * 2));
  bf16* img = reinterpret_cast<bf16*>(ws + S::oImg(nch));
  bf16* dg = reinterpret_cast<bf16*>(ws + S::oDg(nch));

  bf16* Mi = reinterpret_cast<bf16*>(smem + S::oMi);
  bf16* D2l = reinterpret_cast<bf16*>(smem + S::oD2);
  float* cf = reinterpret_cast<float*>(smem + S::oF);   // two coefficient sets, by chunk parity
  bf16* XTl = reinterpret_cast<bf16*>(smem + S::oXTl);
  const float* coef0 = p.coef + (size_t)seq * nch * p.coef_stride;

  // ---- state into registers: MT[m][o][r] = M[16 o + c16][16 (wave + 4 m) + 4 g + r], same for S
  f32x4 MT[FPW][NOT], ST[FPW][NOT];
  {
    const __amdgpu_buffer_rsrc_t rw = buffer_of(Wt, (unsigned)((size_t)DV * D * 4));
    const __amdgpu_buffer_rsrc_t rm = buffer_of(Mo, mom ? (unsigned)((size_t)DV * D * 4) : 0u);
#pragma unroll
    for (int m = 0; m < FPW; ++m)
#pragma unroll
      for (int o = 0; o < NOT; ++o)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * (wave + 4 * m) + 4 * g + r;
          const int off = f < D ? ((16 * o + c16) * D + f) * 4 : kZeroOffset;
          MT[m][o][r] = gload1(rw, off);
          ST[m][o][r] = gload1(rm, off);
        }
  }
  // images of the chunk-start state of chunk chn: M into LDS [o][f] (the
  // window forward's operand); M and S into the workspace (the retrieval's)
  // in the quad-major order of S::img_pos, where a lane's values for all
  // value tiles at one feature quad are adjacent and a wave's store covers
  // one contiguous 64 NOT-element run
  auto write_images = [&](int chn) {
    bf16* im = img + (size_t)chn * 2 * DV * DP;
#pragma unroll
    for (int m = 0; m < FPW; ++m) {
      const int f0 = 16 * (wave + 4 * m) + 4 * g;
      bf16 wq[4 * NOT], sq[4 * NOT];
#pragma unroll
      for (int o = 0; o < NOT; ++o) {
        const int orow = 16 * o + c16;
        const bf16x4 wv{(bf16)MT[m][o][0], (bf16)MT[m][o][1], (bf16)MT[m][o][2], (bf16)MT[m][o][3]};
        *reinterpret_cast<bf16x4*>(Mi + orow * LF + f0) = wv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          wq[4 * o + r] = wv[r];
          sq[4 * o + r] = (bf16)ST[m][o][r];
        }
      }
      const size_t q0 = S::img_pos(c16, f0);
#pragma unroll
      for (int h = 0; h < NOT / 2; ++h) {
        *reinterpret_cast<bf16x8*>(im + q0 + 8 * h) = *reinterpret_cast<const bf16x8*>(wq + 8 * h);
        *reinterpret_cast<bf16x8*>(im + (size_t)DV * DP + q0 + 8 * h) = *reinterpret_cast<const bf16x8*>(sq + 8 * h);
      }
    }
  };
  write_images(0);

  // Per chunk: the window forward, D, the update; then, at the end of the
  // chunk, everything the next one needs that does not depend on the state:
  // its coefficients and window values (registers), and, where they fit, its
  // X^T rows (LDS, by direct loads; the window forward reads X from them
  // through transposed LDS reads).  Those loads are issued after the image
  // stores and waited for before the next chunk's first barrier, so store
  // drain and load latency overlap.
  constexpr int NCR = (NCF + 255) / 256;
  const __amdgpu_buffer_rsrc_t rv = buffer_of(v, (unsigned)((size_t)N * DV * 2));
  const __amdgpu_buffer_rsrc_t rgm = buffer_of(gam_in, (unsigned)((size_t)N * 4));
  const __amdgpu_buffer_rsrc_t rhv = buffer_of(hv, (unsigned)((c - 1) * DV * 4));
  const __amdgpu_buffer_rsrc_t rhg = buffer_of(hg, (unsigned)((c - 1) * 4));
  // this lane's byte offsets in X^T for the staging of a window
  int xt_voff[XtStage<S>::J];
#pragma unroll
  for (int j = 0; j < XtStage<S>::J; ++j) {
    const int off = j * 1024 + lane * 16;
    xt_voff[j] = (off / XtStage<S>::RB) * (int)NR * 2 + off % XtStage<S>::RB;
  }
  float cnext[NCR];
  float4 pv[YPW];
  float pg[YPW];
  auto fetch = [&](int chn) {
    const int t0n = chn * BC, ten = min(N, t0n + BC) - 1;
    const float* cn = coef0 + (size_t)chn * p.coef_stride;
#pragma unroll
    for (int u = 0; u < NCR; ++u) cnext[u] = tid + 256 * u < NCF ? cn[tid + 256 * u] : 0.f;
    // branch-free: both sources are read through range-checked descriptors;
    // the one not meant reads zero at an offset out of range, so the sum is
    // the valid value
#pragma unroll
    for (int u = 0; u < YPW; ++u) {
      const int ot = (wave + 4 * u) % NOT, wt = (wave + 4 * u) / NOT;
      const int w = 16 * wt + c16, o4 = 16 * ot + 4 * g;
      const int i = t0n - (c - 1) + w;
      const bool valid = w < W && i >= -halo_valid && i <= ten;
      const bool cur = valid && i >= 0, old = valid && i < 0;
      const u32x2 vv = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
          rv, cur ? (i * DV + o4) * 2 : kZeroOffset, 0, 0));
      const f32x4 hv4 = buf_load4(rhv, old ? ((c - 1 + i) * DV + o4) * 4 : kZeroOffset, 0);
      const float gc = gload1(rgm, cur ? i * 4 : kZeroOffset);
      const float gh = gload1(rhg, old ? (c - 1 + i) * 4 : kZeroOffset);
      const bf16x4 vb = __builtin_bit_cast(bf16x4, vv);
      pv[u] = make_float4((float)vb[0] + hv4[0], (float)vb[1] + hv4[1], (float)vb[2] + hv4[2], (float)vb[3] + hv4[3]);
      pg[u] = gc + gh;
    }
    if constexpr (S::XT_LDS) {
      typedef XtStage<S> X;
#pragma unroll
      for (int k = 0; k < X::NSB / 4; ++k) {
        const int sb = wave + 4 * k;
        const int soff = (sb * X::R * (int)NR + t0n) * 2;
#pragma unroll
        for (int j = 0; j < X::J; ++j)
          buf_load_lds16(rxt, reinterpret_cast<char*>(XTl) + (sb * X::J + j) * 1024, xt_voff[j], soff);
      }
    }
  };
  auto store_coef = [&](int chn) {
    float* cn = cf + (chn & 1) * NCF;
#pragma unroll
    for (int u = 0; u < NCR; ++u)
      if (tid + 256 * u < NCF) cn[tid + 256 * u] = cnext[u];
  };
  fetch(0);
  wait_vmem();
  store_coef(0);

  for (int ch = 0; ch < nch; ++ch) {
    const int t0 = ch * BC;
    const int te = min(N, t0 + BC) - 1;
    const float* cA = cf + (ch & 1) * NCF;
    const float* cB = cA + BC;
    const float* cP = cA + 2 * BC;
    const float* cM = cA + 2 * BC + 4;
    const float* cS = cM + WP;
    __syncthreads();   // coefficients, the M image of the chunk-start state, X^T

    __builtin_amdgcn_sched_barrier(0);
    // ---- window forward, transposed: Y^T [value rows x window rows], K = DP.
    // Wave tiles i = wave + 4u: value tile i % NOT, window tile i / NOT.
    f32x4 Y[YPW];
#pragma unroll
    for (int u = 0; u < YPW; ++u) Y[u] = zero4();
    if constexpr (S::XT_LDS) {
#pragma unroll 2
      for (int s = 0; s < DP / 32; ++s) {
#pragma unroll
        for (int u = 0; u < YPW; ++u) {
          const int ot = (wave + 4 * u) % NOT, wt = (wave + 4 * u) / NOT;
          Y[u] = mma(ld_nat(Mi, LF, 16 * ot, 32 * s, lane), ld_tr_nat(XTl, WP, 16 * wt, 32 * s, lane), Y[u]);
        }
      }
    } else {
      // X rows from the phi buffer; the fragments of step s + PF are loaded
      // before step s computes
      constexpr int NS = DP / 32, PF = 3;
      bf16x8 xf[PF + 1][YPW];
      auto load = [&](int s, bf16x8* dst) {
#pragma unroll
        for (int u = 0; u < YPW; ++u) {
          const int wt = (wave + 4 * u) / NOT;
          dst[u] = gload8(rxr, ((t0 + 16 * wt + c16) * DP + 32 * s + 8 * g) * 2);
        }
      };
#pragma unroll
      for (int s = 0; s < PF && s < NS; ++s) load(s, xf[s]);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + PF < NS) load(s + PF, xf[(s + PF) % (PF + 1)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < YPW; ++u) {
          const int ot = (wave + 4 * u) % NOT;
          Y[u] = mma(ld_nat(Mi, LF, 16 * ot, 32 * s, lane), xf[s % (PF + 1)][u], Y[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- D = s gamma (Y - V) (dot: -s gamma V) of the valid window rows
    // (zero elsewhere: pg = 0 there): into LDS [WP][LV] and the workspace [WP][DV]
#pragma unroll
    for (int u = 0; u < YPW; ++u) {
      const int ot = (wave + 4 * u) % NOT, wt = (wave + 4 * u) / NOT;
      const int w = 16 * wt + c16, o4 = 16 * ot + 4 * g;
      const int i = t0 - (c - 1) + w;
      const bool valid = w < W && i >= -halo_valid && i <= te;
      const float sg = s_grad * pg[u];
      float d[4];
      d[0] = dot ? -sg * pv[u].x : sg * (Y[u][0] - pv[u].x);
      d[1] = dot ? -sg * pv[u].y : sg * (Y[u][1] - pv[u].y);
      d[2] = dot ? -sg * pv[u].z : sg * (Y[u][2] - pv[u].z);
      d[3] = dot ? -sg * pv[u].w : sg * (Y[u][3] - pv[u].w);
      const bf16x4 d4 = valid ? bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]}
                              : bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
      *reinterpret_cast<bf16x4*>(D2l + w * LV + o4) = d4;
      *reinterpret_cast<bf16x4*>(dg + ((size_t)ch * WP + w) * DV + o4) = d4;
    }
    __syncthreads();   // D complete

    __builtin_amdgcn_sched_barrier(0);
    // ---- update, transposed: (cM .* D)^T X as [feature rows x value cols], K = WP;
    // the wave's feature tiles 16 (wave + 4 m), every value tile
    {
      const int ce = te - t0;
      const float Ate = cA[ce], Bte = cB[ce], Pc = cP[0];
      bf16x8 bm[NOT][WP / 32], bs[NOT][WP / 32];
#pragma unroll
      for (int o = 0; o < NOT; ++o)
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) {
          const bf16x8 d = ld_tr_nat(D2l, LV, 16 * o, 32 * s, lane);
          bm[o][s] = scaled_k(d, cM + 32 * s + 8 * g);
          bs[o][s] = scaled_k(d, cS + 32 * s + 8 * g);
        }
      // X^T fragments of feature tile m + 1 are loaded before tile m computes
      bf16x8 xf[2][WP / 32];
      auto load = [&](int m, bf16x8* dst) {
        const int f = 16 * (wave + 4 * m) + c16;
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) {
          if constexpr (S::XT_LDS) dst[s] = ld_nat(XTl, WP, 16 * (wave + 4 * m), 32 * s, lane);
          else dst[s] = gload8(rxt, (f * (int)NR + t0 + 32 * s + 8 * g) * 2);
        }
      };
      load(0, xf[0]);
#pragma unroll
      for (int m = 0; m < FPW; ++m) {
        if (m + 1 < FPW) load(m + 1, xf[(m + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int o = 0; o < NOT; ++o) {
          f32x4 um = zero4(), us = zero4();
#pragma unroll
          for (int s = 0; s < WP / 32; ++s) {
            um = mma(xf[m & 1][s], bm[o][s], um);
            if (mom) us = mma(xf[m & 1][s], bs[o][s], us);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float w0 = MT[m][o][r], s0 = ST[m][o][r];
            MT[m][o][r] = Ate * w0 + Bte * s0 - um[r];
            ST[m][o][r] = Pc * s0 - us[r];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- the next chunk's images (the window forward's reads of the M image
    // ended before the last barrier), then its inputs.  X^T in LDS is
    // overwritten only once every wave is past its update; the coefficient
    // set of chunk ch + 1 was last read in chunk ch - 1.
    if (ch + 1 < nch) {
      write_images(ch + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (S::XT_LDS) __syncthreads();
      fetch(ch + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (S::XT_LDS) wait_vmem();
      store_coef(ch + 1);
    }
  }

  // ---- the state back to memory
  {
    const __amdgpu_buffer_rsrc_t rw = buffer_of(Wt, (unsigned)((size_t)DV * D * 4));
    const __amdgpu_buffer_rsrc_t rm = buffer_of(Mo, mom ? (unsigned)((size_t)DV * D * 4) : 0u);
#pragma unroll
    for (int m = 0; m < FPW; ++m)
#pragma unroll
      for (int o = 0; o < NOT; ++o)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * (wave + 4 * m) + 4 * g + r;
          const int off = f < D ? ((16 * o + c16) * D + f) * 4 : kZeroOffset;
          gstore1(MT[m][o][r], rw, off);
          gstore1(ST[m][o][r], rm, off);
        }
  }
  // halo and count (every wave has read the old halo before the first
  // chunk's second barrier)
  __syncthreads();
  if (tid < 64) {
    for (int j = 0; j < c - 1; ++j) {
      const int i = N - (c - 1) + j;
      for (int d = lane; d < DK; d += 64) hk[j * DK + d] = i >= 0 ? (float)k[(size_t)i * DK + d] : hk[(N + j) * DK + d];
      for (int o = lane; o < DV; o += 64) hv[j * DV + o] = i >= 0 ? (float)v[(size_t)i * DV + o] : hv[(N + j) * DV + o];
      if (lane == 0) hg[j] = i >= 0 ? gam_in[i] : hg[N + j];
    }
    if (lane == 0) *cnt += N;
  }
}

// One workgroup per (sequence, chunk); wave w owns query rows 16 w .. +15.
// Computed transposed ([value rows x queries]) so that each lane holds four
// adjacent values of one query: one 8-byte store per tile.
template <class S>
__global__ void __launch_bounds__(256) linear_ret_kernel(GroupedParams p) {
  constexpr int DV = S::DV, DP = S::DP, BC = S::BC, WP = S::WP, NOT = S::NOT, LV = S::LV;
  __shared__ __attribute__((aligned(16))) bf16 D2l[WP * LV];
  const int nch = p.nchunks;
  const int ch = (int)(blockIdx.x % (unsigned)nch), seq = (int)(blockIdx.x / (unsigned)nch);
  const int t0 = ch * BC, te = min(p.N, t0 + BC) - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const bool mom = p.momentum != 0;
  const char* ws = p.gws + (size_t)seq * p.gseq_bytes;
  const __amdgpu_buffer_rsrc_t rxq = buffer_of(ws + S::oXQ(nch), (unsigned)((size_t)nch * BC * DP * 2));
  const __amdgpu_buffer_rsrc_t rim =
      buffer_of(ws + S::oImg(nch) + (size_t)ch * 2 * DV * DP * 2, (unsigned)(2 * DV * DP * 2));
  const bf16* dg = reinterpret_cast<const bf16*>(ws + S::oDg(nch)) + (size_t)ch * WP * DV;
  const float* coef = p.coef + ((size_t)seq * nch + ch) * p.coef_stride;
  const bf16* Q1g = reinterpret_cast<const bf16*>(coef + 2 * BC + 4 + 2 * WP + BC * WP);   // [BC][WP]
  bf16* out = reinterpret_cast<bf16*>(p.out) + (size_t)seq * p.N * DV;

  for (int e = tid; e < WP * DV / 8; e += 256) {
    const int w = e / (DV / 8), o8 = (e % (DV / 8)) * 8;
    *reinterpret_cast<bf16x8*>(D2l + w * LV + o8) = *reinterpret_cast<const bf16x8*>(dg + w * DV + o8);
  }
  f32x4 a1[NOT], a2[NOT], a3[NOT];
#pragma unroll
  for (int o = 0; o < NOT; ++o) a1[o] = a2[o] = a3[o] = zero4();
  const int qrow = t0 + 16 * wave + c16;
  // row 16 o + c16, features 32 s + 8 g .. +7 of an image: two quads
  auto img_frag = [&](int base, int o, int s) {
    const int q = (int)S::img_pos(16 * o + c16, 32 * s + 8 * g);
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rim, (base + q) * 2, 0, 0));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rim, (base + q + 64 * NOT) * 2, 0, 0));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
#pragma unroll 2
  for (int s = 0; s < DP / 32; ++s) {
    const bf16x8 xq = gload8(rxq, (qrow * DP + 32 * s + 8 * g) * 2);
#pragma unroll
    for (int o = 0; o < NOT; ++o) {
      a1[o] = mma(img_frag(0, o, s), xq, a1[o]);
      if (mom) a2[o] = mma(img_frag(DV * DP, o, s), xq, a2[o]);
    }
  }
  __syncthreads();   // D in LDS
#pragma unroll
  for (int s = 0; s < WP / 32; ++s) {
    const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(Q1g + (16 * wave + c16) * WP + 32 * s + 8 * g);
#pragma unroll
    for (int o = 0; o < NOT; ++o) a3[o] = mma(ld_tr_nat(D2l, LV, 16 * o, 32 * s, lane), q1, a3[o]);
  }
  const int t = 16 * wave + c16;
  if (t0 + t <= te) {
    const float ca = coef[t], cb = coef[BC + t];
#pragma unroll
    for (int o = 0; o < NOT; ++o) {
      const bf16x4 y{(bf16)(ca * a1[o][0] + cb * a2[o][0] - a3[o][0]), (bf16)(ca * a1[o][1] + cb * a2[o][1] - a3[o][1]),
                     (bf16)(ca * a1[o][2] + cb * a2[o][2] - a3[o][2]), (bf16)(ca * a1[o][3] + cb * a2[o][3] - a3[o][3])};
      *reinterpret_cast<bf16x4*>(out + (size_t)(t0 + t) * DV + 16 * o + 4 * g) = y;
    }
  }
}

}  // namespace grouped

template <int PHI, int DK, int PD, int DV, int WP>
hipError_t launch_linear(const GroupedParams& gp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                         hipEvent_t ev1) {
  typedef grouped::LShape<PHI, DK, PD, DV, WP> S;
  if (gp.N == 0 || gp.n_seq == 0) return hipSuccess;
  hipLaunchKernelGGL((coeff_kernel<S::BC, S::WP>), dim3((unsigned)kp.nchunks * (unsigned)gp.n_seq), dim3(256), 0,
                     stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped::linear_rec_kernel<S>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::lds);
    (void)hipGetLastError();
    attr_set = true;
  }
  const unsigned per_seq = (unsigned)(S::rows_k(gp.nchunks) / 32 + 2 * (size_t)gp.nchunks);
  hipLaunchKernelGGL((grouped::phi_kernel<S>), dim3(per_seq * (unsigned)gp.n_seq), dim3(256), 0, stream, gp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((grouped::q1_phi_kernel<S>), dim3((unsigned)gp.nchunks * (unsigned)gp.n_seq), dim3(256), 0,
                     stream, gp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((grouped::linear_rec_kernel<S>), dim3((unsigned)gp.n_seq), dim3(256), S::lds, stream, gp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((grouped::linear_ret_kernel<S>), dim3((unsigned)gp.nchunks * (unsigned)gp.n_seq), dim3(256), 0,
                     stream, gp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int PHI, int DK, int PD, int DV, int WP>
size_t linear_seq_bytes(int nchunks) { return grouped::LShape<PHI, DK, PD, DV, WP>::seq_bytes(nchunks); }

#define ATLAS_GROUPED(NAME, PHI, DK, PD, DV, H, G)
#define ATLAS_LINEAR(NAME, PHI, DK, PD, DV, WP)                                                              \
  template hipError_t launch_linear<PHI, DK, PD, DV, WP>(const GroupedParams&, const CoeffParams&, hipStream_t, \
                                                         hipEvent_t, hipEvent_t);                             \
  template size_t linear_seq_bytes<PHI, DK, PD, DV, WP>(int);
#include "atlas_mem_grouped_variants.inc"
#undef ATLAS_GROUPED
#undef ATLAS_LINEAR

}  // namespace atlas
