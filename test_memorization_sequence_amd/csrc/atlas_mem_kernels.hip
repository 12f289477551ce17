// atlas_mem_kernels.hip -- gfx950 kernels of the test-time memory.
//
// Two kernels per forward call:
//
//  coeff_kernel   one workgroup per (sequence, chunk), all chunks in parallel.
//                 The gates alone fix how each token's gradient enters every
//                 later weight of the chunk.  Unrolling the momentum/decay
//                 recurrence (Titans review sec. 3.1, "Forgetting Mechanism")
//                 over a chunk that starts at t0 with weights W0, momentum S0:
//                   W_t = A_t W0 + B_t S0 - sum_i C_{t,i} G_i
//                   S_te = P S0 - sum_i cS_i G_i
//                 with G_i the gradient of window token i at W0 (ATLAS review
//                 sec. 3.3: gradients at the previous chunk's final state) and
//                   a_{m->t} = prod_{u=m+1..t} (1 - alpha_u),  e_{n->m} = prod_{u=n+1..m} eta_u
//                   A_t = a_{t0-1->t},  B_t = sum_{m=t0..t} a_{m->t} e_{t0-1->m}
//                   K_{t,n} = sum_{m=n..t} a_{m->t} e_{n->m}
//                   C_{t,i} = sum_{n in [t0,t], i in window(n)} K_{t,n} theta_n
//                   cS_i = sum_{n in chunk, i in window(n)} e_{n->te} theta_n,  P = e_{t0-1->te}
//                 The window of n is [n-c+1, n] (Omega rule, ATLAS review
//                 sec. 3.2); the band of C is the sliding-window mask.
//
//  chunk_kernel   one workgroup per sequence, persistent over the chunks
//                 (the chunk chain is sequential).  Per chunk, as bf16 (or
//                 fp32) MFMA GEMMs with fp32 accumulation:
//                   MLP  Z = X W1^T, A = gelu(Z), E = R + A W2^T - V,
//                        D2 = s*gamma*E (l_p, Huber: s*gamma*slope(E), see
//                        atlas_mem_bias.h), D1 = (D2 W2) .* gelu'(Z)
//                        retrieval with the per-token weights W_t:
//                          Zq = diag(A_t) Xq W1^T + diag(B_t) Xq S1^T - (C .* Xq X^T) D1
//                          y  = Rq + diag(A_t) gelu(Zq) W2^T + diag(B_t) gelu(Zq) S2^T
//                               - (C .* gelu(Zq) A^T) D2
//                        (exact, because every gradient is a sum of outer
//                        products; Titans review sec. 3.1 "Retrieving a Memory")
//                        W1 <- A_te W1 + B_te S1 - (cM .* D1)^T X,  S1 <- P S1 - (cS .* D1)^T X
//                        W2 <- A_te W2 + B_te S2 - (cM .* D2)^T A,  S2 <- P S2 - (cS .* D2)^T A
//                   linear  the same with one layer and no gelu.
//                 phi (ATLAS review sec. 3.1) is applied while staging.
//
// Every GEMM is "NT": C[m][n] = sum_k A[m][k] B[n][k], both operands stored
// with k contiguous, so each lane's MFMA fragment is one 16-byte load.
// Epilogues write each intermediate in the layouts its consumers need.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atlas_mem_internal.h"
#include "atlas_mem_coeff.h"
#include "atlas_mem_gelu.h"
#include "atlas_mem_bias.h"
#include "atlas_mem_group.h"

namespace atlas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }


// ----------------------------------------------------------------------------- MFMA
template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  typedef bf16x8 frag;
  // lane l: row (l & 15) of a 16-row block, k = k0 + 8*(l >> 4) .. +7
  __device__ static frag load(const bf16* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (size_t)(row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
  }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 16;
  typedef f32x4 frag;
  // lane l: row (l & 15), k = k0 + 4*(l >> 4) .. +3, one 16-byte load.  MFMA
  // step e contracts k0 + 4g + e over the four lane groups g: a permutation
  // of the 16 k's, the same for both operands, so the sum is unchanged.
  __device__ static frag load(const float* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const f32x4*>(base + (size_t)(row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
  }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  }
};

template <typename T> struct Op {
  const T* A; int lda;  // [M][K], k contiguous
  const T* B; int ldb;  // [N][K], k contiguous
  int K;                // multiple of Mma<T>::KSTEP; A == nullptr disables the op
};

// C_o[m][n] = sum_k A_o[m][k] B_o[n][k] for each op o, over a 32x32 tile per
// wave (2x2 MFMA blocks); epi(m, n, v[NOPS]) receives every element once.
// M and N must be multiples of 32.  upper (M == N, a symmetric result): only
// the tiles on and above the diagonal, spread evenly over the waves; the
// epilogue mirrors them.
template <typename T, int NOPS, typename Epi>
__device__ __forceinline__ void gemm_nt(int M, int N, const Op<T> (&ops)[NOPS], Epi&& epi, bool upper = false) {
  typedef Mma<T> MM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int tn = N >> 5, ntiles = upper ? tn * (tn + 1) / 2 : (M >> 5) * tn;
  for (int t = wave; t < ntiles; t += nwaves) {
    int m0 = (t / tn) << 5, n0 = (t % tn) << 5;
    if (upper) {  // t-th tile of the upper triangle, row by row
      int mt = 0, rem = t;
      while (rem >= tn - mt) { rem -= tn - mt; ++mt; }
      m0 = mt << 5;
      n0 = (mt + rem) << 5;
    }
    f32x4 acc[NOPS][2][2];
#pragma unroll
    for (int o = 0; o < NOPS; ++o)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[o][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int o = 0; o < NOPS; ++o) {
      const Op<T> op = ops[o];
      if (op.A == nullptr) continue;
      for (int k0 = 0; k0 < op.K; k0 += MM::KSTEP) {
        typename MM::frag a0 = MM::load(op.A, op.lda, m0, k0, lane);
        typename MM::frag a1 = MM::load(op.A, op.lda, m0 + 16, k0, lane);
        typename MM::frag b0 = MM::load(op.B, op.ldb, n0, k0, lane);
        typename MM::frag b1 = MM::load(op.B, op.ldb, n0 + 16, k0, lane);
        acc[o][0][0] = MM::mma(a0, b0, acc[o][0][0]);
        acc[o][0][1] = MM::mma(a0, b1, acc[o][0][1]);
        acc[o][1][0] = MM::mma(a1, b0, acc[o][1][0]);
        acc[o][1][1] = MM::mma(a1, b1, acc[o][1][1]);
      }
    }
    // 16x16 MFMA output: lane l holds column (l & 15), rows 4*(l >> 4) + r
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v[NOPS];
#pragma unroll
          for (int o = 0; o < NOPS; ++o) v[o] = acc[o][i][j][r];
          epi(m0 + 16 * i + 4 * (lane >> 4) + r, n0 + 16 * j + (lane & 15), v);
        }
  }
}

// ----------------------------------------------------------------------------- phi
// Pair table for the degree-2 monomials x_a x_b, a <= b < p, row-major upper
// triangle order (ATLAS review sec. 3.1, polynomial feature map).
template <int P> struct PairTable {
  static constexpr int NP = P * (P + 1) / 2;
  uint8_t a[NP > 0 ? NP : 1], b[NP > 0 ? NP : 1];
  __device__ void fill() {
    for (int idx = threadIdx.x; idx < NP; idx += blockDim.x) {
      int aa = 0, off = 0;
      while (idx >= off + (P - aa)) { off += P - aa; ++aa; }
      a[idx] = (uint8_t)aa;
      b[idx] = (uint8_t)(aa + idx - off);
    }
  }
};

// feature f of phi(row); zero past the feature width (padding)
template <class S, typename TI>
__device__ __forceinline__ float phi_feature(const TI* row, int f, const PairTable<S::PD>& pt) {
  if (f < S::DK) return to_f(row[f]);
  if (S::PHI == PHI_POLY2) {
    if (f < S::D) { const int p = f - S::DK; return to_f(row[pt.a[p]]) * to_f(row[pt.b[p]]); }
    return 0.f;
  }
  if (S::PHI == PHI_RAW_POLY2) {
    if (f < S::DK + S::PD) return to_f(row[f - S::DK]);
    if (f < S::D) { const int p = f - S::DK - S::PD; return to_f(row[pt.a[p]]) * to_f(row[pt.b[p]]); }
  }
  return 0.f;
}

}  // namespace atlas

#include "atlas_mem_muon.h"

namespace atlas {

// ----------------------------------------------------------------------------- chunk kernel
// NT threads: 256 for gradient descent on narrow memories; 512 for Muon,
// whose per-token Newton-Schulz GEMMs are latency-bound and gain from a
// second wave per SIMD, and for gradient descent on wide memories (h >= 512
// or D >= 256), where the same holds for the chunk's GEMMs.
template <class S, int NT>
__global__ void __launch_bounds__(NT) chunk_kernel(ChunkParams p) {
  typedef typename S::T T;    // MFMA operand type
  typedef typename S::TI TI;  // io type of q, k, v, out
  typedef typename S::WS WS;
  constexpr int DK = S::DK, DV = S::DV, D = S::D, DP = S::DP, H = S::H, BC = S::BC, WP = S::WP;
  // Muon on the MLP memory: a pair of workgroups per sequence (pm 0: W1,
  // pm 1: W2), XCD-aware: block b runs on XCD b % 8, and the pair is blocks
  // 8 (2 i + pm) + xcd, so both members share that XCD's L2
  int seq = blockIdx.x, pm = 0;
  const bool pair = p.group > 1;
  if (pair) {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    pm = slot & 1;
    seq = (slot >> 1) * 8 + xcd;
    if (seq >= p.n_seq) return;
  }
  const int member = pair ? 2 * seq + pm : seq;   // index of this workgroup's workspaces
  const int N = p.N, c = p.c, W = BC + c - 1;
  const float s_grad = p.grad_scale;
  const bool mom = p.momentum != 0, dot = p.bias == BIAS_DOT, res = p.residual != 0;
  // l_p and Huber biases: D2 from the raw errors once whole rows are known
  const bool shaped = p.bias == BIAS_LP || p.bias == BIAS_HUBER, huber = p.bias == BIAS_HUBER;
  const float bias_p = p.bias_p, sign_alpha = p.sign_alpha;
  // MLP with a layer norm on the branch: D2 and y need whole-row statistics too
  const bool ln = S::MEM == MEM_MLP && p.layernorm != 0;
  // gated memory: A = gelu(X W1^T) .* (X W3^T), a third weight matrix W3
  const bool gated = S::MEM == MEM_MLP && p.gated != 0;
  const float ln_eps = p.ln_eps;
  const bool rowwise = shaped || ln;
  // Muon memory optimizer: per-token Newton-Schulz steps after the window
  // gradients (atlas_mem_muon.h); no layer norm, no gated memory
  // (only the 512-thread instance carries the Muon code; the launcher picks it)
  const bool muon = NT == 512 && p.muon != 0;

  char* st = p.state + (size_t)seq * p.seq_stride;
  float* Wt = reinterpret_cast<float*>(st + p.off_weights);
  float* Mo = reinterpret_cast<float*>(st + p.off_momentum);
  float* hk = reinterpret_cast<float*>(st + p.off_halo_k);
  float* hv = reinterpret_cast<float*>(st + p.off_halo_v);
  float* hg = reinterpret_cast<float*>(st + p.off_halo_g);
  float* hd = reinterpret_cast<float*>(st + p.off_halo_d);   // Huber only
  int64_t* cnt = reinterpret_cast<int64_t*>(st + p.off_count);
  const int halo_valid = (int)min<int64_t>(*cnt, (int64_t)(c - 1));
  const float* dl_in = huber ? p.delta + (size_t)seq * N : nullptr;

  const TI* q = reinterpret_cast<const TI*>(p.q) + (size_t)seq * N * DK;
  const TI* k = reinterpret_cast<const TI*>(p.k) + (size_t)seq * N * DK;
  const TI* v = reinterpret_cast<const TI*>(p.v) + (size_t)seq * N * DV;
  TI* out = reinterpret_cast<TI*>(p.out) + (size_t)seq * N * DV;
  const float* gam_in = p.gamma + (size_t)seq * N;

  char* ws = p.ws + (size_t)member * WS::bytes;
  T* Xw = reinterpret_cast<T*>(ws + WS::Xw);     // [WP][DP]  phi(k) of the window
  T* XwT = reinterpret_cast<T*>(ws + WS::XwT);   // [DP][WP]
  T* Xq = reinterpret_cast<T*>(ws + WS::Xq);     // [BC][DP]  phi(q) of the chunk
  T* Q1 = reinterpret_cast<T*>(ws + WS::Q1);     // [BC][WP]  C .* (Xq X^T)
  // MLP
  T* W1b = reinterpret_cast<T*>(ws + WS::W1b);   // [H][DP]   operand image of W1
  T* S1b = reinterpret_cast<T*>(ws + WS::S1b);   // [H][DP]
  T* W2b = reinterpret_cast<T*>(ws + WS::W2b);   // [DV][H]
  T* S2b = reinterpret_cast<T*>(ws + WS::S2b);   // [DV][H]
  T* W2T = reinterpret_cast<T*>(ws + WS::W2T);   // [H][DV]
  float* Zf = reinterpret_cast<float*>(ws + WS::Zf);  // [WP][H]
  T* Ab = reinterpret_cast<T*>(ws + WS::Ab);     // [WP][H]   gelu(Z)
  T* AT = reinterpret_cast<T*>(ws + WS::AT);     // [H][WP]
  T* D2 = reinterpret_cast<T*>(ws + WS::D2);     // [WP][DV]
  T* D2T = reinterpret_cast<T*>(ws + WS::D2T);   // [DV][WP]
  T* D2TM = reinterpret_cast<T*>(ws + WS::D2TM); // [DV][WP]  cM-scaled
  T* D2TS = reinterpret_cast<T*>(ws + WS::D2TS); // [DV][WP]  cS-scaled
  T* D1T = reinterpret_cast<T*>(ws + WS::D1T);   // [H][WP]
  T* D1TM = reinterpret_cast<T*>(ws + WS::D1TM);
  T* D1TS = reinterpret_cast<T*>(ws + WS::D1TS);
  T* Ah = reinterpret_cast<T*>(ws + WS::Ah);     // [BC][H]   gelu(Zq)
  T* Q2 = reinterpret_cast<T*>(ws + WS::Q2);     // [BC][WP]  C .* (gelu(Zq) A^T)
  float* Ef = reinterpret_cast<float*>(ws + WS::Ef);  // [WP][DV] raw errors (l_p, Huber) or u (LN)
  float* En = reinterpret_cast<float*>(ws + WS::En);  // [WP][DV] LN: the normalised branch
  T* W3b = reinterpret_cast<T*>(ws + WS::W3b);   // [H][DP]   gated: image of W3
  T* S3b = reinterpret_cast<T*>(ws + WS::S3b);   // [H][DP]
  float* Z3f = reinterpret_cast<float*>(ws + WS::Z3f);  // [WP][H] X W3^T
  T* D3T = reinterpret_cast<T*>(ws + WS::D3T);   // [H][WP]
  T* D3TM = reinterpret_cast<T*>(ws + WS::D3TM);
  T* D3TS = reinterpret_cast<T*>(ws + WS::D3TS);
  // linear (aliases of the MLP names where the roles coincide)
  T* Mb = W2b;   // [DV][DP]
  T* Sb = S2b;   // [DV][DP]

  __shared__ TI kr[WP][DK];   // raw keys of the window (residual path, phi input)
  __shared__ TI qr[BC][DK];   // raw queries of the chunk
  __shared__ float gw[WP], cMw[WP], cSw[WP], cA[BC], cB[BC];
  __shared__ float dw[WP], rsel[WP];   // Huber: thresholds of the window rows, their choice
  __shared__ float cP;
  __shared__ PairTable<S::PD> pt;
  // Muon: block sums; the factors of the window rows entering and leaving
  // (2 (rows + cols) floats of the largest matrix), then gelu(W1 phi(q_n))
  constexpr int MU_STAGE = S::MEM == MEM_MLP ? 2 * ((H > DV ? H : DV) + (D > H ? D : H)) : 2 * (DV + D);
  __shared__ float mu_red[NT / 64];
  extern __shared__ __attribute__((aligned(16))) float mu_bs[];   // Muon: B of Newton-Schulz (launch-sized)
  __shared__ float mu_stage[MU_STAGE];
  float* mu_ah = mu_stage;
  if (S::PHI != PHI_IDENTITY) pt.fill();
  char* mws = muon ? p.mws + (size_t)member * p.mws_stride : nullptr;
  constexpr MuonWs MUL = muon_ws_of(S::MEM == MEM_MLP, D, DV, H, BC);
  // pair: counter and error word, the barrier count so far, and the hidden
  // activations the W1 member hands over (in that member's workspace)
  unsigned* gctr = pair ? p.ctrl + 1 + seq : nullptr;
  unsigned* gerr = pair ? p.ctrl : nullptr;
  unsigned gbase = 0;
  float* abuf = pair ? reinterpret_cast<float*>(p.mws + (size_t)(2 * seq) * p.mws_stride + MUL.ab) : nullptr;
  constexpr long P_W = S::MEM == MEM_MLP ? (long)H * D + (long)DV * H : (long)DV * D;
  // Muon without momentum in the state: S = g every token (eta = 0) in a
  // workspace buffer, zeroed so that 0 * S stays 0
  float* Smu = muon ? (mom ? Mo : reinterpret_cast<float*>(mws)) : nullptr;
  float* Gmu = muon ? reinterpret_cast<float*>(mws + MUL.g) : nullptr;
  if (muon && !mom)
    for (long e = threadIdx.x; e < P_W; e += blockDim.x) Smu[e] = 0.f;

  // operand images of the state
  if (S::MEM == MEM_MLP) {
    const float* W1 = Wt;
    const float* W2 = Wt + (size_t)H * D;
    for (int e = threadIdx.x; e < H * DP; e += blockDim.x) {
      const int j = e / DP, f = e % DP;
      W1b[e] = from_f<T>(f < D ? W1[j * D + f] : 0.f);
      S1b[e] = from_f<T>((f < D && mom) ? Mo[j * D + f] : 0.f);
    }
    for (int e = threadIdx.x; e < DV * H; e += blockDim.x) {
      const int o = e / H, j = e % H;
      W2b[e] = from_f<T>(W2[e]);
      S2b[e] = from_f<T>(mom ? Mo[(size_t)H * D + e] : 0.f);
      W2T[j * DV + o] = from_f<T>(W2[e]);
    }
    if (gated) {
      const float* W3 = Wt + (size_t)H * D + (size_t)DV * H;
      const float* S3 = Mo + (size_t)H * D + (size_t)DV * H;
      for (int e = threadIdx.x; e < H * DP; e += blockDim.x) {
        const int j = e / DP, f = e % DP;
        W3b[e] = from_f<T>(f < D ? W3[j * D + f] : 0.f);
        S3b[e] = from_f<T>((f < D && mom) ? S3[j * D + f] : 0.f);
      }
    }
  } else {
    for (int e = threadIdx.x; e < DV * DP; e += blockDim.x) {
      const int o = e / DP, f = e % DP;
      Mb[e] = from_f<T>(f < D ? Wt[o * D + f] : 0.f);
      Sb[e] = from_f<T>((f < D && mom) ? Mo[o * D + f] : 0.f);
    }
  }
  __syncthreads();

  const int nchunks = (N + BC - 1) / BC;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * BC;
    const int te = min(N, t0 + BC) - 1;
    const float* coef = p.coef + ((size_t)seq * p.nchunks + ch) * p.coef_stride;
    const float* Cc = coef + 2 * BC + 4 + 2 * WP;   // [BC][WP]

    // ---- stage raw rows, gates, coefficients
    for (int e = threadIdx.x; e < WP * DK; e += blockDim.x) {
      const int w = e / DK, d = e % DK;
      const int i = t0 - (c - 1) + w;
      float x = 0.f;
      if (w < W && i >= -halo_valid && i <= te) x = i >= 0 ? to_f(k[(size_t)i * DK + d]) : hk[(c - 1 + i) * DK + d];
      kr[w][d] = from_f<TI>(x);
    }
    for (int e = threadIdx.x; e < BC * DK; e += blockDim.x) {
      const int n = e / DK, d = e % DK;
      qr[n][d] = t0 + n <= te ? q[(size_t)(t0 + n) * DK + d] : from_f<TI>(0.f);
    }
    for (int w = threadIdx.x; w < WP; w += blockDim.x) {
      const int i = t0 - (c - 1) + w;
      float g = 0.f;
      float dd = 0.f;
      if (w < W && i >= -halo_valid && i <= te) {
        g = i >= 0 ? gam_in[i] : hg[c - 1 + i];
        if (huber) dd = i >= 0 ? dl_in[i] : hd[c - 1 + i];
      }
      gw[w] = g;
      dw[w] = dd;
      cMw[w] = coef[2 * BC + 4 + w];
      cSw[w] = coef[2 * BC + 4 + WP + w];
    }
    for (int n = threadIdx.x; n < BC; n += blockDim.x) { cA[n] = coef[n]; cB[n] = coef[BC + n]; }
    if (threadIdx.x == 0) cP = coef[2 * BC];
    __syncthreads();

    // ---- phi of window keys and chunk queries
    for (int e = threadIdx.x; e < WP * DP; e += blockDim.x) {
      const int w = e / DP, f = e % DP;
      const T x = from_f<T>(phi_feature<S>(&kr[w][0], f, pt));
      Xw[e] = x;
      XwT[f * WP + w] = x;
    }
    for (int e = threadIdx.x; e < BC * DP; e += blockDim.x) {
      const int n = e / DP, f = e % DP;
      Xq[e] = from_f<T>(phi_feature<S>(&qr[n][0], f, pt));
    }
    __syncthreads();

    // value of window row w, component o (input or halo); row valid <=> gw != 0 or in range
    auto vrow = [&](int w, int o) -> float {
      const int i = t0 - (c - 1) + w;
      if (w >= W || i < -halo_valid || i > te) return 0.f;
      return i >= 0 ? to_f(v[(size_t)i * DV + o]) : hv[(c - 1 + i) * DV + o];
    };
    // Muon: per token, the Newton-Schulz step of every weight matrix, then
    // y_n = f_{W_n}(phi(q_n)) from the fp32 weights; afterwards the operand
    // images of the chunk-end weights for the next chunk's gradients
    auto muon_chunk = [&]() {
      if constexpr (S::MEM == MEM_MLP) {
        if (pair) {
          // counter per chunk: both arrive (2), then one signal per token
          // from member 0, then both arrive again (2)
          const unsigned m = (unsigned)(te - t0 + 1);
          group_barrier(gctr, gbase + 2u, gerr);   // the partner's image refresh is done
          for (int n = t0; n <= te; ++n) {
            const size_t gi = (size_t)seq * N + n;
            const float al = p.alpha[gi], th = p.theta[gi], et = mom ? p.eta[gi] : 0.f;
            const int w0 = n - t0;
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
            float* an = abuf + (size_t)(n - t0) * H;
            if (pm == 0) {
              muon_matrix<S, H, D>(Wt, Smu, Gmu, et, D1T, XwT, w0, c, n == t0, al, th, p.ns_steps, mws, mu_red,
                                   mu_stage, mu_bs);
              const T* xq = Xq + (size_t)(n - t0) * DP;
              for (int j = wave; j < H; j += nwaves) {
                float acc = 0.f;
                for (int f = lane; f < D; f += 64) acc += Wt[(size_t)j * D + f] * to_f(xq[f]);
                acc = muon_wave_sum(acc);
                if (lane == 0) an[j] = gelu(acc);
              }
              pair_signal(gctr);
            } else {
              muon_matrix<S, DV, H>(Wt + (size_t)H * D, Smu + (size_t)H * D, Gmu + (size_t)H * D, et, D2T, AT, w0, c,
                                    n == t0, al, th, p.ns_steps, mws, mu_red, mu_stage, mu_bs);
              pair_wait(gctr, gbase + 2u + (unsigned)(n - t0 + 1), gerr);
              const float* W2 = Wt + (size_t)H * D;
              for (int o = wave; o < DV; o += nwaves) {
                float acc = 0.f;
                for (int j = lane; j < H; j += 64) acc += W2[(size_t)o * H + j] * an[j];
                acc = muon_wave_sum(acc);
                if (lane == 0) out[(size_t)n * DV + o] = from_f<TI>((res ? to_f(qr[n - t0][o]) : 0.f) + acc);
              }
              __syncthreads();
            }
          }
          group_barrier(gctr, gbase + 4u + m, gerr);   // both matrices are at the chunk end
          gbase += 4u + m;
          for (int e = threadIdx.x; e < H * D; e += blockDim.x) W1b[(e / D) * DP + e % D] = from_f<T>(Wt[e]);
          for (int e = threadIdx.x; e < DV * H; e += blockDim.x) {
            const float w2 = Wt[(size_t)H * D + e];
            W2b[e] = from_f<T>(w2);
            W2T[(e % H) * DV + e / H] = from_f<T>(w2);
          }
          __syncthreads();
          return;
        }
      }
      for (int n = t0; n <= te; ++n) {
        const size_t gi = (size_t)seq * N + n;
        const float al = p.alpha[gi], th = p.theta[gi], et = mom ? p.eta[gi] : 0.f;
        const int w0 = n - t0;
        const T* xq = Xq + (size_t)(n - t0) * DP;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
        if constexpr (S::MEM == MEM_MLP) {
          muon_matrix<S, H, D>(Wt, Smu, Gmu, et, D1T, XwT, w0, c, n == t0, al, th, p.ns_steps, mws, mu_red, mu_stage, mu_bs);
          muon_matrix<S, DV, H>(Wt + (size_t)H * D, Smu + (size_t)H * D, Gmu + (size_t)H * D, et, D2T, AT, w0, c,
                                n == t0, al, th, p.ns_steps, mws, mu_red, mu_stage, mu_bs);
          const float* W1 = Wt;
          const float* W2 = Wt + (size_t)H * D;
          for (int j = wave; j < H; j += nwaves) {
            float acc = 0.f;
            for (int f = lane; f < D; f += 64) acc += W1[(size_t)j * D + f] * to_f(xq[f]);
            acc = muon_wave_sum(acc);
            if (lane == 0) mu_ah[j] = gelu(acc);
          }
          __syncthreads();
          for (int o = wave; o < DV; o += nwaves) {
            float acc = 0.f;
            for (int j = lane; j < H; j += 64) acc += W2[(size_t)o * H + j] * mu_ah[j];
            acc = muon_wave_sum(acc);
            if (lane == 0) out[(size_t)n * DV + o] = from_f<TI>((res ? to_f(qr[n - t0][o]) : 0.f) + acc);
          }
        } else {
          muon_matrix<S, DV, D>(Wt, Smu, Gmu, et, D2T, XwT, w0, c, n == t0, al, th, p.ns_steps, mws, mu_red, mu_stage, mu_bs);
          for (int o = wave; o < DV; o += nwaves) {
            float acc = 0.f;
            for (int f = lane; f < D; f += 64) acc += Wt[(size_t)o * D + f] * to_f(xq[f]);
            acc = muon_wave_sum(acc);
            if (lane == 0) out[(size_t)n * DV + o] = from_f<TI>(acc);
          }
        }
        __syncthreads();
      }
      if (S::MEM == MEM_MLP) {
        for (int e = threadIdx.x; e < H * D; e += blockDim.x) W1b[(e / D) * DP + e % D] = from_f<T>(Wt[e]);
        for (int e = threadIdx.x; e < DV * H; e += blockDim.x) {
          const float w2 = Wt[(size_t)H * D + e];
          W2b[e] = from_f<T>(w2);
          W2T[(e % H) * DV + e / H] = from_f<T>(w2);
        }
      } else {
        for (int e = threadIdx.x; e < DV * D; e += blockDim.x) Mb[(e / D) * DP + e % D] = from_f<T>(Wt[e]);
      }
      __syncthreads();
    };

    // D2 element (w, o) in every layout its consumers read
    auto put_d2 = [&](int w, int o, float d2) {
      if (S::MEM == MEM_MLP) D2[w * DV + o] = from_f<T>(d2);
      D2T[o * WP + w] = from_f<T>(d2);
      D2TM[o * WP + w] = from_f<T>(cMw[w] * d2);
      D2TS[o * WP + w] = from_f<T>(cSw[w] * d2);
    };
    // D2 from whole rows, one thread per window row.  In Ef: the raw errors
    // (l_p, Huber) or, with the layer norm, the branch u = A W2^T.  LN
    // forward (e = r + (u - mean)/sd - v), the bias's slope g (per token for
    // Huber), then the LN backward (g - mean(g) - nhat mean(g nhat)) / sd.
    auto shape_rows = [&]() {
      __syncthreads();
      for (int w = threadIdx.x; w < WP; w += blockDim.x) {
        float* E = Ef + w * DV;
        float* Nh = En + w * DV;
        float sd = 1.f;
        if (ln) {
          float mu = 0.f, var = 0.f;
          for (int o = 0; o < DV; ++o) mu += E[o];
          mu /= DV;
          for (int o = 0; o < DV; ++o) var += (E[o] - mu) * (E[o] - mu);
          var /= DV;
          sd = sqrtf(var + ln_eps);
          for (int o = 0; o < DV; ++o) {
            const float nh = (E[o] - mu) / sd;
            Nh[o] = nh;
            E[o] = (res ? to_f(kr[w][o]) : 0.f) + nh - vrow(w, o);
          }
        }
        bool small = true;
        if (huber) {
          float n2 = 0.f;
          for (int o = 0; o < DV; ++o) n2 += E[o] * E[o];
          small = sqrtf(n2) <= dw[w];
        }
        for (int o = 0; o < DV; ++o)
          E[o] = dot     ? -vrow(w, o)
               : huber   ? huber_slope(E[o], small, dw[w], sign_alpha)
               : shaped  ? lp_slope(E[o], bias_p, sign_alpha)
                         : E[o];
        if (ln) {
          float mg = 0.f, mgn = 0.f;
          for (int o = 0; o < DV; ++o) {
            mg += E[o];
            mgn += E[o] * Nh[o];
          }
          mg /= DV;
          mgn /= DV;
          for (int o = 0; o < DV; ++o) E[o] = (E[o] - mg - Nh[o] * mgn) / sd;
        }
        for (int o = 0; o < DV; ++o) put_d2(w, o, s_grad * gw[w] * E[o]);
      }
    };

    // Q1 = C .* (Xq X^T)
    if (!muon) {
      Op<T> ops[1] = {{Xq, DP, Xw, DP, DP}};
      gemm_nt(BC, WP, ops, [&](int n, int w, const float* a) { Q1[n * WP + w] = from_f<T>(Cc[n * WP + w] * a[0]); });
    }

    if (S::MEM == MEM_MLP) {
      // Z = X W1^T ; A = gelu(Z)   (gated: A = gelu(Z) .* (X W3^T))
      {
        Op<T> ops[2] = {{Xw, DP, W1b, DP, DP}, {gated ? Xw : nullptr, DP, W3b, DP, DP}};
        gemm_nt(WP, H, ops, [&](int w, int j, const float* a) {
          Zf[w * H + j] = a[0];
          if (gated) Z3f[w * H + j] = a[1];
          const T g = from_f<T>(gated ? gelu(a[0]) * a[1] : gelu(a[0]));
          Ab[w * H + j] = g;
          AT[j * WP + w] = g;
        });
      }
      __syncthreads();
      // E = R + A W2^T - V ; D2 = s gamma E  (dot bias: D2 = -s gamma V)
      {
        Op<T> ops[1] = {{Ab, H, W2b, H, H}};
        gemm_nt(WP, DV, ops, [&](int w, int o, const float* a) {
          const float vv = vrow(w, o);
          const float err = (res ? to_f(kr[w][o]) : 0.f) + a[0] - vv;
          if (ln) Ef[w * DV + o] = a[0];
          else if (shaped) Ef[w * DV + o] = err;
          else put_d2(w, o, dot ? -s_grad * gw[w] * vv : s_grad * gw[w] * err);
        });
        if (rowwise) shape_rows();
      }
      __syncthreads();
      // D1 = (D2 W2) .* gelu'(Z)   (gated: .* (X W3^T), and D3 = (D2 W2) .* gelu(Z))
      {
        Op<T> ops[1] = {{D2, DV, W2T, DV, DV}};
        gemm_nt(WP, H, ops, [&](int w, int j, const float* a) {
          const float z = Zf[w * H + j];
          const float d1 = a[0] * gelu_prime(z) * (gated ? Z3f[w * H + j] : 1.f);
          D1T[j * WP + w] = from_f<T>(d1);
          D1TM[j * WP + w] = from_f<T>(cMw[w] * d1);
          D1TS[j * WP + w] = from_f<T>(cSw[w] * d1);
          if (gated) {
            const float d3 = a[0] * gelu(z);
            D3T[j * WP + w] = from_f<T>(d3);
            D3TM[j * WP + w] = from_f<T>(cMw[w] * d3);
            D3TS[j * WP + w] = from_f<T>(cSw[w] * d3);
          }
        });
      }
      __syncthreads();
      if (muon) {
        muon_chunk();
        continue;
      }
      // Zq = A_t Xq W1^T + B_t Xq S1^T - Q1 D1 ; Ah = gelu(Zq)
      // (gated: .* (A_t Xq W3^T + B_t Xq S3^T - Q1 D3))
      {
        Op<T> ops[6] = {{Xq, DP, W1b, DP, DP}, {mom ? Xq : nullptr, DP, S1b, DP, DP}, {Q1, WP, D1T, WP, WP},
                        {gated ? Xq : nullptr, DP, W3b, DP, DP}, {gated && mom ? Xq : nullptr, DP, S3b, DP, DP},
                        {gated ? Q1 : nullptr, WP, D3T, WP, WP}};
        gemm_nt(BC, H, ops, [&](int n, int j, const float* a) {
          const float g1 = gelu(cA[n] * a[0] + cB[n] * a[1] - a[2]);
          Ah[n * H + j] = from_f<T>(gated ? g1 * (cA[n] * a[3] + cB[n] * a[4] - a[5]) : g1);
        });
      }
      __syncthreads();
      // Q2 = C .* (Ah A^T)
      {
        Op<T> ops[1] = {{Ah, H, Ab, H, H}};
        gemm_nt(BC, WP, ops, [&](int n, int w, const float* a) { Q2[n * WP + w] = from_f<T>(Cc[n * WP + w] * a[0]); });
      }
      __syncthreads();
      // y = Rq + A_t Ah W2^T + B_t Ah S2^T - Q2 D2
      {
        Op<T> ops[3] = {{Ah, H, W2b, H, H}, {mom ? Ah : nullptr, H, S2b, H, H}, {Q2, WP, D2T, WP, WP}};
        gemm_nt(BC, DV, ops, [&](int n, int o, const float* a) {
          const float u = cA[n] * a[0] + cB[n] * a[1] - a[2];
          if (ln) Ef[n * DV + o] = u;
          else if (t0 + n <= te) out[(size_t)(t0 + n) * DV + o] = from_f<TI>((res ? to_f(qr[n][o]) : 0.f) + u);
        });
        if (ln) {
          // y = r + LN(u), one thread per query row
          __syncthreads();
          for (int n = threadIdx.x; n < BC; n += blockDim.x) {
            if (t0 + n > te) continue;
            const float* U = Ef + n * DV;
            float mu = 0.f, var = 0.f;
            for (int o = 0; o < DV; ++o) mu += U[o];
            mu /= DV;
            for (int o = 0; o < DV; ++o) var += (U[o] - mu) * (U[o] - mu);
            var /= DV;
            const float sd = sqrtf(var + ln_eps);
            for (int o = 0; o < DV; ++o)
              out[(size_t)(t0 + n) * DV + o] = from_f<TI>((res ? to_f(qr[n][o]) : 0.f) + (U[o] - mu) / sd);
          }
        }
      }
      __syncthreads();
      // state update at the chunk end
      const float Ate = cA[te - t0], Bte = cB[te - t0], Pc = cP;
      {
        Op<T> ops[2] = {{D1TM, WP, XwT, WP, WP}, {mom ? D1TS : nullptr, WP, XwT, WP, WP}};
        gemm_nt(H, DP, ops, [&](int j, int f, const float* a) {
          if (f < D) {
            const size_t e = (size_t)j * D + f;
            const float w1 = Wt[e], s1 = mom ? Mo[e] : 0.f;
            const float nw = Ate * w1 + Bte * s1 - a[0];
            Wt[e] = nw;
            W1b[j * DP + f] = from_f<T>(nw);
            if (mom) {
              const float ns = Pc * s1 - a[1];
              Mo[e] = ns;
              S1b[j * DP + f] = from_f<T>(ns);
            }
          }
        });
      }
      {
        Op<T> ops[2] = {{D2TM, WP, AT, WP, WP}, {mom ? D2TS : nullptr, WP, AT, WP, WP}};
        gemm_nt(DV, H, ops, [&](int o, int j, const float* a) {
          const size_t e = (size_t)H * D + (size_t)o * H + j;
          const float w2 = Wt[e], s2 = mom ? Mo[e] : 0.f;
          const float nw = Ate * w2 + Bte * s2 - a[0];
          Wt[e] = nw;
          W2b[o * H + j] = from_f<T>(nw);
          W2T[j * DV + o] = from_f<T>(nw);
          if (mom) {
            const float ns = Pc * s2 - a[1];
            Mo[e] = ns;
            S2b[o * H + j] = from_f<T>(ns);
          }
        });
      }
      if (gated) {
        // W3 <- A_te W3 + B_te S3 - (cM .* D3)^T X,  S3 <- P S3 - (cS .* D3)^T X
        Op<T> ops[2] = {{D3TM, WP, XwT, WP, WP}, {mom ? D3TS : nullptr, WP, XwT, WP, WP}};
        gemm_nt(H, DP, ops, [&](int j, int f, const float* a) {
          if (f < D) {
            const size_t e = (size_t)H * D + (size_t)DV * H + (size_t)j * D + f;
            const float w3 = Wt[e], s3 = mom ? Mo[e] : 0.f;
            const float nw = Ate * w3 + Bte * s3 - a[0];
            Wt[e] = nw;
            W3b[j * DP + f] = from_f<T>(nw);
            if (mom) {
              const float ns = Pc * s3 - a[1];
              Mo[e] = ns;
              S3b[j * DP + f] = from_f<T>(ns);
            }
          }
        });
      }
      __syncthreads();
    } else {
      // linear: D = s gamma (X M^T - V)  (dot bias: -s gamma V)
      {
        Op<T> ops[1] = {{Xw, DP, Mb, DP, DP}};
        gemm_nt(WP, DV, ops, [&](int w, int o, const float* a) {
          const float vv = vrow(w, o);
          const float err = a[0] - vv;
          if (shaped) Ef[w * DV + o] = err;
          else put_d2(w, o, dot ? -s_grad * gw[w] * vv : s_grad * gw[w] * err);
        });
        if (shaped) shape_rows();
      }
      __syncthreads();
      if (muon) {
        muon_chunk();
        continue;
      }
      // y = A_t Xq M^T + B_t Xq S^T - Q1 D
      {
        Op<T> ops[3] = {{Xq, DP, Mb, DP, DP}, {mom ? Xq : nullptr, DP, Sb, DP, DP}, {Q1, WP, D2T, WP, WP}};
        gemm_nt(BC, DV, ops, [&](int n, int o, const float* a) {
          if (t0 + n <= te) out[(size_t)(t0 + n) * DV + o] = from_f<TI>(cA[n] * a[0] + cB[n] * a[1] - a[2]);
        });
      }
      __syncthreads();
      const float Ate = cA[te - t0], Bte = cB[te - t0], Pc = cP;
      {
        Op<T> ops[2] = {{D2TM, WP, XwT, WP, WP}, {mom ? D2TS : nullptr, WP, XwT, WP, WP}};
        gemm_nt(DV, DP, ops, [&](int o, int f, const float* a) {
          if (f < D) {
            const size_t e = (size_t)o * D + f;
            const float m = Wt[e], s = mom ? Mo[e] : 0.f;
            const float nm = Ate * m + Bte * s - a[0];
            Wt[e] = nm;
            Mb[o * DP + f] = from_f<T>(nm);
            if (mom) {
              const float ns = Pc * s - a[1];
              Mo[e] = ns;
              Sb[o * DP + f] = from_f<T>(ns);
            }
          }
        });
      }
      __syncthreads();
    }
  }

  // ---- halo of the last c-1 tokens (oldest first) and the token count.
  // Slot j takes token N-(c-1)+j: from this call if >= 0, else from old slot
  // N+j >= j, which increasing-j order has not overwritten yet.
  if (threadIdx.x < 64 && pm == 0) {
    const int lane = threadIdx.x;
    for (int j = 0; j < c - 1; ++j) {
      const int i = N - (c - 1) + j;
      for (int d = lane; d < DK; d += 64) hk[j * DK + d] = i >= 0 ? to_f(k[(size_t)i * DK + d]) : hk[(N + j) * DK + d];
      for (int o = lane; o < DV; o += 64) hv[j * DV + o] = i >= 0 ? to_f(v[(size_t)i * DV + o]) : hv[(N + j) * DV + o];
      if (lane == 0) hg[j] = i >= 0 ? gam_in[i] : hg[N + j];
      if (lane == 0 && huber) hd[j] = i >= 0 ? dl_in[i] : hd[N + j];
    }
    if (lane == 0) *cnt += N;
  }
}

// ----------------------------------------------------------------------------- launch
template <class S>
hipError_t launch(const ChunkParams& cp, const CoeffParams& kp, int n_seq, hipStream_t stream,
                  hipEvent_t ev0, hipEvent_t ev1) {
  if (cp.N == 0 || n_seq == 0) return hipSuccess;
  hipLaunchKernelGGL((coeff_kernel<S::BC, S::WP>), dim3((unsigned)kp.nchunks * (unsigned)n_seq), dim3(256), 0, stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  if (cp.muon) {
    // LDS for Newton-Schulz's B when every orientation has at most 128 rows
    constexpr long r1 = S::MEM == MEM_MLP ? lmax(ns_r(S::H, S::D), ns_r(S::DV, S::H)) : ns_r(S::DV, S::D);
    constexpr size_t bs = r1 <= 128 ? (size_t)r1 * (r1 + 4) * 4 : 0;
    static bool attr = false;
    if (!attr) {
      attr = true;
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_kernel<S, 512>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)bs);
    }
    hipLaunchKernelGGL((chunk_kernel<S, 512>), dim3(cp.group > 1 ? (unsigned)((n_seq + 7) / 8) * 16u : (unsigned)n_seq),
                       dim3(512), bs, stream, cp);
  }
  else if constexpr (S::H >= 512 || S::D >= 256)
    // wide memories: a second wave per SIMD hides more of the GEMMs' load
    // latency (atlas-style 688-512-128: 836 -> 617 ms per call; linear on
    // 560 features: 7.48 -> 6.67 ms)
    hipLaunchKernelGGL((chunk_kernel<S, 512>), dim3(n_seq), dim3(512), 0, stream, cp);
  else
    hipLaunchKernelGGL((chunk_kernel<S, 256>), dim3(n_seq), dim3(256), 0, stream, cp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return hipSuccess;
}

#define ATLAS_VARIANT(NAME, ...)                                                            \
  typedef Shape<__VA_ARGS__> NAME;                                                          \
  template hipError_t launch<NAME>(const ChunkParams&, const CoeffParams&, int, hipStream_t, \
                                   hipEvent_t, hipEvent_t);

#include "atlas_mem_variants.inc"

}  // namespace atlas
