// atlas_mem_stream.hip -- MLP memory, one workgroup per sequence, the fp32
// weights and momentum streamed through the workgroup once per chunk.
//
// Method (as in atlas_mem_kernels.hip): per chunk of BC tokens, gradients of
// the Omega-rule window loss (ATLAS review sec. 3.2-3.3) at the chunk-start
// weights, folded into momentum and decay (Titans review sec. 3.1) through the
// gate coefficients A_t, B_t, C_{t,i}, cM_i, cS_i, P, and the retrieval
// y_t = f_{W_t}(q_t) with the per-token weights (Titans review sec. 3.1,
// "Retrieving a Memory").  Per chunk, with X the window keys, Xq the queries:
//   Z = X W1^T, A = gelu(Z), D2 = s*gamma*(x + A W2^T - v)         (l2 bias)
//   D1 = (D2 W2) .* gelu'(Z)
//   Zq = A_q Xq W1^T + B_q Xq S1^T - Q1 D1,  Ah = gelu(Zq),  Q1 = C .* Xq X^T
//   y  = q + A_q Ah W2^T + B_q Ah S2^T - (C .* Ah A^T) D2
//   W1 <- a W1 + b S1 - (cM .* D1)^T X,   S1 <- P S1 - (cS .* D1)^T X
//   W2 <- a W2 + b S2 - D2^T (cM .* A),   S2 <- P S2 - D2^T (cS .* A)
//
// Work split.  The hidden units are visited in super tiles of HJ = 64; wave w
// owns units 16w..16w+15 of the tile for everything indexed by hidden unit
// (Z, D1, Zq, the W1/S1 rows) and value rows DVW*w .. +DVW for everything
// indexed by value row (the W2/S2 rows, the sums A W2^T and Ah W2^T, the
// output).  One pass over the super tiles per chunk reads and writes the
// state once; it also runs the NEXT chunk's forward (Z' = X' W1'^T and its
// sum A' W2'^T) on each tile right after the tile's update, so the next
// chunk's D2 is ready when the pass ends and no second pass is needed.  The
// cross-tile sums (A' W2'^T, Ah W2^T, Ah A^T) stay in registers.
//
// The state tiles use the register layout of MFMA result tiles; as operands
// they are read in perm32 order (atlas_mem_frag.h).  Transposed operands are
// read from LDS with ds_read_b64_tr_b16, so every LDS matrix is stored once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "atlas_mem_internal.h"
#include "atlas_mem_coeff.h"
#include "atlas_mem_frag.h"
#include "atlas_mem_bias.h"
#include "atlas_mem_group.h"
#include "atlas_mem_group_split.h"
#include "atlas_mem_lds_sync.h"

namespace atlas {
namespace streamed {

using namespace mfma;

__device__ __forceinline__ bf16x8 zero8() {
  return bf16x8{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
}

template <int D_, int DV_, int H_, int WP_, int BC_, int G_>
struct TShape {
  static constexpr int D = D_, DV = DV_, H = H_, WP = WP_, BC = BC_, G = G_;
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int HJ = 16 * NW;           // hidden units per super tile
  static constexpr int NJ = H / HJ / G;        // super tiles per member of a group
  static_assert(G == 1 || G == 2, "groups of one or two workgroups");
  static_assert((H / HJ) % G == 0, "super tiles split evenly");
  static constexpr int DVW = DV / NW;          // value rows per wave
  static constexpr int NDT = DVW / 16;
  static constexpr int ND = D / 16;
  static constexpr int NT = WP / 16;           // window token tiles
  static constexpr int NQ = BC / 16;           // query tiles
  static constexpr int NU = HJ / 16;           // unit tiles per super tile
  static_assert(H % HJ == 0 && DVW % 16 == 0 && D % 32 == 0 && WP % 32 == 0 && BC % 32 == 0, "tiles");
  // LDS row strides in bf16 elements (multiples of 8: 16-byte aligned rows)
  static constexpr int LX = D + 8, LV = DV + 8, LT = WP + 8, LH = HJ + 8, LQ = BC + 4, L1Q = WP + 4;
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  //   Xa, Xb : window keys of this chunk and the next [WP][LX] (ping-pong)
  //   Xq     : queries [BC][LX];  Q1 [BC][L1Q] (read 8 bytes at a time);  D2 [WP][LV]
  //   AT     : A^T of the super tile [HJ][LT];  at the end of a pass Q2^T [WP][LQ]
  //   W2     : bf16 image W2^T [DV][LH];  after its use the next chunk's A'^T [HJ][LT];
  //            between passes, with Ah, the value rows of the next window [WP][LV]
  //   Ah     : retrieval activations of the super tile [BC][LH]
  //   Cm     : the weights C_{t,i} of the chunk, bf16 [BC][WP]
  static constexpr size_t szX = align_up((size_t)WP * LX * 2, 256);
  static constexpr size_t oXa = 0, oXb = oXa + szX, oXq = oXb + szX;
  static constexpr size_t oQ1 = oXq + align_up((size_t)BC * LX * 2, 256);
  static constexpr size_t oD2 = oQ1 + align_up((size_t)BC * L1Q * 2, 256);
  static constexpr size_t oAT = oD2 + align_up((size_t)WP * LV * 2, 256);
  static constexpr size_t oW2 = oAT + align_up(mx((size_t)HJ * LT, (size_t)WP * LQ) * 2, 256);
  static constexpr size_t oAh = oW2 + align_up(mx((size_t)DV * LH, (size_t)HJ * LT) * 2, 256);
  static constexpr size_t oCm = oAh + align_up((size_t)BC * LH * 2, 256);  // C [BC][WP] (bf16)
  // gate coefficients in the order of the coefficient kernel's block (A, B,
  // P and 3 spare words, cM, cS), then gamma of the window rows
  static constexpr size_t oF = oCm + align_up((size_t)BC * WP * 2, 256);
  static constexpr size_t lds = oF + (2 * BC + 3 * WP + 4) * 4;   // + s*gamma of the window rows
  static_assert(lds <= 163840, "LDS budget of one CU");
  static_assert(oAh - oW2 + align_up((size_t)BC * LH * 2, 256) >= (size_t)WP * LV * 2, "value rows fit W2 + Ah");
  static_assert(oAh + align_up((size_t)BC * LH * 2, 256) == oCm, "W2 and Ah regions are contiguous");
  // exchange workspace per sequence (G = 2): per chunk parity and member,
  // the partial sums A' W2'^T [NT][NDT] and y [NQ][NDT] as per-lane f32x4
  // tiles in lane order (both members use the same lane layout)
  static constexpr size_t tile_bytes = 256 * 16;
  // the state between passes: one block per super tile J and wave w (block
  // J * NW + w) of lane-ordered f32x4 tiles, 1 KB each: this wave's W1 rows
  // [ND], S1 rows [ND], W2 values [NU][NDT], S2 values [NU][NDT] (fp32), then
  // A = gelu(Z) and gelu'(Z) of the tile at the next window [NT] (bf16, saved
  // for the next pass, which is spared the recomputation of Z)
  static constexpr int TW1 = 0, TS1 = ND, TW2 = 2 * ND, TS2 = 2 * ND + NU * NDT, TAG = 2 * ND + 2 * NU * NDT;
  static constexpr int NTB = TAG + NT;            // tiles per block
  static constexpr size_t SB = (size_t)NTB * 1024;
  static constexpr size_t xTS = 0;
  static constexpr size_t ts_bytes = (size_t)(H / HJ) * NW * SB;
  static constexpr size_t xYh = xTS + ts_bytes;
  static constexpr size_t xYp = xYh + 2ull * G * NT * NDT * tile_bytes;
  static constexpr size_t xbytes = G == 1 ? xYh : xYp + 2ull * G * NQ * NDT * tile_bytes;
  static_assert(D == DV, "one tile-major stride for both layers");
  static_assert(WP <= 2 * BC, "windows of chunks >= 1 start inside the call");
  static_assert((size_t)(1 + NW) * WP * 4 <= mx((size_t)HJ * LT, (size_t)WP * LQ) * 2, "Huber scratch fits AT");
  static_assert((size_t)(4 * WP + 2 * BC) * NW * 4 <= mx((size_t)HJ * LT, (size_t)WP * LQ) * 2, "LN scratch fits AT");
};

// SHAPE: 0 for the l2 and dot-product biases, BIAS_LP or BIAS_HUBER for the
// biases that form D2 from whole error rows; LNORM: the layer-norm memory
// r + LN(W2 gelu(W1 x)) (with any bias but dot under a SHAPE).  Each instance
// holds only its own code.
template <class S, int SHAPE, bool LNORM>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
stream_mlp_kernel(ShardedParams p) {
  constexpr int D = S::D, DV = S::DV, H = S::H, WP = S::WP, BC = S::BC;
  constexpr int HJ = S::HJ, NJ = S::NJ, NDT = S::NDT, ND = S::ND, NT = S::NT, NQ = S::NQ, NU = S::NU;
  constexpr int LX = S::LX, LV = S::LV, LT = S::LT, LH = S::LH, LQ = S::LQ, L1Q = S::L1Q;
  constexpr int oCM = 2 * BC + 4, oCS = oCM + WP, oCC = oCS + WP, oQ1g = oCC + BC * WP, oCbg = oQ1g + BC * L1Q / 2;
  static_assert(L1Q == q1_pitch(WP, true), "Q1 of the coefficient block is the LDS image");
  extern __shared__ __attribute__((aligned(256))) char smem[];

  // group membership (G = 2): XCD-aware, as in the sharded kernel: block b
  // runs on XCD b % 8 and the members of a group are blocks 8*(gi*G + p) + xcd
  constexpr int G = S::G;
  int seq = blockIdx.x, pm = 0;
  if constexpr (G > 1) {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    pm = slot % G;
    seq = (slot / G) * 8 + xcd;
  }
  if (seq >= p.n_seq) return;
  const int J0 = pm * NJ;   // first super tile of this member
  unsigned* ctr = G > 1 ? p.ctrl + 1 + seq : nullptr;
  unsigned* err = p.ctrl;
  unsigned* xmask = G > 1 ? p.ctrl + 1 + p.n_seq + seq : nullptr;
  if (G > 1 && threadIdx.x == 0) report_xcc(xmask);
  unsigned nbar = 0;
  char* xw = p.xws + (size_t)seq * S::xbytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int N = p.N, c = p.c, W = BC + c - 1;
  const bool mom = p.momentum != 0, dot = p.bias == BIAS_DOT, res = p.residual != 0;
  const float s_grad = p.grad_scale;
  // l_p and Huber biases reshape the errors once whole rows are known
  constexpr bool shaped = SHAPE != 0, huber = SHAPE == BIAS_HUBER, lnorm = LNORM;
  // the layer norm's scratch follows the Huber deltas when both are in use
  static_assert(!(LNORM && SHAPE == BIAS_HUBER) ||
                    (size_t)(WP + (4 * WP + 2 * BC) * S::NW) * 4 <= S::oW2 - S::oAT,
                "layer-norm scratch after the Huber deltas fits AT");
  const float ln_eps = p.ln_eps;
  const float bias_p = p.bias_p, sign_alpha = p.sign_alpha;

  char* st = p.state + (size_t)seq * p.seq_stride;
  float* W1g = reinterpret_cast<float*>(st + p.off_weights);
  float* W2g = W1g + (size_t)H * D;
  float* S1g = reinterpret_cast<float*>(st + p.off_momentum);
  float* S2g = S1g + (size_t)H * D;
  float* hk = reinterpret_cast<float*>(st + p.off_halo_k);
  float* hv = reinterpret_cast<float*>(st + p.off_halo_v);
  float* hg = reinterpret_cast<float*>(st + p.off_halo_g);
  float* hd = reinterpret_cast<float*>(st + p.off_halo_d);   // Huber only
  int64_t* cnt = reinterpret_cast<int64_t*>(st + p.off_count);
  const int halo_valid = (int)min<int64_t>(*cnt, (int64_t)(c - 1));
  const bf16* q = reinterpret_cast<const bf16*>(p.q) + (size_t)seq * N * D;
  const bf16* k = reinterpret_cast<const bf16*>(p.k) + (size_t)seq * N * D;
  const bf16* v = reinterpret_cast<const bf16*>(p.v) + (size_t)seq * N * DV;
  bf16* out = reinterpret_cast<bf16*>(p.out) + (size_t)seq * N * DV;
  const float* gam_in = p.gamma + (size_t)seq * N;
  const float* dl_in = huber ? p.delta + (size_t)seq * N : nullptr;
  const float* coef_seq = p.coef + (size_t)seq * p.nchunks * p.coef_stride;

  bf16* Xc = reinterpret_cast<bf16*>(smem + S::oXa);   // window keys of the current chunk
  bf16* Xn = reinterpret_cast<bf16*>(smem + S::oXb);   // ... and of the next one
  bf16* Xq = reinterpret_cast<bf16*>(smem + S::oXq);
  bf16* Q1 = reinterpret_cast<bf16*>(smem + S::oQ1);
  bf16* D2 = reinterpret_cast<bf16*>(smem + S::oD2);
  bf16* AT = reinterpret_cast<bf16*>(smem + S::oAT);
  bf16* Q2T = AT;
  // Huber: thresholds of the window rows and the four waves' partial |e|^2
  // per row, in the AT region (free from the end of a pass's exchange to its
  // next tile, and in the prologue)
  float* dlw = reinterpret_cast<float*>(smem + S::oAT);
  float* rn = dlw + WP;
  // layer norm: per-wave partial row sums in the same region, four arrays
  // [NW][WP] for the window rows, two [NW][BC] for the output rows
  float* lnS = reinterpret_cast<float*>(smem + S::oAT) + (LNORM && SHAPE == BIAS_HUBER ? WP : 0);
  bf16* W2L = reinterpret_cast<bf16*>(smem + S::oW2);
  bf16* An = W2L;
  bf16* Ah = reinterpret_cast<bf16*>(smem + S::oAh);
  bf16* Cm = reinterpret_cast<bf16*>(smem + S::oCm);
  float* cA = reinterpret_cast<float*>(smem + S::oF);
  float* cB = cA + BC;
  float* cP = cB + BC;
  float* cM = cP + 4;
  float* cS = cM + WP;
  float* sgw = cS + WP;   // gamma of the window rows (0 outside the window)

  const int dvw = S::DVW * wave;
  const int nchunks = (N + BC - 1) / BC;

  // token i (relative to the call start) of window row w, and its validity
  auto row_ok = [&](int w, int t0, int te) {
    const int i = t0 - (c - 1) + w;
    return w < W && i >= -halo_valid && i <= te;
  };

  // Inputs of a chunk are moved in two halves: the loads into registers
  // (issued early, so their latency overlaps other work), then the LDS stores.
  // HALO = false for chunks >= 1, whose windows never reach before the call.
  constexpr int NXV = (WP * (D / 8) + 255) / 256;   // window key vectors per thread
  constexpr int NQV = (BC * (D / 8) + 255) / 256;   // query vectors per thread
  constexpr int NQ1V = (BC * L1Q / 8 + 255) / 256;  // Q1 vectors per thread (LDS image, pitch L1Q)
  constexpr int NCV = (BC * WP / 8 + 255) / 256;    // C (bf16) vectors per thread
  struct WinRegs { bf16x8 x[NXV]; };
  struct ChunkRegs { bf16x8 q[NQV], q1[NQ1V], cc[NCV]; float ca, cb, cm, cs, cp, sg; };
  struct D2Regs { bf16x4 vv[NT][NDT]; };

  // window keys of chunk ch (halo rows from the state, invalid rows zero)
  auto load_window = [&](int ch, WinRegs& R, auto halo_tag) {
    const int tid = fresh(threadIdx.x);
    constexpr bool HALO = decltype(halo_tag)::value;
    const int t0 = ch * BC, te = min(N, t0 + BC) - 1;
#pragma unroll
    for (int u = 0; u < NXV; ++u) {
      const int e = tid + 256 * u, w = e / (D / 8), d8 = (e % (D / 8)) * 8, i = t0 - (c - 1) + w;
      const bool ok = (WP * (D / 8) % 256 == 0 || e < WP * (D / 8)) && row_ok(w, t0, te);
      if (HALO) {
#pragma unroll
        for (int z = 0; z < 8; ++z) R.x[u][z] = (bf16)0.f;
        if (ok) {
          if (i >= 0) R.x[u] = *reinterpret_cast<const bf16x8*>(k + (size_t)i * D + d8);
          else
#pragma unroll
            for (int z = 0; z < 8; ++z) R.x[u][z] = (bf16)hk[(c - 1 + i) * D + d8 + z];
        }
      } else {
        // branch-free: a clamped (always valid) row, then a select
        const unsigned ic = (unsigned)min(max(i, 0), N - 1);
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(k + ic * D + d8);
        bf16x8 zz;
#pragma unroll
        for (int z = 0; z < 8; ++z) zz[z] = (bf16)0.f;
        R.x[u] = ok ? x : zz;
      }
    }
  };
  auto store_window = [&](bf16* Xdst, const WinRegs& R) {
    const int tid = fresh(threadIdx.x);
#pragma unroll
    for (int u = 0; u < NXV; ++u) {
      const int e = tid + 256 * u;
      if (e < WP * (D / 8)) *reinterpret_cast<bf16x8*>(Xdst + (e / (D / 8)) * LX + (e % (D / 8)) * 8) = R.x[u];
    }
  };

  // queries, Q1, the weights C, the gate coefficients and s*gamma of the
  // window rows of chunk ch
  auto load_chunk = [&](int ch, ChunkRegs& R, auto halo_tag) {
    const int tid = fresh(threadIdx.x);
    constexpr bool HALO = decltype(halo_tag)::value;
    const int t0 = ch * BC, te = min(N, t0 + BC) - 1;
    const float* coef = coef_seq + (size_t)ch * p.coef_stride;
#pragma unroll
    for (int u = 0; u < NQV; ++u) {
      const int e = tid + 256 * u, n = e / (D / 8), d8 = (e % (D / 8)) * 8;
      const bool ok = (BC * (D / 8) % 256 == 0 || e < BC * (D / 8)) && t0 + n <= te;
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(q + (unsigned)min(t0 + n, N - 1) * D + d8);
      bf16x8 zz;
#pragma unroll
      for (int z = 0; z < 8; ++z) zz[z] = (bf16)0.f;
      R.q[u] = ok ? x : zz;
    }
    const bf16* q1g = reinterpret_cast<const bf16*>(coef + oQ1g);
#pragma unroll
    for (int u = 0; u < NQ1V; ++u) {
      const int e = tid + 256 * u;
      if (e < BC * L1Q / 8) R.q1[u] = *reinterpret_cast<const bf16x8*>(q1g + 8 * e);
    }
    const bf16* cbg = reinterpret_cast<const bf16*>(coef + oCbg);
#pragma unroll
    for (int u = 0; u < NCV; ++u) {
      const int e = tid + 256 * u;
      if (e < BC * WP / 8) R.cc[u] = *reinterpret_cast<const bf16x8*>(cbg + 8 * e);
    }
    R.ca = tid < BC ? coef[tid] : 0.f;
    R.cb = tid < BC ? coef[BC + tid] : 0.f;
    R.cm = tid < WP ? coef[oCM + tid] : 0.f;
    R.cs = tid < WP ? coef[oCS + tid] : 0.f;
    R.cp = coef[2 * BC];
    {
      const int i = t0 - (c - 1) + tid;
      const bool ok = tid < WP && row_ok(tid, t0, te);
      if (HALO) R.sg = ok ? (i >= 0 ? gam_in[i] : hg[c - 1 + i]) : 0.f;
      else R.sg = ok ? gam_in[(unsigned)min(max(i, 0), N - 1)] : 0.f;
    }
  };
  auto store_chunk = [&](const ChunkRegs& R) {
    const int tid = fresh(threadIdx.x);
#pragma unroll
    for (int u = 0; u < NQV; ++u) {
      const int e = tid + 256 * u;
      if (e < BC * (D / 8)) *reinterpret_cast<bf16x8*>(Xq + (e / (D / 8)) * LX + (e % (D / 8)) * 8) = R.q[u];
    }
#pragma unroll
    for (int u = 0; u < NQ1V; ++u) {
      const int e = tid + 256 * u;
      if (e < BC * L1Q / 8) *reinterpret_cast<bf16x8*>(Q1 + 8 * e) = R.q1[u];
    }
#pragma unroll
    for (int u = 0; u < NCV; ++u) {
      const int e = tid + 256 * u;
      if (e < BC * WP / 8) *reinterpret_cast<bf16x8*>(Cm + 8 * e) = R.cc[u];
    }
    if (tid < BC) { cA[tid] = R.ca; cB[tid] = R.cb; }
    if (tid < WP) { cM[tid] = R.cm; cS[tid] = R.cs; }
    if (tid == 0) cP[0] = R.cp;
    if (tid < WP) sgw[tid] = R.sg;
  };

  // D2 of chunk ch from the sums yh = A W2^T of its window (Xw: its window
  // keys).  yh is held transposed: tile [m][bb] gives lane l the window row
  // w = 16 m + (l & 15) and the four value columns o = dvw + 16 bb + 4 (l >> 4) + r,
  // so every access below moves four adjacent bf16.
  f32x4 yh[NT][NDT];
  auto load_d2 = [&](int ch, D2Regs& R) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
    const int t0 = ch * BC, te = min(N, t0 + BC) - 1;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16, i = t0 - (c - 1) + w;
      const bool ok = row_ok(w, t0, te);
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const int o = dvw + 16 * bb + 4 * g;
        bf16x4 x = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        if (ok) {
          if (i >= 0) x = *reinterpret_cast<const bf16x4*>(v + (size_t)i * DV + o);
          else
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (bf16)hv[(c - 1 + i) * DV + o + r];
        }
        R.vv[m][bb] = x;
      }
    }
  };
  // one element of D2 (rows outside the window have sg = 0)
  auto d2_of = [&](float sg, float x, float y, float vv) {
    float t = y + (res ? x : 0.f);
    t = dot ? 0.f : t;
    return (bf16)(sg * (t - vv));
  };
  // l_p / Huber: D2 = s gamma slope(e) from the errors e, which have replaced
  // the window sums in yh.  The Huber choice needs each row's |e|_2: the
  // lanes of a row within a wave add over xor-shuffles, the four waves
  // through rn.  Needs sgw (and for Huber dlw) of the chunk in LDS.
  auto shape_d2 = [&]() __attribute__((always_inline)) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, wv = threadIdx.x >> 6;
    const int dvw = S::DVW * wv;
    if (huber) {
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        float s2 = 0.f;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s2 = fmaf(yh[m][bb][r], yh[m][bb][r], s2);
        s2 += __shfl_xor(s2, 16);
        s2 += __shfl_xor(s2, 32);
        if (g == 0) rn[wv * WP + 16 * m + c16] = s2;
      }
      lds_sync();
    }
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16;
      const float sg = s_grad * sgw[w];
      bool small = true;
      float dl = 0.f;
      if (huber) {
        const float n2 = ((rn[w] + rn[WP + w]) + rn[2 * WP + w]) + rn[3 * WP + w];
        dl = dlw[w];
        small = sqrtf(n2) <= dl;
      }
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        bf16x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = yh[m][bb][r];
          d[r] = (bf16)(sg * (huber ? huber_slope(e, small, dl, sign_alpha) : lp_slope(e, bias_p, sign_alpha)));
        }
        *reinterpret_cast<bf16x4*>(D2 + w * LV + dvw + 16 * bb + 4 * g) = d;
      }
    }
  };
  // sum over the four lane groups that hold one row of a transposed tile
  auto rowsum = [&](float v) {
    v += __shfl_xor(v, 16);
    return v + __shfl_xor(v, 32);
  };
  auto across = [&](const float* P, int n, int w) { return ((P[w] + P[n + w]) + P[2 * n + w]) + P[3 * n + w]; };
  // Layer norm: the branch u is in yh (window sums), t holds v - r (l2, l_p,
  // Huber) or v (dot).  Mean and variance of u per row (two passes),
  // nhat = (u - mean) / sd, the error e = nhat - t = y - v, the slope g = e
  // (l2), -t (dot), the l_p or Huber slope of e (Huber: the row's |e|_2
  // against its delta, a third pass), then
  // D2 = s gamma (g - mean(g) - nhat mean(g nhat)) / sd.
  auto ln_d2 = [&](const float (&t)[NT][NDT][4]) __attribute__((always_inline)) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, wv = threadIdx.x >> 6;
    const int dvw = S::DVW * wv;
    float* A_ = lnS;
    float* B_ = A_ + S::NW * WP;
    float* C_ = B_ + S::NW * WP;
    float* E_ = C_ + S::NW * WP;
    float mu[NT], rs[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      float sum = 0.f;
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += yh[m][bb][r];
      sum = rowsum(sum);
      if (g == 0) A_[wv * WP + 16 * m + c16] = sum;
    }
    lds_sync();
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      mu[m] = across(A_, WP, 16 * m + c16) * (1.f / DV);
      float sum = 0.f;
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = yh[m][bb][r] - mu[m];
          sum = fmaf(d, d, sum);
        }
      sum = rowsum(sum);
      if (g == 0) B_[wv * WP + 16 * m + c16] = sum;
    }
    lds_sync();
#pragma unroll
    for (int m = 0; m < NT; ++m) rs[m] = 1.f / sqrtf(across(B_, WP, 16 * m + c16) * (1.f / DV) + ln_eps);
    bool small[NT];
    float dl[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      small[m] = true;
      dl[m] = 0.f;
    }
    if constexpr (huber) {
      // every wave read A_ (the means) before the barrier above
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        float s2 = 0.f;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = (yh[m][bb][r] - mu[m]) * rs[m] - t[m][bb][r];
            s2 = fmaf(e, e, s2);
          }
        s2 = rowsum(s2);
        if (g == 0) A_[wv * WP + 16 * m + c16] = s2;
      }
      lds_sync();
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const int w = 16 * m + c16;
        dl[m] = dlw[w];
        small[m] = sqrtf(across(A_, WP, w)) <= dl[m];
      }
    }
    auto slope = [&](float nh, float tv, int m) {
      if constexpr (huber) return huber_slope(nh - tv, small[m], dl[m], sign_alpha);
      else if constexpr (shaped) return lp_slope(nh - tv, bias_p, sign_alpha);
      else return dot ? -tv : nh - tv;
    };
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float nh = (yh[m][bb][r] - mu[m]) * rs[m];
          const float gg = slope(nh, t[m][bb][r], m);
          s1 += gg;
          s2 = fmaf(gg, nh, s2);
        }
      s1 = rowsum(s1);
      s2 = rowsum(s2);
      if (g == 0) {
        C_[wv * WP + 16 * m + c16] = s1;
        E_[wv * WP + 16 * m + c16] = s2;
      }
    }
    lds_sync();
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16;
      const float sg = s_grad * sgw[w];
      const float mg = across(C_, WP, w) * (1.f / DV), mgn = across(E_, WP, w) * (1.f / DV);
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        bf16x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float nh = (yh[m][bb][r] - mu[m]) * rs[m];
          const float gg = slope(nh, t[m][bb][r], m);
          d[r] = (bf16)(sg * (gg - mg - nh * mgn) * rs[m]);
        }
        *reinterpret_cast<bf16x4*>(D2 + w * LV + dvw + 16 * bb + 4 * g) = d;
      }
    }
  };
  // chunk 0 (window rows may come from the halo); needs sgw of the chunk in LDS
  auto finish_d2 = [&](int ch, const D2Regs& R, const bf16* Xw) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
    const int t0 = ch * BC;
    float tln[lnorm ? NT : 1][NDT][4];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16, i = t0 - (c - 1) + w;
      const float sg = s_grad * sgw[w];
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const int o = dvw + 16 * bb + 4 * g;
        float xr[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (D == DV) {
          if (i >= 0 || sg == 0.f) {
            const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(Xw + w * LX + o);
#pragma unroll
            for (int r = 0; r < 4; ++r) xr[r] = (float)x4[r];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) xr[r] = hk[(c - 1 + i) * D + o + r];
          }
        }
        if constexpr (lnorm) {
#pragma unroll
          for (int r = 0; r < 4; ++r) tln[m][bb][r] = (float)R.vv[m][bb][r] - (res && !dot ? xr[r] : 0.f);
        } else if constexpr (shaped) {
#pragma unroll
          for (int r = 0; r < 4; ++r) yh[m][bb][r] += (res ? xr[r] : 0.f) - (float)R.vv[m][bb][r];
        } else {
          bf16x4 d;
#pragma unroll
          for (int r = 0; r < 4; ++r) d[r] = d2_of(sg, xr[r], yh[m][bb][r], (float)R.vv[m][bb][r]);
          *reinterpret_cast<bf16x4*>(D2 + w * LV + o) = d;
        }
      }
    }
    if constexpr (lnorm) ln_d2(tln);
    else if constexpr (shaped) shape_d2();
  };
  // chunks >= 1, l_p / Huber: the errors from the staged value rows Vw
  auto shaped_d2_lds = [&](const bf16* Vw, const bf16* Xw) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16;
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const int o = dvw + 16 * bb + 4 * g;
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(Vw + w * LV + o);
        bf16x4 x4 = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        if constexpr (D == DV) x4 = *reinterpret_cast<const bf16x4*>(Xw + w * LX + o);
#pragma unroll
        for (int r = 0; r < 4; ++r) yh[m][bb][r] += (res ? (float)x4[r] : 0.f) - (float)v4[r];
      }
    }
    shape_d2();
  };
  // chunks >= 1, layer norm: the targets from the staged value rows Vw
  auto ln_d2_lds = [&](const bf16* Vw, const bf16* Xw) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
    float t[NT][NDT][4];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16;
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const int o = dvw + 16 * bb + 4 * g;
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(Vw + w * LV + o);
        bf16x4 x4 = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        if constexpr (D == DV) x4 = *reinterpret_cast<const bf16x4*>(Xw + w * LX + o);
#pragma unroll
        for (int r = 0; r < 4; ++r) t[m][bb][r] = (float)v4[r] - (res && !dot ? (float)x4[r] : 0.f);
      }
    }
    ln_d2(t);
  };
  // chunks >= 1: from the staged value rows Vw, branch-free
  auto finish_d2_lds = [&](const bf16* Vw, const bf16* Xw) {
    const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int w = 16 * m + c16;
      const float sg = s_grad * sgw[w];
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const int o = dvw + 16 * bb + 4 * g;
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(Vw + w * LV + o);
        bf16x4 x4 = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        if constexpr (D == DV) x4 = *reinterpret_cast<const bf16x4*>(Xw + w * LX + o);
        bf16x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = d2_of(sg, (float)x4[r], yh[m][bb][r], (float)v4[r]);
        *reinterpret_cast<bf16x4*>(D2 + w * LV + o) = d;
      }
    }
  };

  // State tiles.  Two layouts: the row-major one of the call's state buffer
  // (W1 [H][D], W2 [DV][H], the momentum alike), copied into the workspace's
  // blocks before the first pass and back after the last, and the blocks
  // (see the layout notes at the top), in which every access of a wave is one
  // contiguous 1 KB tile.  A block access is the lane offset vT, the tile's
  // place within its 4 KB (the compiler keeps the three sums of vT in
  // registers, or folds them into the instruction's immediate offset) and a
  // wave-uniform scalar offset in steps of 4 KB.
  const int wave_s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rT = buffer_of(xw + S::xTS, (unsigned)S::ts_bytes);
  const int vT = (threadIdx.x & 63) * 16;
  auto blk = [&](int J, int T) { return (J * S::NW + wave_s) * (int)S::SB + (T / 4) * 4096; };
  auto tld = [&](int J, int T) -> f32x4 { return buf_load4(rT, vT + (T % 4) * 1024, blk(J, T)); };
  auto tst = [&](const f32x4& x, int J, int T) { buf_store4(x, rT, vT + (T % 4) * 1024, blk(J, T)); };
  // which: 0 = W1, 1 = S1 (tile t of this wave's rows)
  auto ld1 = [&](int which, int J, int t) { return tld(J, (which ? S::TS1 : S::TW1) + t); };
  auto st1 = [&](const f32x4& x, int which, int J, int t) { tst(x, J, (which ? S::TS1 : S::TW1) + t); };
  // which: 0 = W2, 1 = S2 (unit tile a, value tile bb of this wave's rows)
  auto ld2 = [&](int which, int J, int a, int bb) { return tld(J, (which ? S::TS2 : S::TW2) + a * NDT + bb); };
  auto st2 = [&](const f32x4& x, int which, int J, int a, int bb) {
    tst(x, J, (which ? S::TS2 : S::TW2) + a * NDT + bb);
  };
  // Row-major <-> blocks: each lane moves the f32x4 it holds in both (the
  // MFMA tile layout: unit row 16 w + (l & 15), four columns at 4 (l >> 4)).
  // Without momentum the caller's momentum is never touched (a descriptor of
  // size zero: loads read zeros, stores are dropped) and the blocks' S holds
  // the zeros read here, so S stays zero without branches.
  auto convert = [&](bool to_blocks) {
    const __amdgpu_buffer_rsrc_t rW = buffer_of(W1g, 2u * H * D * 4);
    const __amdgpu_buffer_rsrc_t rM = buffer_of(S1g, mom ? 2u * H * D * 4 : 0u);
    const int vW1 = (threadIdx.x & 15) * D * 4 + ((threadIdx.x >> 4) & 3) * 16;
    const int vW2 = (threadIdx.x & 15) * H * 4 + ((threadIdx.x >> 4) & 3) * 16;
    for (int J = J0; J < J0 + NJ; ++J) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const __amdgpu_buffer_rsrc_t r = which ? rM : rW;
        f32x4 x[ND], y[NU][NDT];
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          const int so = (J * HJ + 16 * wave_s) * D * 4 + 64 * t;
          x[t] = to_blocks ? buf_load4(r, vW1, so) : ld1(which, J, t);
        }
#pragma unroll
        for (int a = 0; a < NU; ++a)
#pragma unroll
          for (int bb = 0; bb < NDT; ++bb) {
            const int so = H * D * 4 + (S::DVW * wave_s + 16 * bb) * H * 4 + (J * HJ + 16 * a) * 4;
            y[a][bb] = to_blocks ? buf_load4(r, vW2, so) : ld2(which, J, a, bb);
          }
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          const int so = (J * HJ + 16 * wave_s) * D * 4 + 64 * t;
          if (to_blocks) st1(x[t], which, J, t);
          else buf_store4(x[t], r, vW1, so);
        }
#pragma unroll
        for (int a = 0; a < NU; ++a)
#pragma unroll
          for (int bb = 0; bb < NDT; ++bb) {
            const int so = H * D * 4 + (S::DVW * wave_s + 16 * bb) * H * 4 + (J * HJ + 16 * a) * 4;
            if (to_blocks) st2(y[a][bb], which, J, a, bb);
            else buf_store4(y[a][bb], r, vW2, so);
          }
      }
    }
  };

  // State prefetch, one super tile ahead, into loop-carried registers: the
  // W1/S1 rows of the tile and the W2 values of its bf16 image.  They are
  // issued after the loads the current tile still waits for (vmcnt retires in
  // order), so no wait in the current tile covers them.
  f32x4 pW1[ND], pS1[ND], pW2[NU][NDT], pAG[NT];
  auto prefetch = [&](int J) {
#pragma unroll
    for (int i = 0; i < NT; ++i) pAG[i] = tld(J, S::TAG + i);
#pragma unroll
    for (int t = 0; t < ND; ++t) {
      pW1[t] = ld1(0, J, t);
      pS1[t] = ld1(1, J, t);   // without momentum: zeros
    }
#pragma unroll
    for (int a = 0; a < NU; ++a)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) pW2[a][bb] = ld2(0, J, a, bb);
  };

  // Forward of super tile J on a window Xs with first-layer rows W1 (this
  // wave's 16 units): Z [tok x unit] = Xs W1^T, A = gelu(Z) -> An^T [unit][tok]
  // in LDS, and A, gelu'(Z) saved (bf16, lane order) for the pass that will
  // update this tile with this window.
  auto forward_tile = [&](const bf16* Xs, const f32x4 (&W1)[ND], int J) {
    const int lane = fresh(threadIdx.x) & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
    f32x4 z1[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) z1[m] = zero4();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const bf16x8 bw = tiles_to_frag(W1[2 * s], W1[2 * s + 1]);
#pragma unroll
      for (int m = 0; m < NT; ++m) z1[m] = mma(ld_perm(Xs, LX, 16 * m, 32 * s, lane), bw, z1[m]);
    }
    bf16x8 ca[NT / 2], cd[NT / 2];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      bf16x4 a4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a, da;
        gelu_and_prime(z1[m][r], a, da);
        a4[r] = (bf16)a;
        ca[m / 2][4 * (m % 2) + r] = a4[r];
        cd[m / 2][4 * (m % 2) + r] = (bf16)da;
      }
      *reinterpret_cast<bf16x4*>(An + (16 * wave + c16) * LT + 16 * m + 4 * g) = a4;
    }
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      tst(__builtin_bit_cast(f32x4, ca[i]), J, S::TAG + i);
      tst(__builtin_bit_cast(f32x4, cd[i]), J, S::TAG + NT / 2 + i);
    }
  };
  // A' W2'^T of the tile into the window sums (after An^T is complete)
  auto window_sums = [&](const f32x4 (&W2)[NU][NDT]) {
    const int lane = fresh(threadIdx.x) & 63;
#pragma unroll
    for (int s = 0; s < HJ / 32; ++s)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        const bf16x8 bw = tiles_to_frag(W2[2 * s][bb], W2[2 * s + 1][bb]);
#pragma unroll
        for (int m = 0; m < NT; ++m) yh[m][bb] = mma(bw, ld_tr_perm(An, LT, 16 * m, 32 * s, lane), yh[m][bb]);
      }
  };

  // lane-ordered exchange of per-lane accumulator tiles with the partner
  // (G = 2): tile i of member m at xw + base + (i * 256 + tid) * 16
  auto xYh_at = [&](int par, int m) { return S::xYh + ((size_t)par * G + m) * NT * NDT * S::tile_bytes; };
  auto xYp_at = [&](int par, int m) { return S::xYp + ((size_t)par * G + m) * NQ * NDT * S::tile_bytes; };
  auto xput = [&](size_t off, const f32x4 (&a)[NT][NDT]) {
    f32x4* d = reinterpret_cast<f32x4*>(xw + off) + threadIdx.x;
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) d[(m * NDT + bb) * 256] = a[m][bb];
  };
  auto xadd = [&](size_t off, f32x4 (&a)[NT][NDT]) {
    const f32x4* d = reinterpret_cast<const f32x4*>(xw + off) + threadIdx.x;
    f32x4 t[NT][NDT];
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) t[m][bb] = d[(m * NDT + bb) * 256];
    __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first add
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) a[m][bb] += t[m][bb];
  };

  // The inputs of chunk cn (cn >= 1) that the passes read from LDS, and the
  // keys of chunk cn + 1's window, loaded straight into LDS (no registers), so
  // the loads overlap the exchange with the partner; invalid rows read zeros.
  // Needs every wave past its last read of the target regions.
  auto stage_next = [&](int cn) {
    const int lane = fresh(threadIdx.x) & 63;
    const int t0n = cn * BC, ten = min(N, t0n + BC) - 1, wb = t0n - (c - 1);
    const __amdgpu_buffer_rsrc_t rV = buffer_of(v, (unsigned)N * DV * 2);
    const __amdgpu_buffer_rsrc_t rK = buffer_of(k, (unsigned)N * D * 2);
    const __amdgpu_buffer_rsrc_t rQ = buffer_of(q, (unsigned)N * D * 2);
    const __amdgpu_buffer_rsrc_t rG = buffer_of(gam_in, (unsigned)N * 4);
    const __amdgpu_buffer_rsrc_t rC = buffer_of(coef_seq, (unsigned)nchunks * p.coef_stride * 4);
    const int cb = cn * p.coef_stride * 4;   // byte offset of the chunk's coefficient block
    // value rows of the window -> W2L [WP][LV] (with the Ah region)
    // (window rows of chunks >= 1 start at token >= 0: valid iff w < W and token <= te)
    auto win = [&](int w, int wb_, int te_) { return (w < W) & (wb_ + w <= te_); };
    rows_to_lds<16, WP, DV * 2, LV * 2, S::NW>(rV, reinterpret_cast<char*>(W2L), wave_s, lane,
                                               [&](int w) { return win(w, wb, ten) ? (wb + w) * DV * 2 : -1; });
    // keys of the window of chunk cn + 1 -> Xc (free: the pass is done with it)
    if (cn + 1 < nchunks) {
      const int t0w = t0n + BC, tew = min(N, t0w + BC) - 1;
      rows_to_lds<16, WP, D * 2, LX * 2, S::NW>(rK, reinterpret_cast<char*>(Xc), wave_s, lane, [&](int w) {
        return win(w, t0w - (c - 1), tew) ? (t0w - (c - 1) + w) * D * 2 : -1;
      });
    }
    // queries -> Xq [BC][LX]
    rows_to_lds<16, BC, D * 2, LX * 2, S::NW>(rQ, reinterpret_cast<char*>(Xq), wave_s, lane,
                                              [&](int n) { return t0n + n <= ten ? (t0n + n) * D * 2 : -1; });
    // A, B, P, cM, cS (fp32, the block's layout) -> cA ..
    constexpr int NCF = (2 * BC + 4 + 2 * WP) * 4;
    rows_to_lds<16, 1, NCF, NCF, S::NW>(rC, reinterpret_cast<char*>(cA), wave_s, lane, [&](int) { return cb; });
    // Q1 (bf16, already in the LDS image [BC][L1Q]): one contiguous block
    rows_to_lds<16, 1, BC * L1Q * 2, BC * L1Q * 2, S::NW>(rC, reinterpret_cast<char*>(Q1), wave_s, lane,
                                                          [&](int) { return cb + oQ1g * 4; });
    // C (bf16 [BC][WP]) -> Cm
    rows_to_lds<16, 1, BC * WP * 2, BC * WP * 2, S::NW>(rC, reinterpret_cast<char*>(Cm), wave_s, lane,
                                                        [&](int) { return cb + oCbg * 4; });
    // gamma of the window rows
    rows_to_lds<4, WP, 4, 4, S::NW>(rG, reinterpret_cast<char*>(sgw), wave_s, lane,
                                    [&](int w) { return win(w, wb, ten) ? (wb + w) * 4 : -1; });
    // Huber: their thresholds (AT region, free now)
    if (huber) {
      const __amdgpu_buffer_rsrc_t rD = buffer_of(dl_in, (unsigned)N * 4);
      rows_to_lds<4, WP, 4, 4, S::NW>(rD, reinterpret_cast<char*>(dlw), wave_s, lane,
                                      [&](int w) { return win(w, wb, ten) ? (wb + w) * 4 : -1; });
    }
  };

  // ---- the state into the blocks
  convert(true);

  // ---- prologue: inputs of chunk 0 (and the keys of chunk 1), then chunk 0's forward
  if (nchunks > 0) {
    WinRegs w0, w1;
    ChunkRegs c0;
    D2Regs d0;
    load_window(0, w0, std::true_type{});
    if (nchunks > 1) load_window(1, w1, std::false_type{});
    load_chunk(0, c0, std::true_type{});
    load_d2(0, d0);
    store_window(Xc, w0);
    if (nchunks > 1) store_window(Xn, w1);
    store_chunk(c0);
    if (huber && tid < WP) {
      const int i = -(c - 1) + tid;
      dlw[tid] = row_ok(tid, 0, min(N, BC) - 1) ? (i >= 0 ? dl_in[i] : hd[c - 1 + i]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) yh[m][bb] = zero4();
    for (int J = J0; J < J0 + NJ; ++J) {
      f32x4 W1T[ND], W2T[NU][NDT];
#pragma unroll
      for (int t = 0; t < ND; ++t) W1T[t] = ld1(0, J, t);
#pragma unroll
      for (int a = 0; a < NU; ++a)
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) W2T[a][bb] = ld2(0, J, a, bb);
      forward_tile(Xc, W1T, J);
      __syncthreads();
      window_sums(W2T);
      __syncthreads();
    }
    if constexpr (G > 1) {
      // the partner's partial sums of the window forward
      const int par = 1;   // chunk 0 uses parity 0; the prologue the other slot
      xput(xYh_at(par, pm), yh);
      group_barrier(ctr, G * (++nbar), err);
      if (tid == 0) check_xcc(xmask, err);
      xadd(xYh_at(par, 1 - pm), yh);
    }
    prefetch(J0);
    finish_d2(0, d0, Xc);
    __syncthreads();
  }

  // ---- one pass over the super tiles per chunk
  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * BC, te = min(N, t0 + BC) - 1, ce = te - t0;
    const bool more = ch + 1 < nchunks;
    const float Ate = cA[ce], Bte = cB[ce], Pc = cP[0];
    // Ah W2^T, Ah S2^T (scaled by A_q, B_q at the end), held transposed like
    // yh: tile [m][bb] gives lane l the query row 16 m + (l & 15) and the value
    // columns dvw + 16 bb + 4 (l >> 4) + r
    f32x4 yw[NQ][NDT], ys[NQ][NDT], q2[NT];
#pragma unroll
    for (int m = 0; m < NQ; ++m)
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) {
        yw[m][bb] = zero4();
        ys[m][bb] = zero4();
      }
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      q2[m] = zero4();
#pragma unroll
      for (int bb = 0; bb < NDT; ++bb) yh[m][bb] = zero4();
    }

    for (int J = J0; J < J0 + NJ; ++J) {
      // per-iteration lane ids: keeps the lane-dependent LDS address
      // arithmetic inside the loop instead of in registers across the call
      const int tid = fresh(threadIdx.x), lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
      const int dvw = S::DVW * wave;
      // ======== W1 side: W1/S1 in registers, W2 only long enough for its bf16 image
      f32x4 W1T[ND], S1T[ND];
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        W1T[t] = pW1[t];
        S1T[t] = pS1[t];
      }
      // ---- bf16 image W2^T [dv][unit] of the tile (this wave's value rows)
#pragma unroll
      for (int a = 0; a < NU; ++a)
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          const f32x4 w = pW2[a][bb];
          *reinterpret_cast<bf16x4*>(W2L + (dvw + 16 * bb + c16) * LH + 16 * a + 4 * g) =
              bf16x4{(bf16)w[0], (bf16)w[1], (bf16)w[2], (bf16)w[3]};
        }
      // ---- A = gelu(Z) and gelu'(Z) of this tile at this chunk's window, saved
      // by the previous pass (or the prologue): A -> AT [unit][tok], z = gelu'
      f32x4 z[NT];
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const bf16x8 ca = __builtin_bit_cast(bf16x8, pAG[m / 2]);
        const bf16x8 cd = __builtin_bit_cast(bf16x8, pAG[NT / 2 + m / 2]);
        bf16x4 a4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a4[r] = ca[4 * (m % 2) + r];
          z[m][r] = (float)cd[4 * (m % 2) + r];
        }
        *reinterpret_cast<bf16x4*>(AT + (16 * wave + c16) * LT + 16 * m + 4 * g) = a4;
      }
      lds_sync();   // W2 image, AT

      // ---- D1 = (D2 W2) .* gelu'(Z) [tok x 16 units], then perm32 operands over tokens
      bf16x8 fd[NT / 2], fm[NT / 2], fs[NT / 2];
      {
        f32x4 d1[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) d1[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DV; k0 += 32) {
          const bf16x8 bw = ld_tr_nat(W2L, LH, 16 * wave, k0, lane);
#pragma unroll
          for (int m = 0; m < NT; ++m) d1[m] = mma(ld_nat(D2, LV, 16 * m, k0, lane), bw, d1[m]);
        }
#pragma unroll
        for (int s = 0; s < NT / 2; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tl = 32 * s + 4 * g + r, th = tl + 16;
            const float lo = d1[2 * s][r] * z[2 * s][r], hi = d1[2 * s + 1][r] * z[2 * s + 1][r];
            fd[s][r] = (bf16)(-lo);
            fd[s][4 + r] = (bf16)(-hi);
            fm[s][r] = (bf16)(-(lo * cM[tl]));
            fm[s][4 + r] = (bf16)(-(hi * cM[th]));
            fs[s][r] = (bf16)(-(lo * cS[tl]));
            fs[s][4 + r] = (bf16)(-(hi * cS[th]));
          }
        // without momentum S and its operands are zero, so every momentum
        // product below is an exact zero and needs no branch
#pragma unroll
        for (int s = 0; s < NT / 2; ++s) fs[s] = mom ? fs[s] : zero8();
      }

      // ---- Zq^T = A_q (W1 Xq^T) + B_q (S1 Xq^T) - D1^T Q1^T [16 units x q]; Ah = gelu
      {
        f32x4 a1[NQ], a2[NQ], a3[NQ];
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          a1[m] = zero4();
          a2[m] = zero4();
          a3[m] = zero4();
        }
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 aw = tiles_to_frag(W1T[2 * s], W1T[2 * s + 1]);
          const bf16x8 as = tiles_to_frag(S1T[2 * s], S1T[2 * s + 1]);
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const bf16x8 xb = ld_perm(Xq, LX, 16 * m, 32 * s, lane);
            a1[m] = mma(aw, xb, a1[m]);
            a2[m] = mma(as, xb, a2[m]);
          }
        }
#pragma unroll
        for (int s = 0; s < NT / 2; ++s)
#pragma unroll
          for (int m = 0; m < NQ; ++m) a3[m] = mma(fd[s], ld_perm(Q1, L1Q, 16 * m, 32 * s, lane), a3[m]);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          const float qa = cA[16 * m + c16], qb = cB[16 * m + c16];
          bf16x4 h4;
#pragma unroll
          for (int r = 0; r < 4; ++r) h4[r] = (bf16)gelu(fmaf(qa, a1[m][r], fmaf(qb, a2[m][r], a3[m][r])));
          *reinterpret_cast<bf16x4*>(Ah + (16 * m + c16) * LH + 16 * wave + 4 * g) = h4;
        }
      }

      // ---- W1/S1 update [d x 16 units]: the products accumulate onto the
      // decayed state (their operands fm, fs carry the minus sign); written
      // back at once
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        f32x4 um, us;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w1 = W1T[t][r], s1 = S1T[t][r];
          um[r] = Ate * w1 + Bte * s1;
          us[r] = Pc * s1;
        }
#pragma unroll
        for (int s = 0; s < NT / 2; ++s) {
          const bf16x8 xa = ld_tr_perm(Xc, LX, 16 * t, 32 * s, lane);
          um = mma(xa, fm[s], um);
          us = mma(xa, fs[s], us);
        }
        W1T[t] = um;
        S1T[t] = us;
        st1(W1T[t], 0, J, t);
        st1(S1T[t], 1, J, t);
      }
      lds_sync();   // Ah complete; every wave is done with the W2 image

      // ---- next chunk's forward on the updated rows: A' -> An^T, saved for the next pass
      if (more) forward_tile(Xn, W1T, J);

      // ======== W2 side: W2/S2 (this wave's value rows, recently loaded: in L2),
      // then the next tile's prefetch
      f32x4 W2T[NU][NDT], S2T[NU][NDT];
#pragma unroll
      for (int a = 0; a < NU; ++a)
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          W2T[a][bb] = ld2(0, J, a, bb);
          S2T[a][bb] = ld2(1, J, a, bb);
        }
      // (the next pass's first tile is fetched after the chunk inputs are staged)
      if (J + 1 < J0 + NJ) prefetch(J + 1);
      // ---- Q2 partial: Ah A^T, this wave's 16 query rows [q x tok]
#pragma unroll
      for (int k0 = 0; k0 < HJ; k0 += 32) {
        const bf16x8 ah = ld_nat(Ah, LH, 16 * wave, k0, lane);
#pragma unroll
        for (int m = 0; m < NT; ++m) q2[m] = mma(ah, ld_tr_nat(AT, LT, 16 * m, k0, lane), q2[m]);
      }
      // ---- output partials: Ah W2^T and Ah S2^T [q x this wave's dv]
#pragma unroll
      for (int s = 0; s < HJ / 32; ++s) {
        bf16x8 bw[NDT], bs[NDT];
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          bw[bb] = tiles_to_frag(W2T[2 * s][bb], W2T[2 * s + 1][bb]);
          bs[bb] = tiles_to_frag(S2T[2 * s][bb], S2T[2 * s + 1][bb]);
        }
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          const bf16x8 ah = ld_perm(Ah, LH, 16 * m, 32 * s, lane);
#pragma unroll
          for (int bb = 0; bb < NDT; ++bb) {
            yw[m][bb] = mma(bw[bb], ah, yw[m][bb]);
            ys[m][bb] = mma(bs[bb], ah, ys[m][bb]);
          }
        }
      }
      // ---- W2/S2 update [units x this wave's dv]: A^T (cM .* D2), the D2
      // operand scaled along the tokens (and negated: the products accumulate
      // onto the decayed state); written back at once
      {
        bf16x8 dm[NDT][NT / 2], ds[NDT][NT / 2];
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int s = 0; s < NT / 2; ++s) {
            const bf16x8 bd = ld_tr_nat(D2, LV, dvw + 16 * bb, 32 * s, lane);
            const float* sm = cM + 32 * s + 8 * g;
            const float* ss = cS + 32 * s + 8 * g;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float x = (float)bd[i];
              dm[bb][s][i] = (bf16)(-(x * sm[i]));
              ds[bb][s][i] = (bf16)(-(x * ss[i]));
            }
            ds[bb][s] = mom ? ds[bb][s] : zero8();
          }
#pragma unroll
        for (int a = 0; a < NU; ++a) {
          bf16x8 at[NT / 2];
#pragma unroll
          for (int s = 0; s < NT / 2; ++s) at[s] = ld_nat(AT, LT, 16 * a, 32 * s, lane);
#pragma unroll
          for (int bb = 0; bb < NDT; ++bb) {
            f32x4 um, us;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float w2 = W2T[a][bb][r], s2 = S2T[a][bb][r];
              um[r] = Ate * w2 + Bte * s2;
              us[r] = Pc * s2;
            }
#pragma unroll
            for (int s = 0; s < NT / 2; ++s) {
              um = mma(at[s], dm[bb][s], um);
              us = mma(at[s], ds[bb][s], us);
            }
            W2T[a][bb] = um;
            S2T[a][bb] = us;
            st2(W2T[a][bb], 0, J, a, bb);
            st2(S2T[a][bb], 1, J, a, bb);
          }
        }
      }
      // ---- next chunk's window sums A' W2'^T [tok x this wave's dv]
      if (more) {
        lds_sync();   // An^T complete
        window_sums(W2T);
      }
      lds_sync();
    }

    // ---- end of the pass: Q2 = C .* (Ah A^T) -> Q2^T [tok][q]
    {
    const int tid = fresh(threadIdx.x), lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      bf16x4 c4;
#pragma unroll
      for (int r = 0; r < 4; ++r) c4[r] = (bf16)((float)Cm[(16 * wave + 4 * g + r) * WP + 16 * m + c16] * q2[m][r]);
      *reinterpret_cast<bf16x4*>(Q2T + (16 * m + c16) * LQ + 16 * wave + 4 * g) = c4;
    }
    }
    lds_sync();
    // this member's part of y - q = A_q Ah W2^T + B_q Ah S2^T - Q2 D2 (transposed tiles)
    f32x4 yp[NQ][NDT];
    {
      const int lane = fresh(threadIdx.x) & 63, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        const float a = cA[16 * m + c16], b = cB[16 * m + c16];
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          f32x4 acc = zero4();
#pragma unroll
          for (int k0 = 0; k0 < WP; k0 += 32)
            acc = mma(ld_tr_nat(D2, LV, dvw + 16 * bb, k0, lane), ld_tr_nat(Q2T, LQ, 16 * m, k0, lane), acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) yp[m][bb][r] = fmaf(a, yw[m][bb][r], fmaf(b, ys[m][bb][r], -acc[r]));
        }
      }
    }
    // G = 2: exchange the partial sums; each member writes half of the output
    // rows, and hands the partner only the tiles of the partner's half
    constexpr int MQ = NQ / G;
    const int mlo = pm * MQ;
    // the residual part of this member's output rows, read before the next
    // chunk's queries replace Xq
    bf16x4 xres[MQ][NDT];
    {
      const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
#pragma unroll
      for (int mi = 0; mi < MQ; ++mi)
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          xres[mi][bb] = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
          if constexpr (D == DV)
            xres[mi][bb] = *reinterpret_cast<const bf16x4*>(Xq + (16 * (mlo + mi) + c16) * LX + dvw + 16 * bb + 4 * g);
        }
    }
    const int par = ch & 1;
    if constexpr (G > 1) {
      {
        f32x4* d = reinterpret_cast<f32x4*>(xw + xYp_at(par, pm)) + threadIdx.x;
#pragma unroll
        for (int m = 0; m < NQ; ++m)
          if (m < mlo || m >= mlo + MQ)
#pragma unroll
            for (int bb = 0; bb < NDT; ++bb) d[(m * NDT + bb) * 256] = yp[m][bb];
      }
      if (more) xput(xYh_at(par, pm), yh);
      // ---- the next chunk's inputs into LDS, in flight during the wait for
      // the partner, its reads and the output stores: every wave is past
      // its last read of the target regions once it has arrived (the
      // residual rows are in registers already)
      group_arrive(ctr);
      if (more) stage_next(ch + 1);
      group_wait(ctr, G * (++nbar), err);
    } else {
      lds_sync();
      if (more) stage_next(ch + 1);
    }
    if constexpr (G > 1) {
      if (more) xadd(xYh_at(par, 1 - pm), yh);
      // every tile is loaded (the ones of the other half are not used), all
      // before the first add, so the partner's partials cost one round trip
      const f32x4* d = reinterpret_cast<const f32x4*>(xw + xYp_at(par, 1 - pm)) + threadIdx.x;
      f32x4 tp[NQ][NDT];
#pragma unroll
      for (int m = 0; m < NQ; ++m)
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) tp[m][bb] = d[(m * NDT + bb) * 256];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        const bool mine = m >= mlo && m < mlo + MQ;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) yp[m][bb][r] += mine ? tp[m][bb][r] : 0.f;
      }
    }
    if constexpr (lnorm) {
      // y = r + LN(u) on this member's rows: mean and variance of each row of
      // u (yp) over the four lane groups and the four waves
      const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, wv = threadIdx.x >> 6;
      float* OA = lnS + 4 * S::NW * WP;
      float* OB = OA + S::NW * BC;
      float mu[MQ], rs[MQ];
#pragma unroll
      for (int mi = 0; mi < MQ; ++mi) {
        float sum = 0.f;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sum += yp[mlo + mi][bb][r];
        sum = rowsum(sum);
        if (g == 0) OA[wv * BC + 16 * mi + c16] = sum;
      }
      lds_sync();
#pragma unroll
      for (int mi = 0; mi < MQ; ++mi) {
        mu[mi] = across(OA, BC, 16 * mi + c16) * (1.f / DV);
        float sum = 0.f;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = yp[mlo + mi][bb][r] - mu[mi];
            sum = fmaf(d, d, sum);
          }
        sum = rowsum(sum);
        if (g == 0) OB[wv * BC + 16 * mi + c16] = sum;
      }
      lds_sync();
#pragma unroll
      for (int mi = 0; mi < MQ; ++mi) {
        rs[mi] = 1.f / sqrtf(across(OB, BC, 16 * mi + c16) * (1.f / DV) + ln_eps);
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) yp[mlo + mi][bb][r] = (yp[mlo + mi][bb][r] - mu[mi]) * rs[mi];
      }
    }
    {
      // four adjacent values of one output row per lane and tile
      const int lane = fresh(threadIdx.x) & 63, g = lane >> 4, c16 = lane & 15, dvw = S::DVW * (threadIdx.x >> 6);
#pragma unroll
      for (int mi = 0; mi < MQ; ++mi) {
        const int m = mlo + mi, qq = 16 * m + c16;
        if (t0 + qq > te) continue;
#pragma unroll
        for (int bb = 0; bb < NDT; ++bb) {
          const int o = dvw + 16 * bb + 4 * g;
          bf16x4 y4;
#pragma unroll
          for (int r = 0; r < 4; ++r) y4[r] = (bf16)(yp[m][bb][r] + (res ? (float)xres[mi][bb][r] : 0.f));
          *reinterpret_cast<bf16x4*>(out + (size_t)(t0 + qq) * DV + o) = y4;
        }
      }
    }
    if (more) {
      wait_vmem();       // this wave's loads into LDS have landed
      lds_sync();   // and everyone's
      if constexpr (lnorm) ln_d2_lds(W2L, Xn);
      else if constexpr (shaped) shaped_d2_lds(W2L, Xn);
      else finish_d2_lds(W2L, Xn);
      prefetch(J0);
      bf16* tmp = Xc;
      Xc = Xn;
      Xn = tmp;
      lds_sync();
    }
  }

  // ---- the state back to the caller's layout
  convert(false);

  // ---- halo and count (every read of the old halo happened in the
  // prologue; with G = 2 the barrier orders it after the partner's reads)
  if constexpr (G > 1) group_barrier(ctr, G * (++nbar), err);
  if (pm == 0 && tid < 64) {
    for (int j = 0; j < c - 1; ++j) {
      const int i = N - (c - 1) + j;
      for (int d = lane; d < D; d += 64) hk[j * D + d] = i >= 0 ? (float)k[(size_t)i * D + d] : hk[(N + j) * D + d];
      for (int o = lane; o < DV; o += 64) hv[j * DV + o] = i >= 0 ? (float)v[(size_t)i * DV + o] : hv[(N + j) * DV + o];
      if (lane == 0) hg[j] = i >= 0 ? gam_in[i] : hg[N + j];
      if (lane == 0 && huber) hd[j] = i >= 0 ? dl_in[i] : hd[N + j];
    }
    if (lane == 0) *cnt += N;
  }
}

}  // namespace streamed

template <int D, int DV, int H, int WP, int BC, int G>
hipError_t launch_streamed(const ShardedParams& sp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  typedef streamed::TShape<D, DV, H, WP, BC, G> S;
  if (sp.N == 0 || sp.n_seq == 0) return hipSuccess;
  hipLaunchKernelGGL((coeff_kernel<BC, WP, D, true>), dim3((unsigned)kp.nchunks * (unsigned)sp.n_seq), dim3(256), 0,
                     stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // instance: 0 plain, 1 l_p, 2 Huber, 3 layer norm (l2 / dot), 4 layer norm
  // with l_p, 5 layer norm with Huber
  const int shape = sp.bias == BIAS_LP ? 1 : sp.bias == BIAS_HUBER ? 2 : 0;
  const int inst = sp.layernorm ? (shape == 0 ? 3 : 3 + shape) : shape;
  const void* fns[6] = {reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, 0, false>),
                        reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, BIAS_LP, false>),
                        reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, BIAS_HUBER, false>),
                        reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, 0, true>),
                        reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, BIAS_LP, true>),
                        reinterpret_cast<const void*>(&streamed::stream_mlp_kernel<S, BIAS_HUBER, true>)};
  static bool attr_set[6] = {false, false, false, false, false, false};
  if (!attr_set[inst]) {
    // allow more than the default dynamic LDS; a refusal shows up at launch
    (void)hipFuncSetAttribute(fns[inst], hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::lds);
    (void)hipGetLastError();
    attr_set[inst] = true;
  }
  const unsigned blocks = G == 1 ? (unsigned)sp.n_seq : (unsigned)((sp.n_seq + 7) / 8) * 8u * G;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  switch (inst) {
    case 1: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, BIAS_LP, false>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
    case 2: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, BIAS_HUBER, false>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
    case 3: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, 0, true>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
    case 4: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, BIAS_LP, true>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
    case 5: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, BIAS_HUBER, true>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
    default: hipLaunchKernelGGL((streamed::stream_mlp_kernel<S, 0, false>), dim3(blocks), dim3(256), S::lds, stream, sp); break;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int D, int DV, int H, int WP, int BC, int G>
size_t streamed_xbytes() { return streamed::TShape<D, DV, H, WP, BC, G>::xbytes; }

#define ATLAS_STREAMED(NAME, D, DV, H, WP, BC, G, AUTO)                                                  \
  template hipError_t launch_streamed<D, DV, H, WP, BC, G>(const ShardedParams&, const CoeffParams&,      \
                                                           hipStream_t, hipEvent_t, hipEvent_t);          \
  template size_t streamed_xbytes<D, DV, H, WP, BC, G>();
#include "atlas_mem_stream_variants.inc"
#undef ATLAS_STREAMED

}  // namespace atlas
