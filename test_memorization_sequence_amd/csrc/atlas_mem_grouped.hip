// atlas_mem_grouped.hip -- MLP memory on a wide feature map (ATLAS review,
// sec. 3.1 "Polynomial Feature Mapping": [k, poly2(k[:p])] or
// [k, upper-tri(k k^T)]) with the hidden units of every sequence split over a
// group of G workgroups of one XCD, 16 hidden units per workgroup, the fp32
// weights and momentum resident in registers for the whole call.
//
// Method (as in atlas_mem_kernels.hip): per chunk of BC tokens, gradients of
// the Omega-rule window loss (ATLAS review sec. 3.2-3.3) at the chunk-start
// weights, folded into momentum and decay (Titans review sec. 3.1) through the
// gate coefficients A_t, B_t, C_{t,i}, cM_i, cS_i, P, and the retrieval
// y_t = f_{W_t}(phi(q_t)) with the per-token weights (Titans review sec. 3.1,
// "Retrieving a Memory").
//
// A call runs four kernels:
//   coeff_kernel     gate coefficients of every chunk (fp32 C included);
//   phi_kernel       phi of every key (rows and a feature-major copy, the
//                    halo of the state in front) and of every query, bf16
//                    (atlas_mem_phi.h);
//   q1_phi_kernel    Q1 = C .* (phi(Q) phi(K)^T) of every chunk (bf16 MFMA;
//                    atlas_mem_phi.h);
//   grouped_kernel   the recurrence.  Workgroup p of a group owns hidden units
//                    [16p, 16p + 16) of W1 (rows), W3 is absent, W2 (columns).
//                    Its 4 waves split the window rows (forward), the query
//                    rows (retrieval) and the feature columns (W1 update).
//                    Two sums over all hidden units cross the group through
//                    L2: the window forward A W2^T (reduce-scatter, then an
//                    all-gather of D2 = s gamma E; two group barriers per
//                    chunk) and the retrieval output (partials reduced by the
//                    group one chunk later).
//
// Window rows: row w of chunk t0 is token t0 - (c - 1) + w, w < 128 (rows at
// and beyond b + c - 1 carry zero coefficients), so row w of the phi buffers
// (which start c - 1 tokens before the call) is t0 + w: 16-byte aligned for
// the k-contiguous loads of both layouts.
//
// Every global access of the recurrence goes through a buffer descriptor sized
// to its array: an index out of range reads zero and drops the write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atlas_mem_internal.h"
#include "atlas_mem_coeff.h"
#include "atlas_mem_frag.h"
#include "atlas_mem_group.h"
#include "atlas_mem_group_split.h"
#include "atlas_mem_phi.h"

namespace atlas {

namespace grouped {

using namespace mfma;

// ----------------------------------------------------------------------------- shapes
template <int PHI_, int DK_, int PD_, int DV_, int H_, int G_>
struct GShape {
  static constexpr int PHI = PHI_, DK = DK_, PD = PD_, DV = DV_, H = H_, G = G_;
  static constexpr int D = feature_dim(PHI_, DK_, PD_);
  static constexpr int DP = (D + 63) / 64 * 64;   // features, padded to 4 waves x 16-column tiles
  static constexpr int BC = 64, WP = 128, NW = 4;
  static constexpr int HL = H / G;                // hidden units per workgroup
  static constexpr int NFW = DP / 64;             // W1 feature tiles per wave
  static constexpr int NDW = DV / 64;             // W2 value-row tiles per wave
  static constexpr int RW = WP / G, RQ = BC / G;  // rows each member reduces
  static_assert(HL == 16, "16 hidden units per workgroup");
  static_assert(DV % 64 == 0 && DK % 8 == 0, "tiles");
  static_assert(WP % G == 0 && BC % G == 0, "reduce split");
  // LDS (bf16 element pitches: multiples of 8, 16-byte rows)
  static constexpr int LF = DP + 8, LV = DV + 8, LT = WP + 8, LU = HL + 8;
  static constexpr size_t oW1 = 0;                                   // W1 image [16][LF]
  static constexpr size_t oS1 = oW1 + align_up(HL * LF * 2, 256);    // S1 image [16][LF]
  static constexpr size_t oW2 = oS1 + align_up(HL * LF * 2, 256);    // W2 image [16 units][LV]
  static constexpr size_t oS2 = oW2 + align_up(HL * LV * 2, 256);
  static constexpr size_t oAl = oS2 + align_up(HL * LV * 2, 256);    // A [WP][LU]
  static constexpr size_t oAT = oAl + align_up(WP * LU * 2, 256);    // A^T [16][LT]
  static constexpr size_t oD2 = oAT + align_up(HL * LT * 2, 256);    // D2 [WP][LV]
  static constexpr size_t oD1T = oD2 + align_up(WP * LV * 2, 256);   // D1^T [16][LT]
  static constexpr size_t oAh = oD1T + align_up(HL * LT * 2, 256);   // Ahat [BC][LU]
  static constexpr size_t oQ2 = oAh + align_up(BC * LU * 2, 256);    // Q2 [BC][LT]
  static constexpr size_t oC = oQ2 + align_up(BC * LT * 2, 256);     // C [BC][WP] f32 (coefficient block)
  static constexpr size_t oF = oC + BC * WP * 4;                      // cA[BC] cB[BC] cM[WP] cS[WP] P
  static constexpr size_t lds = oF + (2 * BC + 2 * WP + 4) * 4;
  // the reduce-scatter and the output reduction split their partial sums over
  // all 256 threads: NPAIR (row, 4 values) pairs, G / NSPLIT partials per thread
  static constexpr int NPAIR = RW * (DV / 4), NSPLIT = 256 / NPAIR;
  static constexpr int NPAIR_O = RQ * (DV / 4), NSPLIT_O = 256 / NPAIR_O;
  static_assert(256 % NPAIR == 0 && G % NSPLIT == 0 && 256 % NPAIR_O == 0 && G % NSPLIT_O == 0, "split");
  static_assert((NSPLIT - 1) * NPAIR * 16 + (NSPLIT_O - 1) * NPAIR_O * 16 <= BC * LT * 2, "combine scratch in Q2");
  static_assert(lds <= 163840, "LDS budget of one CU");
  // exchange workspace per sequence (bytes)
  static constexpr size_t xY = 0;                                          // [2][G][WP][DV] f32
  static constexpr size_t xD2 = xY + 2ull * G * WP * DV * 4;               // [2][WP][DV] bf16
  static constexpr size_t xYo = align_up(xD2 + 2ull * WP * DV * 2, 256);   // [2][G][BC][DV] f32
  static constexpr size_t xMask = align_up(xYo + 2ull * G * BC * DV * 4, 256);   // XCDs the members ran on
  static constexpr size_t xbytes = xMask + 256;
  // phi buffers per sequence for nch chunks (bytes): key rows [NR][DP], the
  // same feature-major [DP][NR], query rows [nch*BC][DP]; NR = nch*BC + BC
  __host__ __device__ static size_t rows_k(int nch) { return (size_t)nch * BC + BC; }
  __host__ __device__ static size_t oXR(int) { return xbytes; }
  __host__ __device__ static size_t oXT(int nch) { return align_up(oXR(nch) + rows_k(nch) * DP * 2, 256); }
  __host__ __device__ static size_t oXQ(int nch) { return align_up(oXT(nch) + rows_k(nch) * DP * 2, 256); }
  __host__ __device__ static size_t seq_bytes(int nch) { return align_up(oXQ(nch) + (size_t)nch * BC * DP * 2, 256); }
};

// ----------------------------------------------------------------------------- recurrence
template <class S>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
grouped_kernel(GroupedParams p) {
  constexpr int DK = S::DK, DV = S::DV, H = S::H, G = S::G, DP = S::DP, D = S::D, BC = S::BC, WP = S::WP;
  constexpr int HL = S::HL, NFW = S::NFW, NDW = S::NDW, RW = S::RW, RQ = S::RQ;
  constexpr int LF = S::LF, LV = S::LV, LT = S::LT, LU = S::LU;
  extern __shared__ __attribute__((aligned(256))) char smem[];

  // ---- XCD-aware group membership: members of group gi on XCD x are blocks 8 (gi G + p) + x
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int pm = slot % G, gi = slot / G;
  const int seq = gi * 8 + xcd;
  if (seq >= p.n_seq) return;
  unsigned* ctr = p.ctrl + 1 + seq;
  unsigned* err = p.ctrl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  unsigned* xmask = reinterpret_cast<unsigned*>(p.gws + (size_t)seq * p.gseq_bytes + S::xMask);
  // the barrier needs every member on one L2: each member reports the XCD it
  // runs on; checked after the first group barrier
  if (tid == 0) report_xcc(xmask);

  const int N = p.N, c = p.c, W = BC + c - 1, nch = p.nchunks;
  const bool mom = p.momentum != 0, dot = p.bias == BIAS_DOT, res = p.residual != 0;
  const float s_grad = p.grad_scale;

  char* st = p.state + (size_t)seq * p.seq_stride;
  float* Wt = reinterpret_cast<float*>(st + p.off_weights);
  float* Mo = reinterpret_cast<float*>(st + p.off_momentum);
  float* hk = reinterpret_cast<float*>(st + p.off_halo_k);
  float* hv = reinterpret_cast<float*>(st + p.off_halo_v);
  float* hg = reinterpret_cast<float*>(st + p.off_halo_g);
  int64_t* cnt = reinterpret_cast<int64_t*>(st + p.off_count);
  const int halo_valid = (int)min<int64_t>(*cnt, (int64_t)(c - 1));
  const bf16* q = reinterpret_cast<const bf16*>(p.q) + (size_t)seq * N * DK;
  const bf16* k = reinterpret_cast<const bf16*>(p.k) + (size_t)seq * N * DK;
  const bf16* v = reinterpret_cast<const bf16*>(p.v) + (size_t)seq * N * DV;
  bf16* out = reinterpret_cast<bf16*>(p.out) + (size_t)seq * N * DV;
  const float* gam_in = p.gamma + (size_t)seq * N;

  char* ws = p.gws + (size_t)seq * p.gseq_bytes;
  const __amdgpu_buffer_rsrc_t rxr = buffer_of(ws + S::oXR(nch), (unsigned)(S::rows_k(nch) * DP * 2));
  const __amdgpu_buffer_rsrc_t rxt = buffer_of(ws + S::oXT(nch), (unsigned)(S::rows_k(nch) * DP * 2));
  const __amdgpu_buffer_rsrc_t rxq = buffer_of(ws + S::oXQ(nch), (unsigned)((size_t)nch * BC * DP * 2));
  const __amdgpu_buffer_rsrc_t rxy = buffer_of(ws + S::xY, (unsigned)(2ull * G * WP * DV * 4));
  const __amdgpu_buffer_rsrc_t rxo = buffer_of(ws + S::xYo, (unsigned)(2ull * G * BC * DV * 4));
  bf16* d2buf = reinterpret_cast<bf16*>(ws + S::xD2);
  const float* yobuf = reinterpret_cast<const float*>(ws + S::xYo);
  const float* ybuf = reinterpret_cast<const float*>(ws + S::xY);
  const size_t NR = S::rows_k(nch);
  unsigned nbar = 0;

  bf16* W1i = reinterpret_cast<bf16*>(smem + S::oW1);
  bf16* S1i = reinterpret_cast<bf16*>(smem + S::oS1);
  bf16* W2i = reinterpret_cast<bf16*>(smem + S::oW2);
  bf16* S2i = reinterpret_cast<bf16*>(smem + S::oS2);
  bf16* Al = reinterpret_cast<bf16*>(smem + S::oAl);
  bf16* AT = reinterpret_cast<bf16*>(smem + S::oAT);
  bf16* D2 = reinterpret_cast<bf16*>(smem + S::oD2);
  bf16* D1T = reinterpret_cast<bf16*>(smem + S::oD1T);
  bf16* Ah = reinterpret_cast<bf16*>(smem + S::oAh);
  bf16* Q2 = reinterpret_cast<bf16*>(smem + S::oQ2);
  float* Cl = reinterpret_cast<float*>(smem + S::oC);
  float4* comb = reinterpret_cast<float4*>(smem + S::oQ2);   // partial-sum scratch (Q2 is dead then)
  float* cA = reinterpret_cast<float*>(smem + S::oF);
  float* cB = cA + BC;
  float* cM = cB + BC;
  float* cS = cM + WP;
  float* cP = cS + WP;

  // ---- state slices into registers
  //   W1T[t]: units 16 pm + 4g + r, feature fb + 16 t + c16 (fb = 16 NFW wave)
  //   W2T[t]: value rows 16 (NDW wave + t) + 4g + r, unit 16 pm + c16
  const int fb = 16 * NFW * wave;
  const int j0 = HL * pm;
  f32x4 W1T[NFW], S1T[NFW], W2T[NDW], S2T[NDW];
  {
    const __amdgpu_buffer_rsrc_t rw = buffer_of(Wt, (unsigned)(((size_t)H * D + (size_t)DV * H) * 4));
    const __amdgpu_buffer_rsrc_t rm = buffer_of(Mo, mom ? (unsigned)(((size_t)H * D + (size_t)DV * H) * 4) : 0u);
#pragma unroll
    for (int t = 0; t < NFW; ++t) {
      const int f = fb + 16 * t + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = f < D ? ((j0 + 4 * g + r) * D + f) * 4 : kZeroOffset;
        W1T[t][r] = gload1(rw, off);
        S1T[t][r] = gload1(rm, off);
      }
    }
#pragma unroll
    for (int t = 0; t < NDW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = (H * D + (16 * (NDW * wave + t) + 4 * g + r) * H + j0 + c16) * 4;
        W2T[t][r] = gload1(rw, off);
        S2T[t][r] = gload1(rm, off);
      }
  }
  // bf16 images of this workgroup's slices: W1/S1 [16 units][LF], W2/S2 [16 units][LV]
  auto write_images = [&]() {
#pragma unroll
    for (int t = 0; t < NFW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        W1i[(4 * g + r) * LF + fb + 16 * t + c16] = (bf16)W1T[t][r];
        S1i[(4 * g + r) * LF + fb + 16 * t + c16] = (bf16)S1T[t][r];
      }
#pragma unroll
    for (int t = 0; t < NDW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        W2i[c16 * LV + 16 * (NDW * wave + t) + 4 * g + r] = (bf16)W2T[t][r];
        S2i[c16 * LV + 16 * (NDW * wave + t) + 4 * g + r] = (bf16)S2T[t][r];
      }
  };
  write_images();

  // reduce the retrieval partials of chunk pc (query rows owned by this member)
  // into out: NSPLIT_O threads per (row, 4 values), each over G / NSPLIT_O
  // partials, combined through LDS
  auto reduce_out = [&](int pc) {
    constexpr int NP = S::NPAIR_O, NS = S::NSPLIT_O, PER = G / NS;
    const int pt0 = pc * BC, pte = min(N, pt0 + BC) - 1;
    const int tf = fresh(tid), e = tf % NP, h = tf / NP;
    const int qq = pm * RQ + e / (DV / 4), o4 = (e % (DV / 4)) * 4;
    const float* yo = yobuf + (size_t)(pc & 1) * G * BC * DV + (size_t)qq * DV + o4;
    float4 part[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) part[u] = *reinterpret_cast<const float4*>(yo + (size_t)(h * PER + u) * BC * DV);
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < PER; ++u) { y.x += part[u].x; y.y += part[u].y; y.z += part[u].z; y.w += part[u].w; }
    float4* cmb = comb + (S::NSPLIT - 1) * S::NPAIR;
    if (h > 0) cmb[(h - 1) * NP + e] = y;
    __syncthreads();
    if (h == 0 && pt0 + qq <= pte) {
#pragma unroll
      for (int u = 1; u < NS; ++u) {
        const float4 o = cmb[(u - 1) * NP + e];
        y.x += o.x; y.y += o.y; y.z += o.z; y.w += o.w;
      }
      if (res) {
        const bf16x4 r4 = *reinterpret_cast<const bf16x4*>(q + (size_t)(pt0 + qq) * DK + o4);
        y.x += (float)r4[0]; y.y += (float)r4[1]; y.z += (float)r4[2]; y.w += (float)r4[3];
      }
      *reinterpret_cast<bf16x4*>(out + (size_t)(pt0 + qq) * DV + o4) = bf16x4{(bf16)y.x, (bf16)y.y, (bf16)y.z, (bf16)y.w};
    }
  };

  const int R0 = 32 * wave;   // the wave's window rows (forward, backward)
  const int Q0 = 16 * wave;   // the wave's query rows (retrieval)
  for (int ch = 0; ch < nch; ++ch) {
    const int t0 = ch * BC;
    const int te = min(N, t0 + BC) - 1;
    const int sl = ch & 1;
    const float* coef = p.coef + ((size_t)seq * nch + ch) * p.coef_stride;
    const float* Cc = coef + 2 * BC + 4 + 2 * WP;                                    // [BC][WP] f32
    const bf16* Q1g = reinterpret_cast<const bf16*>(coef + 2 * BC + 4 + 2 * WP + BC * WP);   // [BC][WP]

    // ---- coefficients of the chunk; C straight into LDS (complete after the
    // first group barrier's wait for every memory access)
    {
      const __amdgpu_buffer_rsrc_t rc = buffer_of(Cc, (unsigned)(BC * WP * 4));
      rows_to_lds<16, BC, WP * 4, WP * 4, 4>(rc, reinterpret_cast<char*>(Cl), fresh(wave), fresh(lane),
                                            [&](int row) { return row * WP * 4; });
    }
    if (tid < BC) { cA[tid] = coef[tid]; cB[tid] = coef[BC + tid]; }
    if (tid < WP) { cM[tid] = coef[2 * BC + 4 + tid]; cS[tid] = coef[2 * BC + 4 + WP + tid]; }
    if (tid == 0) cP[0] = coef[2 * BC];
    __syncthreads();   // (also: the images of the previous update are complete)

    // ---- forward Z = X W1^T  [rows R0.. (2 tiles) x 16 units], K = DP; the
    // X fragments of step s + PF are loaded before step s computes
    f32x4 Z[2] = {zero4(), zero4()};
    {
      constexpr int NS = DP / 32, PF = 5;
      bf16x8 xf[PF + 1][2];
      // each member walks the K steps from its own starting step, so that the
      // 32 members of a group do not all read the same L2 lines at once
      const int k0 = pm % NS;
      auto kstep = [&](int st) { const int k = st + k0; return k < NS ? k : k - NS; };
      auto load = [&](int st, bf16x8* dst) {
        const int ks = kstep(st);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) dst[mt] = gload8(rxr, ((t0 + R0 + 16 * mt + c16) * DP + 32 * ks + 8 * g) * 2);
      };
#pragma unroll
      for (int st = 0; st < PF && st < NS; ++st) load(st, xf[st]);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (st + PF < NS) load(st + PF, xf[(st + PF) % (PF + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 bw = ld_nat(W1i, LF, 0, 32 * kstep(st), lane);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) Z[mt] = mma(xf[st % (PF + 1)][mt], bw, Z[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    f32x4 GP[2];   // gelu'(Z)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a, da;
        gelu_and_prime(Z[mt][r], a, da);
        GP[mt][r] = da;
        const int row = R0 + 16 * mt + 4 * g + r;
        Al[row * LU + c16] = (bf16)a;
        AT[c16 * LT + row] = (bf16)a;
      }
    __syncthreads();

    // ---- partial window forward Y_p = A W2_p^T  [rows R0.. x DV], K = 16 units,
    // computed transposed (W2_p A^T) so that each lane holds four adjacent
    // values of one row: one 16-byte store per tile
    {
      const int yb = ((sl * G + pm) * WP) * DV * 4;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(Al + (R0 + 16 * mt + c16) * LU + 4 * g);
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) {
          const f32x4 y = mma16(ld_tr16(W2i, LV, 16 * nt, 0, lane), a, zero4());
          buf_store4(y, rxy, yb + ((R0 + 16 * mt + c16) * DV + 16 * nt + 4 * g) * 4, 0);
        }
      }
    }
    // the retrieval's terms of the chunk-start state, A_q Xq W1^T and
    // B_q Xq S1^T (this member's 16 units; queries from L2, the state
    // images in LDS), need neither the partners' partials nor D1: they run
    // between this member's arrival at the barrier and its wait
    group_arrive(ctr);
    f32x4 ra1 = zero4(), ra2 = zero4();
    {
      const int qrow = t0 + Q0 + c16;
      constexpr int NS = DP / 32, PF = 8;
      const int k0 = pm % NS;   // per-member starting step, as in the forward
      auto kstep = [&](int st) { const int k = st + k0; return k < NS ? k : k - NS; };
      bf16x8 xf[PF + 1];
#pragma unroll
      for (int st = 0; st < PF && st < NS; ++st) xf[st] = gload8(rxq, (qrow * DP + 32 * kstep(st) + 8 * g) * 2);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (st + PF < NS) xf[(st + PF) % (PF + 1)] = gload8(rxq, (qrow * DP + 32 * kstep(st + PF) + 8 * g) * 2);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 xq = xf[st % (PF + 1)];
        const int ks = kstep(st);
        ra1 = mma(xq, ld_nat(W1i, LF, 0, 32 * ks, lane), ra1);
        if (mom) ra2 = mma(xq, ld_nat(S1i, LF, 0, 32 * ks, lane), ra2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    group_wait(ctr, G * (++nbar), err);
    if (ch == 0 && tid == 0) check_xcc(xmask, err);

    // ---- reduce-scatter: this member's window rows -> D2 rows; the previous chunk's outputs
    {
      constexpr int NP = S::NPAIR, NS = S::NSPLIT, PER = G / NS;
      const int tf = fresh(tid), e = tf % NP, h = tf / NP;
      const int w = pm * RW + e / (DV / 4), o4 = (e % (DV / 4)) * 4;
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!dot) {
        const float* yb = ybuf + (size_t)sl * G * WP * DV + (size_t)w * DV + o4;
        float4 part[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) part[u] = *reinterpret_cast<const float4*>(yb + (size_t)(h * PER + u) * WP * DV);
#pragma unroll
        for (int u = 0; u < PER; ++u) { y.x += part[u].x; y.y += part[u].y; y.z += part[u].z; y.w += part[u].w; }
      }
      if (h > 0) comb[(h - 1) * NP + e] = y;
      __syncthreads();
      if (h == 0) {
#pragma unroll
        for (int u = 1; u < NS; ++u) {
          const float4 o = comb[(u - 1) * NP + e];
          y.x += o.x; y.y += o.y; y.z += o.z; y.w += o.w;
        }
        const int i = t0 - (c - 1) + w;
        float4 pv = make_float4(0.f, 0.f, 0.f, 0.f), pr = pv;
        float pg = 0.f;
        if (w < W && i >= -halo_valid && i <= te) {
          if (i >= 0) {
            const bf16x4 vv = *reinterpret_cast<const bf16x4*>(v + (size_t)i * DV + o4);
            pv = make_float4((float)vv[0], (float)vv[1], (float)vv[2], (float)vv[3]);
            if (res) {
              const bf16x4 rr = *reinterpret_cast<const bf16x4*>(k + (size_t)i * DK + o4);
              pr = make_float4((float)rr[0], (float)rr[1], (float)rr[2], (float)rr[3]);
            }
            pg = gam_in[i];
          } else {
            pv = *reinterpret_cast<const float4*>(hv + (c - 1 + i) * DV + o4);
            if (res) pr = *reinterpret_cast<const float4*>(hk + (c - 1 + i) * DK + o4);
            pg = hg[c - 1 + i];
          }
        }
        const float sg = s_grad * pg;
        bf16x4 d4;
        if (dot) {
          d4 = bf16x4{(bf16)(-sg * pv.x), (bf16)(-sg * pv.y), (bf16)(-sg * pv.z), (bf16)(-sg * pv.w)};
        } else {
          d4 = bf16x4{(bf16)(sg * (pr.x + y.x - pv.x)), (bf16)(sg * (pr.y + y.y - pv.y)),
                      (bf16)(sg * (pr.z + y.z - pv.z)), (bf16)(sg * (pr.w + y.w - pv.w))};
        }
        *reinterpret_cast<bf16x4*>(d2buf + ((size_t)sl * WP + w) * DV + o4) = d4;
      }
    }
    // the previous chunk's outputs need neither this barrier nor the
    // partners' D2 rows (their partials were published at the first
    // barrier, and their slot is rewritten only after the next one): they
    // are reduced between this member's arrival and its wait
    group_arrive(ctr);
    if (ch > 0) reduce_out(ch - 1);
    group_wait(ctr, G * (++nbar), err);

    // ---- all-gather D2 -> LDS [WP][LV]
    {
      const bf16* d2b = d2buf + (size_t)sl * WP * DV;
      constexpr int NG = WP * (DV / 8) / 256;
      static_assert(WP * (DV / 8) % 256 == 0, "whole passes");
      bf16x8 t8[NG];
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int e = fresh(tid) + 256 * u;
        t8[u] = *reinterpret_cast<const bf16x8*>(d2b + (size_t)(e / (DV / 8)) * DV + (e % (DV / 8)) * 8);
      }
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int e = fresh(tid) + 256 * u;
        *reinterpret_cast<bf16x8*>(D2 + (e / (DV / 8)) * LV + (e % (DV / 8)) * 8) = t8[u];
      }
    }
    __syncthreads();

    // ---- D1 = (D2 W2_p) .* gelu'(Z)  [rows R0.. x 16 units], K = DV -> D1T [16][LT]
    {
      f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
      for (int s = 0; s < DV / 32; ++s) {
        const bf16x8 bw = ld_nat(W2i, LV, 0, 32 * s, lane);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt] = mma(ld_nat(D2, LV, R0 + 16 * mt, 32 * s, lane), bw, acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) D1T[c16 * LT + R0 + 16 * mt + 4 * g + r] = (bf16)(acc[mt][r] * GP[mt][r]);
    }
    __syncthreads();

    // ---- retrieval, layer 1: Zq = A_q Xq W1^T + B_q Xq S1^T - Q1 D1  [query rows Q0.. x 16 units]
    // (the first two terms were formed during the first barrier)
    {
      const f32x4 a1 = ra1, a2 = ra2;
      f32x4 a3 = zero4();
#pragma unroll
      for (int s = 0; s < WP / 32; ++s) {
        const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(Q1g + (Q0 + c16) * WP + 32 * s + 8 * g);
        a3 = mma(q1, ld_nat(D1T, LT, 0, 32 * s, lane), a3);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = Q0 + 4 * g + r;
        Ah[qq * LU + c16] = (bf16)gelu(cA[qq] * a1[r] + cB[qq] * a2[r] - a3[r]);
      }
    }
    __syncthreads();

    // ---- Q2 = C .* (Ah A^T)  [query rows Q0.. x WP], K = 16 units (this wave's rows only)
    {
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(Ah + (Q0 + c16) * LU + 4 * g);
#pragma unroll
      for (int nt = 0; nt < WP / 16; ++nt) {
        const f32x4 acc = mma16(a, *reinterpret_cast<const bf16x4*>(Al + (16 * nt + c16) * LU + 4 * g), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = Q0 + 4 * g + r, w = 16 * nt + c16;
          Q2[qq * LT + w] = (bf16)(Cl[qq * WP + w] * acc[r]);
        }
      }
    }

    // ---- retrieval, layer 2 partial: A_q Ah W2^T + B_q Ah S2^T - Q2 D2  [Q0.. x DV]
    {
      // transposed (value rows x queries): lane holds four adjacent values of
      // query Q0 + (l & 15), one 16-byte store per tile
      const int yo = ((sl * G + pm) * BC) * DV * 4;
      const bf16x4 ah = *reinterpret_cast<const bf16x4*>(Ah + (Q0 + c16) * LU + 4 * g);
      bf16x8 q2f[WP / 32];
#pragma unroll
      for (int s = 0; s < WP / 32; ++s) q2f[s] = ld_nat(Q2, LT, Q0, 32 * s, lane);
      const int qq = Q0 + c16;
      const float ca = cA[qq], cb = cB[qq];
#pragma unroll
      for (int nt = 0; nt < DV / 16; ++nt) {
        const f32x4 b1 = mma16(ld_tr16(W2i, LV, 16 * nt, 0, lane), ah, zero4());
        const f32x4 b2 = mom ? mma16(ld_tr16(S2i, LV, 16 * nt, 0, lane), ah, zero4()) : zero4();
        f32x4 b3 = zero4();
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) b3 = mma(ld_tr_nat(D2, LV, 16 * nt, 32 * s, lane), q2f[s], b3);
        f32x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = ca * b1[r] + cb * b2[r] - b3[r];
        buf_store4(y, rxo, yo + (qq * DV + 16 * nt + 4 * g) * 4, 0);
      }
    }

    // ---- state update at the chunk end (registers)
    {
      const int ce = te - t0;
      const float Ate = cA[ce], Bte = cB[ce], Pc = cP[0];
      // W1 [16 units x features fb..]: (cM .* D1)^T X, K = WP window rows
      bf16x8 bm[WP / 32], bs[WP / 32];
#pragma unroll
      for (int s = 0; s < WP / 32; ++s) {
        bm[s] = ld_nat_scaled(D1T, LT, 0, 32 * s, lane, cM);
        bs[s] = ld_nat_scaled(D1T, LT, 0, 32 * s, lane, cS);
      }
      // X^T fragments of tile t + 1 are loaded before tile t computes
      bf16x8 xf[2][WP / 32];
      auto load = [&](int t, bf16x8* dst) {
        const int f = fb + 16 * t + c16;
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) dst[s] = gload8(rxt, (f * (int)NR + t0 + 32 * s + 8 * g) * 2);
      };
      load(0, xf[0]);
#pragma unroll
      for (int t = 0; t < NFW; ++t) {
        if (t + 1 < NFW) load(t + 1, xf[(t + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 um = zero4(), us = zero4();
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) {
          um = mma(bm[s], xf[t & 1][s], um);
          if (mom) us = mma(bs[s], xf[t & 1][s], us);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w1 = W1T[t][r], s1 = S1T[t][r];
          W1T[t][r] = Ate * w1 + Bte * s1 - um[r];
          S1T[t][r] = Pc * s1 - us[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // W2 [value rows x 16 units]: (cM .* D2)^T A, K = WP
#pragma unroll
      for (int t = 0; t < NDW; ++t) {
        f32x4 um = zero4(), us = zero4();
        const int o0 = 16 * (NDW * wave + t);
#pragma unroll
        for (int s = 0; s < WP / 32; ++s) {
          const bf16x8 d2 = ld_tr_nat(D2, LV, o0, 32 * s, lane);
          const bf16x8 at = ld_nat(AT, LT, 0, 32 * s, lane);
          um = mma(scaled_k(d2, cM + 32 * s + 8 * g), at, um);
          if (mom) us = mma(scaled_k(d2, cS + 32 * s + 8 * g), at, us);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w2 = W2T[t][r], s2 = S2T[t][r];
          W2T[t][r] = Ate * w2 + Bte * s2 - um[r];
          S2T[t][r] = Pc * s2 - us[r];
        }
      }
    }
    __syncthreads();   // every wave is done with this chunk's images
    write_images();
  }

  // ---- last chunk's outputs, then the state back to memory
  group_barrier(ctr, G * (++nbar), err);
  if (nch > 0) reduce_out(nch - 1);
  {
    const __amdgpu_buffer_rsrc_t rw = buffer_of(Wt, (unsigned)(((size_t)H * D + (size_t)DV * H) * 4));
    const __amdgpu_buffer_rsrc_t rm = buffer_of(Mo, mom ? (unsigned)(((size_t)H * D + (size_t)DV * H) * 4) : 0u);
#pragma unroll
    for (int t = 0; t < NFW; ++t) {
      const int f = fb + 16 * t + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = f < D ? ((j0 + 4 * g + r) * D + f) * 4 : kZeroOffset;
        gstore1(W1T[t][r], rw, off);
        gstore1(S1T[t][r], rm, off);
      }
    }
#pragma unroll
    for (int t = 0; t < NDW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = (H * D + (16 * (NDW * wave + t) + 4 * g + r) * H + j0 + c16) * 4;
        gstore1(W2T[t][r], rw, off);
        gstore1(S2T[t][r], rm, off);
      }
  }
  // halo and count: member 0, after every member has read the old halo (the
  // barrier above orders it after every member's last chunk)
  if (pm == 0 && tid < 64) {
    for (int j = 0; j < c - 1; ++j) {
      const int i = N - (c - 1) + j;
      for (int d = lane; d < DK; d += 64) hk[j * DK + d] = i >= 0 ? (float)k[(size_t)i * DK + d] : hk[(N + j) * DK + d];
      for (int o = lane; o < DV; o += 64) hv[j * DV + o] = i >= 0 ? (float)v[(size_t)i * DV + o] : hv[(N + j) * DV + o];
      if (lane == 0) hg[j] = i >= 0 ? gam_in[i] : hg[N + j];
    }
    if (lane == 0) *cnt += N;
  }
}

}  // namespace grouped

template <int PHI, int DK, int PD, int DV, int H, int G>
hipError_t launch_grouped(const GroupedParams& gp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1) {
  typedef grouped::GShape<PHI, DK, PD, DV, H, G> S;
  if (gp.N == 0 || gp.n_seq == 0) return hipSuccess;
  hipLaunchKernelGGL((coeff_kernel<S::BC, S::WP>), dim3((unsigned)kp.nchunks * (unsigned)gp.n_seq), dim3(256), 0,
                     stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool attr_set = false;
  if (!attr_set) {
    // allow more than the default dynamic LDS; a refusal shows up at launch
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped::grouped_kernel<S>),
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
  const unsigned groups8 = (unsigned)((gp.n_seq + 7) / 8);
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((grouped::grouped_kernel<S>), dim3(groups8 * 8u * G), dim3(256), S::lds, stream, gp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int PHI, int DK, int PD, int DV, int H, int G>
size_t grouped_seq_bytes(int nchunks) { return grouped::GShape<PHI, DK, PD, DV, H, G>::seq_bytes(nchunks); }

#define ATLAS_GROUPED(NAME, PHI, DK, PD, DV, H, G)                                                             \
  template hipError_t launch_grouped<PHI, DK, PD, DV, H, G>(const GroupedParams&, const CoeffParams&, hipStream_t, \
                                                            hipEvent_t, hipEvent_t);                           \
  template size_t grouped_seq_bytes<PHI, DK, PD, DV, H, G>(int);
#define ATLAS_LINEAR(NAME, PHI, DK, PD, DV, WP)
#include "atlas_mem_grouped_variants.inc"
#undef ATLAS_GROUPED
#undef ATLAS_LINEAR

}  // namespace atlas
