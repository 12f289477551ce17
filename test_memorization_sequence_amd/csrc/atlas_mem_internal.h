// atlas_mem_internal.h -- shapes, workspace layout and launch parameters
// shared by the kernels and the C ABI implementation of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace atlas {

typedef __bf16 bf16;

enum { MEM_LINEAR = 0, MEM_MLP = 1 };
enum { PHI_IDENTITY = 0, PHI_POLY2 = 1, PHI_RAW_POLY2 = 2 };
enum { BIAS_L2 = 0, BIAS_DOT = 1, BIAS_LP = 2, BIAS_HUBER = 3 };

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// sets the message of atlas_mem_last_hip_error (defined with the C ABI)
void record_hip_error(const char* what);

constexpr int feature_dim(int phi, int dk, int pd) {
  return phi == PHI_IDENTITY ? dk
       : phi == PHI_POLY2    ? dk + dk * (dk + 1) / 2
                             : dk + pd + pd * (pd + 1) / 2;
}

// Per-sequence workspace of the chunk kernel (operand images of the state and
// the per-chunk intermediates), byte offsets.
template <class S>
struct WsLayout {
  typedef typename S::T T;
  static constexpr bool MLP = S::MEM == MEM_MLP;
  static constexpr size_t e = sizeof(T);
  static constexpr size_t WP = S::WP, DP = S::DP, BC = S::BC, DV = S::DV, H = S::H;
  static constexpr size_t Xw = 0;
  static constexpr size_t XwT = align_up(Xw + WP * DP * e, 256);
  static constexpr size_t Xq = align_up(XwT + DP * WP * e, 256);
  static constexpr size_t Q1 = align_up(Xq + BC * DP * e, 256);
  static constexpr size_t Q2 = align_up(Q1 + BC * WP * e, 256);
  static constexpr size_t W1b = align_up(Q2 + BC * WP * e, 256);
  static constexpr size_t S1b = align_up(W1b + (MLP ? H * DP : 0) * e, 256);
  static constexpr size_t W2b = align_up(S1b + (MLP ? H * DP : 0) * e, 256);
  static constexpr size_t S2b = align_up(W2b + (MLP ? DV * H : DV * DP) * e, 256);
  static constexpr size_t W2T = align_up(S2b + (MLP ? DV * H : DV * DP) * e, 256);
  static constexpr size_t Zf = align_up(W2T + (MLP ? H * DV : 0) * e, 256);
  static constexpr size_t Ab = align_up(Zf + (MLP ? WP * H * 4 : 0), 256);
  static constexpr size_t AT = align_up(Ab + (MLP ? WP * H : 0) * e, 256);
  static constexpr size_t D2 = align_up(AT + (MLP ? H * WP : 0) * e, 256);
  static constexpr size_t D2T = align_up(D2 + WP * DV * e, 256);
  static constexpr size_t D2TM = align_up(D2T + DV * WP * e, 256);
  static constexpr size_t D2TS = align_up(D2TM + DV * WP * e, 256);
  static constexpr size_t D1T = align_up(D2TS + DV * WP * e, 256);
  static constexpr size_t D1TM = align_up(D1T + (MLP ? H * WP : 0) * e, 256);
  static constexpr size_t D1TS = align_up(D1TM + (MLP ? H * WP : 0) * e, 256);
  static constexpr size_t Ah = align_up(D1TS + (MLP ? H * WP : 0) * e, 256);
  // rows that need whole-row statistics (fp32 [WP][DV]): raw errors for the
  // l_p / Huber biases, the pre-norm branch u with the layer norm; En keeps
  // the normalised branch for the LN backward
  static constexpr size_t Ef = align_up(Ah + (MLP ? BC * H : 0) * e, 256);
  static constexpr size_t En = align_up(Ef + WP * DV * 4, 256);
  // gated memory: images of W3, S3, the pre-activation X W3^T, and D3 in the
  // layouts of D1
  static constexpr size_t W3b = align_up(En + (MLP ? WP * DV * 4 : 0), 256);
  static constexpr size_t S3b = align_up(W3b + (MLP ? H * DP : 0) * e, 256);
  static constexpr size_t Z3f = align_up(S3b + (MLP ? H * DP : 0) * e, 256);
  static constexpr size_t D3T = align_up(Z3f + (MLP ? WP * H * 4 : 0), 256);
  static constexpr size_t D3TM = align_up(D3T + (MLP ? H * WP : 0) * e, 256);
  static constexpr size_t D3TS = align_up(D3TM + (MLP ? H * WP : 0) * e, 256);
  static constexpr size_t bytes = align_up(D3TS + (MLP ? H * WP : 0) * e, 256);
};

// Muon (per-sequence kernel): Newton-Schulz runs on the orientation of a
// rows x cols weight matrix with fewer rows, r x n (r <= n), both padded to
// multiples of 32 with zeros, which the iteration keeps zero.
constexpr long ns_r(long rows, long cols) { return ((rows > cols ? cols : rows) + 31) / 32 * 32; }
constexpr long ns_n(long rows, long cols) { return ((rows > cols ? rows : cols) + 31) / 32 * 32; }
constexpr long lmax(long a, long b) { return a > b ? a : b; }

// Muon workspace of one workgroup (fp32, byte offsets): the momentum of a
// call without momentum in the state (P floats), the running window gradient
// (P floats), two ping-pong iterates X and their transposes (r x n each, the
// largest matrix of the memory), the r x r products A = X X^T and
// B = b A + c A A, and (MLP) the hidden activations gelu(W1_t phi(q_t)) of
// the chunk's tokens [chunk][h], which the W1 workgroup of a pair hands to the
// W2 workgroup.
struct MuonWs {
  size_t sloc, g, x0, x1, xt0, xt1, am, bm, ab, bytes;
};
constexpr MuonWs muon_ws(long P, long rn, long rr, long nab) {
  const size_t g = align_up((size_t)P * 4, 256);
  const size_t x0 = align_up(g + (size_t)P * 4, 256);
  const size_t x1 = align_up(x0 + (size_t)rn * 4, 256);
  const size_t xt0 = align_up(x1 + (size_t)rn * 4, 256);
  const size_t xt1 = align_up(xt0 + (size_t)rn * 4, 256);
  const size_t am = align_up(xt1 + (size_t)rn * 4, 256);
  const size_t bm = align_up(am + (size_t)rr * 4, 256);
  const size_t ab = align_up(bm + (size_t)rr * 4, 256);
  return MuonWs{0, g, x0, x1, xt0, xt1, am, bm, ab, align_up(ab + (size_t)nab * 4, 256)};
}
// linear memory: M [dv][D]; MLP: W1 [h][D], W2 [dv][h]; bc the chunk
constexpr MuonWs muon_ws_of(bool mlp, long D, long dv, long h, long bc) {
  return mlp ? muon_ws(h * D + dv * h, lmax(ns_r(h, D) * ns_n(h, D), ns_r(dv, h) * ns_n(dv, h)),
                       lmax(ns_r(h, D) * ns_r(h, D), ns_r(dv, h) * ns_r(dv, h)), bc * h)
             : muon_ws(dv * D, ns_r(dv, D) * ns_n(dv, D), ns_r(dv, D) * ns_r(dv, D), 0);
}

// T: MFMA operand type (bf16 or float); TI: io type of q, k, v, out.
// H = 0 for a linear memory.  WP: window rows (chunk + c - 1) padded to 32.
// PD: degree-2 map width (== DK for PHI_POLY2).
template <typename T_, typename TI_, int MEM_, int PHI_, int DK_, int DV_, int H_, int BC_, int WP_, int PD_>
struct Shape {
  typedef T_ T;
  typedef TI_ TI;
  static constexpr int MEM = MEM_, PHI = PHI_, DK = DK_, DV = DV_, H = H_, BC = BC_, WP = WP_, PD = PD_;
  static constexpr int D = feature_dim(PHI_, DK_, PD_);
  static constexpr int DP = (D + 31) / 32 * 32;
  typedef WsLayout<Shape> WS;
  static_assert(WP % 32 == 0 && BC % 32 == 0 && DV % 32 == 0 && H % 32 == 0, "MFMA tile multiples");
  static_assert(BC <= 64, "coefficient kernel handles chunks up to 64");
};

// Coefficient block of one chunk (floats):
//   [0, BC)            A_t           [BC, 2BC)  B_t        [2BC] P (+3 pad)
//   [2BC+4, +WP)       cM_i = C_{te,i}
//   [2BC+4+WP, +WP)    cS_i
//   [2BC+4+2WP, +BC*WP) C_{t,i} row-major
//   with a precomputed Q1 (sharded and streamed kernels, identity feature
//   map) the block continues with Q1 = C .* (Xq X^T) as bf16 [BC][pitch]
//   (pitch WP; WP + 4 for the streamed kernel, its LDS pitch, so that the
//   block is the LDS image), and for the streamed kernel then with C itself
//   as bf16 [BC][WP].
constexpr int q1_pitch(int wp, bool cb16) { return cb16 ? wp + 4 : wp; }
constexpr int coef_stride(int bc, int wp, bool q1 = false, bool cb16 = false) {
  return 2 * bc + 4 + 2 * wp + bc * wp + (q1 ? bc * q1_pitch(wp, cb16) / 2 : 0) + (cb16 ? bc * wp / 2 : 0);
}

struct CoeffParams {
  const float* alpha;
  const float* eta;
  const float* theta;
  const char* state;
  float* coef;
  unsigned* ctrl;   // groups: [0] error word, [1 + s] barrier counter and [1 + n + s] XCD mask of sequence s (n sequences); else null
  const void* q;    // Q1 precompute (sharded kernel): bf16 queries and keys [seq][N][d]
  const void* k;
  size_t off_halo_k;
  int N, c, nchunks, coef_stride, momentum;
  size_t seq_stride, off_count;
};

struct ChunkParams {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  char* state;
  void* out;
  char* ws;
  const float* coef;
  int N, c, nchunks, coef_stride;
  size_t seq_stride, off_weights, off_momentum, off_halo_k, off_halo_v, off_halo_g, off_count;
  float grad_scale;
  int momentum, bias, residual;
  // l_p exponent; Huber thresholds of the call [n_seq][N] (else null) and the
  // state offset of the thresholds of the halo
  float bias_p, sign_alpha;
  const float* delta;
  size_t off_halo_d;
  int layernorm;   // MLP: f = r + LN(W2 gelu(W1 x)), no gain or shift
  float ln_eps;
  int gated;       // MLP: f = r + W2 (gelu(W1 x) .* (W3 x)) (per-sequence kernel)
  // Muon: raw gates per token, Newton-Schulz steps, workspace (MuonWs per
  // workgroup, mws_stride bytes apart); muon == 0 for gradient descent.
  // group = 2 (MLP memory): a pair of workgroups of one XCD per sequence,
  // one per weight matrix, synchronised through ctrl ([0] error word,
  // [1 + s] counter of sequence s, reset by the coefficient kernel); the
  // chunk workspace (ws) is then per workgroup as well.
  const float* alpha;
  const float* eta;
  const float* theta;
  int muon, ns_steps;
  char* mws;
  size_t mws_stride;
  unsigned* ctrl;
  int n_seq, group;
};

struct ShardedParams {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  char* state;
  void* out;
  char* xws;        // exchange workspace, per sequence
  unsigned* ctrl;   // [0] error word, [1 + s] barrier counter of sequence s
  const float* coef;
  int n_seq, N, c, nchunks, coef_stride;
  size_t seq_stride, off_weights, off_momentum, off_halo_k, off_halo_v, off_halo_g, off_count;
  float grad_scale;
  int momentum, bias, residual;
  // l_p exponent; Huber thresholds of the call [n_seq][N] (else null) and the
  // state offset of the thresholds of the halo
  float bias_p, sign_alpha;
  const float* delta;
  size_t off_halo_d;
  int layernorm;   // MLP: f = r + LN(W2 gelu(W1 x)), no gain or shift
  float ln_eps;
  int gated;       // MLP: f = r + W2 (gelu(W1 x) .* (W3 x)) (per-sequence kernel)
};

// Grouped MLP kernel family (wide feature maps): G workgroups of one XCD per
// sequence, 16 hidden units each; phi of every key and query precomputed per
// call into the workspace (gws, gseq_bytes per sequence).
struct GroupedParams {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  char* state;
  void* out;
  char* gws;        // per sequence: exchange buffers, then the phi buffers
  size_t gseq_bytes;
  unsigned* ctrl;   // [0] error word, [1 + s] barrier counter of sequence s
  float* coef;      // the Q1 kernel writes Q1 into the coefficient blocks
  int n_seq, N, c, nchunks, coef_stride;
  size_t seq_stride, off_weights, off_momentum, off_halo_k, off_halo_v, off_halo_g, off_count;
  float grad_scale;
  int momentum, bias, residual;
};

template <int PHI, int DK, int PD, int DV, int H, int G>
hipError_t launch_grouped(const GroupedParams& gp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1);
template <int PHI, int DK, int PD, int DV, int H, int G>
size_t grouped_seq_bytes(int nchunks);

template <int D, int DV, int H, int G, int WP, int BC>
hipError_t launch_sharded(const ShardedParams& sp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1);
template <int D, int DV, int H, int G, int WP, int BC>
size_t sharded_xbytes();
// Streamed-state MLP kernel (G workgroups per sequence; for G = 1 xws and
// ctrl are unused).
template <int D, int DV, int H, int WP, int BC, int G>
hipError_t launch_streamed(const ShardedParams& sp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1);
template <int D, int DV, int H, int WP, int BC, int G>
size_t streamed_xbytes();

// Enqueues the coefficient kernel, then the chunk kernel; ev0/ev1 (optional)
// are recorded right before and right after the chunk kernel.
template <class S>
hipError_t launch(const ChunkParams& cp, const CoeffParams& kp, int n_seq, hipStream_t stream,
                  hipEvent_t ev0, hipEvent_t ev1);

}  // namespace atlas
