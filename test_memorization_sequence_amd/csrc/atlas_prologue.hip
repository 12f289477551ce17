// atlas_prologue.hip -- the fused prologue (include/atlas_prologue.h).  By
// default one kernel (atlas_prologue_gemm.hip) computes the projections tile
// by tile and applies the rest of each token's work to the tile in LDS.  The
// two-kernel path below -- the projection GEMM into a workspace, then
// prologue_kernel -- serves the shapes the fused kernel does not and gives
// the same bits.
//
// Kernel layout: one wave per (run of TOK consecutive tokens of one sequence,
// head), head fastest, so the waves of a workgroup share the tokens'
// projection rows (their gate columns) in cache.  Lane l owns DPL = d / 64
// adjacent channels of the head in each of q, k, v and keeps their conv taps
// and the last K-1 projection rows in registers while it walks the run: each
// projection value is loaded once.  SiLU follows the causal depthwise
// convolution, and the L2 norm of q and k is a wave reduction.  The gate
// projections V_g (U_g x) run on 4 r lanes: lane g*r + j multiplies the
// token's j-th U_g output by V_g[h][j]; a reduction over r lanes and a
// sigmoid give the gate.  HBM-bound: P is read once, q, k, v and the gates
// are written once.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <new>

#include "atlas_prologue.h"
#include "atlas_mem_internal.h"
#include "atlas_mem_frag.h"
#include "atlas_prologue_gemm.h"
#include "atlas_prologue_math.h"

namespace atlas {
namespace prologue {

using mfma::buffer_of;
using mfma::kZeroOffset;

struct Params {
  const bf16* P;       // [B*N][ncol] projections
  const float* w_conv; // [3*H*d][K]
  const float* gv;     // [4][H][r]
  const float* gb;     // [4][H]
  bf16* q;
  bf16* k;
  bf16* v;
  float* gate[4];
  int B, N, H, K, r, ncol;
};

constexpr int TOK = 32;   // tokens per wave
constexpr int TB = 8;     // tokens per load batch
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D, int K>
__global__ void __launch_bounds__(256) prologue_kernel(Params p) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int tiles = (p.N + TOK - 1) / TOK;
  // wave-uniform (scalar registers): the row descriptors below need it
  const long item = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const long items = (long)p.B * tiles * p.H;
  if (item >= items) return;
  const int h = (int)(item % p.H);
  const long bt = item / p.H;
  const int tile = (int)(bt % tiles);
  const long b = bt / tiles;
  const int n0 = tile * TOK, n1 = min(p.N, n0 + TOK);
  const int HD = p.H * D;
  bf16* outs[3] = {p.q, p.k, p.v};
  // taps and the sliding window (oldest first) of this lane's channels
  float tap[3][DPL][K], win[3][DPL][K];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int ch = m * HD + h * D + lane * DPL + i;
#pragma unroll
      for (int j = 0; j < K; ++j) tap[m][i][j] = p.w_conv[(size_t)ch * K + j];
#pragma unroll
      for (int j = 0; j + 1 < K; ++j) {
        const int src = n0 - (K - 1) + j;
        // a ring when K divides the batch (token n in slot n mod K; n0 is a
        // multiple of TB), else oldest first
        win[m][i][TB % K == 0 ? (j + 1) % K : j] = src >= 0 ? (float)p.P[(size_t)(b * p.N + src) * p.ncol + ch] : 0.f;
      }
    }
  const int g = lane / p.r, jj = lane - g * p.r;
  const float gvv = g < 4 ? p.gv[(g * p.H + h) * p.r + jj] : 0.f;
  const float gbb = g < 4 ? p.gb[g * p.H + h] : 0.f;
  // Tokens in batches of TB: every projection value of the batch is loaded
  // first (rows past the run re-read its last row and are not stored), so
  // one memory latency covers TB tokens; then the batch is computed in order.
  // the batch's rows through one descriptor (base and token offsets in
  // scalar registers, this lane's column offsets fixed for the run); gate
  // columns past the 4 r the ranks use read zero
  const int voff_m = (h * D + lane * DPL) * 2;
  const int voff_g = g < 4 ? (3 * HD + lane) * 2 : kZeroOffset;
  for (int nb = n0; nb < n1; nb += TB) {
    float x[TB][3][DPL], xg[TB], gq[TB];
    const int nlast = n1 - 1 - nb;
    const __amdgpu_buffer_rsrc_t rp = buffer_of(p.P + (size_t)(b * p.N + nb) * p.ncol, (unsigned)(TB * p.ncol * 2));
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int soff = min(t, nlast) * p.ncol * 2;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        if constexpr (DPL == 1) {
          x[t][m][0] = (float)__builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rp, voff_m + m * HD * 2, soff, 0));
        } else if constexpr (DPL == 2) {
          const bf16x2 v2 = __builtin_bit_cast(bf16x2, __builtin_amdgcn_raw_buffer_load_b32(rp, voff_m + m * HD * 2, soff, 0));
          x[t][m][0] = (float)v2[0];
          x[t][m][1] = (float)v2[1];
        } else {
          static_assert(DPL % 4 == 0, "channels per lane");
#pragma unroll
          for (int i = 0; i < DPL; i += 4) {
            const bf16x4 v4 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rp, voff_m + (m * HD + i) * 2, soff, 0));
#pragma unroll
            for (int z = 0; z < 4; ++z) x[t][m][i + z] = (float)v4[z];
          }
        }
      }
      xg[t] = (float)__builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rp, voff_g, soff, 0));
    }
    bf16* ob[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) ob[m] = outs[m] + ((size_t)(b * p.H + h) * p.N + nb) * D + lane * DPL;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int n = nb + t;
      if (n >= n1) break;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float acc[DPL];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float a = 0.f;
          if constexpr (TB % K == 0) {
            win[m][i][t % K] = x[t][m][i];
#pragma unroll
            for (int j = 0; j < K; ++j) a = fmaf(tap[m][i][j], win[m][i][(t + 1 + j) % K], a);
          } else {
            win[m][i][K - 1] = x[t][m][i];
#pragma unroll
            for (int j = 0; j < K; ++j) a = fmaf(tap[m][i][j], win[m][i][j], a);
#pragma unroll
            for (int j = 0; j + 1 < K; ++j) win[m][i][j] = win[m][i][j + 1];
          }
          acc[i] = silu(a);
          ss = fmaf(acc[i], acc[i], ss);
        }
        float scale = 1.f;
        if (m < 2) {
          ss = wave_sum(ss);
          scale = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(|x|, 1e-12)
        }
        bf16* o = ob[m] + t * D;
        if constexpr (DPL == 2) {
          *reinterpret_cast<bf16x2*>(o) = bf16x2{(bf16)(acc[0] * scale), (bf16)(acc[1] * scale)};
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[i] = (bf16)(acc[i] * scale);
        }
      }
      float u = xg[t] * gvv;
      u = group_sum(u, p.r);   // within aligned groups of r lanes
      gq[t] = sigm(u + gbb);
    }
    // the batch's gates: lane g r of each of the four groups writes TB
    // consecutive values of its gate (32 bytes) rather than one per token
    if (g < 4 && jj == 0) {
      float* dst = p.gate[g] + (size_t)(b * p.H + h) * p.N + nb;
      if (n1 - nb >= TB && ((uintptr_t)dst & 15) == 0) {
#pragma unroll
        for (int t = 0; t < TB; t += 4)
          *reinterpret_cast<float4*>(dst + t) = make_float4(gq[t], gq[t + 1], gq[t + 2], gq[t + 3]);
      } else {
#pragma unroll
        for (int t = 0; t < TB; ++t)
          if (nb + t < n1) dst[t] = gq[t];
      }
    }
  }
}

template <int D>
void launch_d(const Params& p, int K, unsigned blocks, hipStream_t st) {
  switch (K) {
    case 1: hipLaunchKernelGGL((prologue_kernel<D, 1>), dim3(blocks), dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((prologue_kernel<D, 2>), dim3(blocks), dim3(256), 0, st, p); break;
    case 3: hipLaunchKernelGGL((prologue_kernel<D, 3>), dim3(blocks), dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((prologue_kernel<D, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    case 5: hipLaunchKernelGGL((prologue_kernel<D, 5>), dim3(blocks), dim3(256), 0, st, p); break;
    case 6: hipLaunchKernelGGL((prologue_kernel<D, 6>), dim3(blocks), dim3(256), 0, st, p); break;
    case 7: hipLaunchKernelGGL((prologue_kernel<D, 7>), dim3(blocks), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((prologue_kernel<D, 8>), dim3(blocks), dim3(256), 0, st, p); break;
  }
}

}  // namespace prologue
}  // namespace atlas

struct atlas_prologue_s {
  uint32_t magic;
  atlas_prologue_config cfg;
  int device;
  atlas::bf16* P;   // projections of the two-kernel path (null until needed)
  int fused;        // the one-kernel path serves this shape and is selected
  hipEvent_t ev_gemm, ev_before, ev_after;
};

static bool fused_ok(const atlas_prologue_config& c) {
  return atlas::prologue::fused_supported(c.d_head, c.heads, c.gate_rank, c.seq_len, c.d_model);
}

static const uint32_t kProMagic = 0xA7A5F10Bu;

static atlas_status check(const atlas_prologue_config* c) {
  if (!c || c->batch < 1 || c->seq_len < 0 || c->d_model < 8 || c->d_model % 8 || c->heads < 1 || c->d_head < 1 ||
      c->conv_taps < 1 || c->gate_rank < 1)
    return ATLAS_ERR_INVALID_ARGUMENT;
  if (c->d_head != 64 && c->d_head != 128 && c->d_head != 256) return ATLAS_ERR_UNSUPPORTED;
  if (c->conv_taps > 8) return ATLAS_ERR_UNSUPPORTED;
  if (c->gate_rank != 1 && c->gate_rank != 2 && c->gate_rank != 4 && c->gate_rank != 8 && c->gate_rank != 16)
    return ATLAS_ERR_UNSUPPORTED;
  const long rows = (long)c->batch * c->seq_len, ncol = 3L * c->heads * c->d_head + 4L * c->gate_rank;
  if (rows > 0x7fffffffL || ncol > 0x7fffffffL || rows * c->heads > (1L << 40)) return ATLAS_ERR_INVALID_ARGUMENT;
  return ATLAS_OK;
}

extern "C" {

atlas_status atlas_prologue_init(const atlas_prologue_config* cfg, atlas_prologue_t* out) {
  if (!out) return ATLAS_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  atlas_status s = check(cfg);
  if (s != ATLAS_OK) return s;
  atlas_prologue_s* h = new (std::nothrow) atlas_prologue_s();
  if (!h) return ATLAS_ERR_OUT_OF_MEMORY;
  h->magic = kProMagic;
  h->cfg = *cfg;
  h->P = nullptr;
  h->ev_gemm = h->ev_before = h->ev_after = nullptr;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    atlas::record_hip_error(hipGetErrorString(e));
    delete h;
    return ATLAS_ERR_HIP;
  }
  h->fused = fused_ok(*cfg) ? 1 : 0;
  const size_t rows = (size_t)cfg->batch * cfg->seq_len;
  const size_t ncol = 3 * (size_t)cfg->heads * cfg->d_head + 4 * (size_t)cfg->gate_rank;
  if (!h->fused && rows && hipMalloc(&h->P, rows * ncol * sizeof(atlas::bf16)) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return ATLAS_ERR_OUT_OF_MEMORY;
  }
  *out = h;
  return ATLAS_OK;
}

atlas_status atlas_prologue_forward(atlas_prologue_t h, const void* x, const void* w, const float* w_conv,
                                    const float* gate_v, const float* gate_b, void* q, void* k, void* v,
                                    float* alpha, float* eta, float* theta, float* gamma, void* stream) {
  if (!h || h->magic != kProMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  const atlas_prologue_config& c = h->cfg;
  if (c.seq_len == 0) return ATLAS_OK;
  const void* p16[] = {x, w, q, k, v};
  for (const void* p : p16)
    if (!p || (uintptr_t)p % 16) return ATLAS_ERR_INVALID_ARGUMENT;
  const void* p4[] = {w_conv, gate_v, gate_b, alpha, eta, theta, gamma};
  for (const void* p : p4)
    if (!p || (uintptr_t)p % 4) return ATLAS_ERR_INVALID_ARGUMENT;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev != h->device) return e != hipSuccess ? (atlas::record_hip_error(hipGetErrorString(e)), ATLAS_ERR_HIP)
                                                                  : ATLAS_ERR_INVALID_ARGUMENT;
  hipStream_t st = (hipStream_t)stream;
  const int rows = c.batch * c.seq_len;
  const int ncol = 3 * c.heads * c.d_head + 4 * c.gate_rank;
  if (h->ev_gemm && (e = hipEventRecord(h->ev_gemm, st)) != hipSuccess) {
    atlas::record_hip_error(hipGetErrorString(e));
    return ATLAS_ERR_HIP;
  }
  if (h->fused) {
    atlas::prologue::FusedParams f{};
    f.x = (const atlas::bf16*)x;
    f.w = (const atlas::bf16*)w;
    f.w_conv = w_conv;
    f.gv = gate_v;
    f.gb = gate_b;
    f.q = (atlas::bf16*)q;
    f.k = (atlas::bf16*)k;
    f.v = (atlas::bf16*)v;
    f.gate[0] = alpha;
    f.gate[1] = eta;
    f.gate[2] = theta;
    f.gate[3] = gamma;
    f.B = c.batch;
    f.N = c.seq_len;
    f.dm = c.d_model;
    f.H = c.heads;
    f.K = c.conv_taps;
    f.r = c.gate_rank;
    f.ncol = ncol;
    if ((h->ev_before && (e = hipEventRecord(h->ev_before, st)) != hipSuccess) ||
        (e = atlas::prologue::fused_prologue(f, c.d_head, st)) != hipSuccess ||
        (h->ev_after && (e = hipEventRecord(h->ev_after, st)) != hipSuccess)) {
      atlas::record_hip_error(hipGetErrorString(e));
      return ATLAS_ERR_HIP;
    }
    return ATLAS_OK;
  }
  // P [rows][ncol] = x [rows][d_model] . W^T, W [ncol][d_model]
  if ((e = atlas::prologue::gemm_nt_bf16((const atlas::bf16*)x, (const atlas::bf16*)w, h->P, rows, ncol, c.d_model, st)) !=
      hipSuccess) {
    atlas::record_hip_error(hipGetErrorString(e));
    return ATLAS_ERR_HIP;
  }
  atlas::prologue::Params p;
  p.P = h->P;
  p.w_conv = w_conv;
  p.gv = gate_v;
  p.gb = gate_b;
  p.q = (atlas::bf16*)q;
  p.k = (atlas::bf16*)k;
  p.v = (atlas::bf16*)v;
  p.gate[0] = alpha;
  p.gate[1] = eta;
  p.gate[2] = theta;
  p.gate[3] = gamma;
  p.B = c.batch;
  p.N = c.seq_len;
  p.H = c.heads;
  p.K = c.conv_taps;
  p.r = c.gate_rank;
  p.ncol = ncol;
  const long tiles = (c.seq_len + atlas::prologue::TOK - 1) / atlas::prologue::TOK;
  const long items = (long)c.batch * tiles * c.heads;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  if (h->ev_before && (e = hipEventRecord(h->ev_before, st)) != hipSuccess) {
    atlas::record_hip_error(hipGetErrorString(e));
    return ATLAS_ERR_HIP;
  }
  switch (c.d_head) {
    case 64: atlas::prologue::launch_d<64>(p, c.conv_taps, blocks, st); break;
    case 128: atlas::prologue::launch_d<128>(p, c.conv_taps, blocks, st); break;
    default: atlas::prologue::launch_d<256>(p, c.conv_taps, blocks, st); break;
  }
  if ((e = hipGetLastError()) != hipSuccess ||
      (h->ev_after && (e = hipEventRecord(h->ev_after, st)) != hipSuccess)) {
    atlas::record_hip_error(hipGetErrorString(e));
    return ATLAS_ERR_HIP;
  }
  return ATLAS_OK;
}

atlas_status atlas_prologue_set_fused(atlas_prologue_t h, int fused) {
  if (!h || h->magic != kProMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  if (fused) {
    if (!fused_ok(h->cfg)) return ATLAS_ERR_UNSUPPORTED;
    h->fused = 1;
    return ATLAS_OK;
  }
  const atlas_prologue_config& c = h->cfg;
  const size_t rows = (size_t)c.batch * c.seq_len;
  const size_t ncol = 3 * (size_t)c.heads * c.d_head + 4 * (size_t)c.gate_rank;
  if (!h->P && rows) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return ATLAS_ERR_INVALID_ARGUMENT;
    if (hipMalloc(&h->P, rows * ncol * sizeof(atlas::bf16)) != hipSuccess) {
      (void)hipGetLastError();
      h->P = nullptr;
      return ATLAS_ERR_OUT_OF_MEMORY;
    }
  }
  h->fused = 0;
  return ATLAS_OK;
}

atlas_status atlas_prologue_set_events(atlas_prologue_t h, void* gemm_before, void* before, void* after) {
  if (!h || h->magic != kProMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  h->ev_gemm = (hipEvent_t)gemm_before;
  h->ev_before = (hipEvent_t)before;
  h->ev_after = (hipEvent_t)after;
  return ATLAS_OK;
}

atlas_status atlas_prologue_free(atlas_prologue_t h) {
  if (!h) return ATLAS_OK;
  if (h->magic != kProMagic) return ATLAS_ERR_INVALID_ARGUMENT;
  h->magic = 0;
  const hipError_t e = h->P ? hipFree(h->P) : hipSuccess;
  delete h;
  if (e != hipSuccess) {
    atlas::record_hip_error(hipGetErrorString(e));
    return ATLAS_ERR_HIP;
  }
  return ATLAS_OK;
}

}  // extern "C"
