// atlas_mem_muon.h -- the Muon memory optimizer inside the per-sequence chunk
// kernel (included by atlas_mem_kernels.hip after gemm_nt and the MFMA types).
//
// ATLAS summary sec. 5, "Memory Optimization": Muon takes the place of plain
// gradient descent on the memory.  Read as the published Muon optimizer
// (K. Jordan et al., 2024) with the memory's gates in its roles.  For every
// token n of a chunk and every weight matrix W of the memory, with the
// gradients of the window tokens taken at the chunk-start weights exactly as
// for gradient descent (ATLAS review sec. 3.3):
//   S <- eta_n S + g_n,    g_n = sum_{i = n-c+1..n} D_i x_i^T
//   O  = NS(S):  X = S / (|S|_F + 1e-7), on the orientation with fewer rows;
//                then ns_steps times X <- a X + (b A + c A A) X, A = X X^T,
//                (a, b, c) = (3.4445, -4.7750, 2.0315)
//   W <- (1 - alpha_n) W - theta_n O
// and then y_n = f_W(phi(q_n)) with the token's own weights.
//
// O is a nonlinear function of S, so unlike gradient descent the per-token
// weights are not sums of outer products and the chunk's dual form does not
// apply: every token materialises S and W (fp32, in the state and an
// L2-resident workspace) and runs the iteration.  Its three GEMMs per step are
// fp32 MFMA (16x16x4) through gemm_nt, in fp32 because the iteration
// amplifies noise along the near-null directions of S (about 3.4x per step),
// which a low-rank momentum has many of.
#pragma once

namespace atlas {

// Hand-off inside a pair of workgroups of one XCD (the counter is the pair's
// group-barrier counter; see atlas_mem_group.h).  signal: every wave's stores
// are complete (they write through the CU's L1 to the shared L2), then one
// arrival.  wait: bounded poll until the counter reaches target, then the
// CU's L1 is invalidated so that later loads see the partner's stores.
__device__ __forceinline__ void pair_signal(unsigned* ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(ctr, 1u);
}

__device__ __forceinline__ void pair_wait(unsigned* ctr, unsigned target, unsigned* err) {
  if (threadIdx.x == 0) {
    unsigned polls = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
      if (++polls > (1u << 24)) {
        atomicOr(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  asm volatile("buffer_inv sc0" ::: "memory");
}

__device__ __forceinline__ float muon_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// B X step for an orientation with R <= 128 rows: B (R x R) sits in LDS at
// pitch R + 4 (16-byte fragment reads without bank conflicts), X is read
// straight from the workspace as the MFMA's B operand (lane l: row k, column
// l & 15, so 16 lanes read 64 contiguous bytes), and each wave owns whole
// 32-column strips of Y = sx (a X + B X) over all R / 32 row blocks.  Every
// X element is read once, and no transposed copy of X is needed.
template <int R, int NN>
__device__ void ns_bx(const float* Bs, const float* X, float* Y, float ca, float sx) {
  constexpr int BP = R + 4, RB = R / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
#pragma unroll 1
  for (int n0 = 32 * wave; n0 < NN; n0 += 32 * nwaves) {
    f32x4 acc[RB][2][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[rb][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k0 = 0; k0 < R; k0 += 16) {
      // MFMA step e contracts k = k0 + 4 g + e (the fragment order of Mma<float>)
      f32x4 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) b[j][e] = X[(size_t)(k0 + 4 * g + e) * NN + n0 + 16 * j + c16];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(Bs + (32 * rb + 16 * i + c16) * BP + k0 + 4 * g);
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[rb][i][j] = Mma<float>::mma(a, b[j], acc[rb][i][j]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const size_t e = (size_t)(32 * rb + 16 * i + 4 * g + r) * NN + n0 + 16 * j + c16;
            Y[e] = sx * (ca * X[e] + acc[rb][i][j][r]);
          }
  }
}

// A = sa X X^T for R <= 128: X passes through LDS (the region of B, R x (R + 4)
// floats) one block of R columns at a time, so every X element is read from
// the workspace once; the upper tiles of A (32 x 32, at most two per wave)
// keep their accumulators across the blocks, and the epilogue mirrors them.
template <int R, int NN>
__device__ void ns_xxt(const float* X, float* Am, float* Ls, float sa) {
  constexpr int BP = R + 4, TN = R / 32, NTL = TN * (TN + 1) / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int tm[2], tn[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {   // the wave's tiles, row by row of the upper triangle
    int t = wave + s * nwaves, mt = 0;
    while (mt < TN && t >= TN - mt) { t -= TN - mt; ++mt; }
    tm[s] = mt;
    tn[s] = mt + t;
  }
  f32x4 acc[2][2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[s][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < NN; kb += R) {
    const int kw = NN - kb < R ? NN - kb : R;   // a multiple of 32
    __syncthreads();   // the previous block is consumed
    for (int e = threadIdx.x; e < R * (kw / 4); e += blockDim.x) {
      const int row = e / (kw / 4), q4 = e % (kw / 4);
      *reinterpret_cast<f32x4*>(Ls + row * BP + 4 * q4) =
          *reinterpret_cast<const f32x4*>(X + (size_t)row * NN + kb + 4 * q4);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (wave + s * nwaves >= NTL) break;
      const float* ra = Ls + (32 * tm[s] + c16) * BP + 4 * g;
      const float* rb = Ls + (32 * tn[s] + c16) * BP + 4 * g;
#pragma unroll 1
      for (int k0 = 0; k0 < kw; k0 += 16) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ra + k0);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(ra + 16 * BP + k0);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(rb + k0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(rb + 16 * BP + k0);
        acc[s][0][0] = Mma<float>::mma(a0, b0, acc[s][0][0]);
        acc[s][0][1] = Mma<float>::mma(a0, b1, acc[s][0][1]);
        acc[s][1][0] = Mma<float>::mma(a1, b0, acc[s][1][0]);
        acc[s][1][1] = Mma<float>::mma(a1, b1, acc[s][1][1]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (wave + s * nwaves >= NTL) break;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 32 * tm[s] + 16 * i + 4 * g + r, col = 32 * tn[s] + 16 * j + c16;
          const float v = sa * acc[s][i][j][r];
          Am[row * R + col] = v;
          if (tm[s] != tn[s]) Am[col * R + row] = v;
        }
  }
}

// One token's Muon step on the weight matrix Wm [ROWS][COLS] (fp32, row
// major) with momentum Sm of the same shape and the running window gradient
// Gm (workspace, same shape).  Dt [ROWS][WP] and Xc [>= COLS][WP] hold the
// gradient factors of the window rows: G_w = Dt[:, w] Xc[:, w]^T.  The
// window of the token is rows w0 .. w0 + c - 1.  first: the chunk's first
// token (the window sum is formed directly); later tokens add row w0 + c - 1
// and drop row w0 - 1, with both rows' factors staged in `stage` (LDS,
// 2 (ROWS + COLS) floats).  c == 1 takes G_{w0} itself.  bs: LDS for B
// (R (R + 4) floats) when R <= 128; larger orientations keep B and a
// transposed copy of X in the workspace.
// Every thread of the workgroup calls this; it ends on a barrier.
template <class S, int ROWS, int COLS, typename T>
__device__ void muon_matrix(float* Wm, float* Sm, float* Gm, float eta, const T* Dt, const T* Xc, int w0, int c,
                            bool first, float alpha, float theta, int steps, char* mws, float* red, float* stage,
                            float* bs) {
  constexpr int WP = S::WP;
  constexpr bool TR = ROWS > COLS;
  constexpr int R = (int)ns_r(ROWS, COLS), NN = (int)ns_n(ROWS, COLS);
  // B in LDS when every orientation of the memory has at most 128 rows (the
  // launch sizes the LDS by the largest)
  constexpr long RMAX = S::MEM == MEM_MLP ? lmax(ns_r(S::H, S::D), ns_r(S::DV, S::H)) : ns_r(S::DV, S::D);
  constexpr bool LDSB = RMAX <= 128;
  constexpr MuonWs L = muon_ws_of(S::MEM == MEM_MLP, S::D, S::DV, S::H, S::BC);
  float* X[2] = {reinterpret_cast<float*>(mws + L.x0), reinterpret_cast<float*>(mws + L.x1)};
  float* Xt[2] = {reinterpret_cast<float*>(mws + L.xt0), reinterpret_cast<float*>(mws + L.xt1)};
  float* Am = reinterpret_cast<float*>(mws + L.am);
  float* Bm = reinterpret_cast<float*>(mws + L.bm);

  // factors of the rows entering (dn, xn) and leaving (dd, xd) the window
  float* dn = stage;
  float* dd = stage + ROWS;
  float* xn = stage + 2 * ROWS;
  float* xd = stage + 2 * ROWS + COLS;
  const bool running = c > 1 && !first;
  const int wn = c == 1 ? w0 : w0 + c - 1, wd = w0 - 1;
  for (int r = threadIdx.x; r < ROWS; r += blockDim.x) {
    dn[r] = to_f(Dt[r * WP + wn]);
    dd[r] = running ? to_f(Dt[r * WP + wd]) : 0.f;
  }
  for (int q = threadIdx.x; q < COLS; q += blockDim.x) {
    xn[q] = to_f(Xc[q * WP + wn]);
    xd[q] = running ? to_f(Xc[q * WP + wd]) : 0.f;
  }
  __syncthreads();

  // the chunk's first window sum as one GEMM (bf16 MFMA, fp32 sums) when the
  // window is a whole number of MFMA k-steps and the matrix whole tiles;
  // otherwise each element sums its c terms below
  const bool gemm_first = c > 1 && first && c % Mma<T>::KSTEP == 0 && ROWS % 32 == 0 && COLS % 32 == 0;
  if (gemm_first) {
    Op<T> ops[1] = {{Dt + w0, WP, Xc + w0, WP, c}};
    gemm_nt(ROWS, COLS, ops, [&](int r, int q, const float* a) { Gm[r * COLS + q] = a[0]; });
    __syncthreads();
  }

  // g, S <- eta S + g, |S|_F^2; S into X[0] and X[0]^T (unscaled), walking S
  // in its own row-major order
  float ss = 0.f;
  for (int e = threadIdx.x; e < ROWS * COLS; e += blockDim.x) {
    const int r = e / COLS, q = e % COLS;
    float g;
    if (c == 1) {
      g = dn[r] * xn[q];
    } else if (gemm_first) {
      g = Gm[e];
    } else if (first) {
      g = 0.f;
      for (int w = w0; w < w0 + c; ++w) g += to_f(Dt[r * WP + w]) * to_f(Xc[q * WP + w]);
      Gm[e] = g;
    } else {
      g = Gm[e] + dn[r] * xn[q] - dd[r] * xd[q];
      Gm[e] = g;
    }
    const float s = eta * Sm[e] + g;
    Sm[e] = s;
    ss += s * s;
    const int i = TR ? q : r, j = TR ? r : q;   // position in the R x NN orientation
    X[0][i * NN + j] = s;
    if (!LDSB) Xt[0][j * R + i] = s;
  }
  // zero padding of the R x NN orientation (a no-op when both are multiples of 32)
  constexpr int RR = TR ? COLS : ROWS, NR = TR ? ROWS : COLS;
  if (RR != R || NR != NN)
    for (int e = threadIdx.x; e < R * NN; e += blockDim.x) {
      const int i = e / NN, j = e % NN;
      if (i >= RR || j >= NR) {
        X[0][e] = 0.f;
        if (!LDSB) Xt[0][j * R + i] = 0.f;
      }
    }
  ss = muon_wave_sum(ss);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
  // X_0 = S / (|S|_F + 1e-7): the scale is folded into the first step
  const float inv = 1.f / (sqrtf(tot) + 1e-7f);

  const float ca = 3.4445f, cb = -4.7750f, cc = 2.0315f;
  int cur = 0;
  for (int it = 0; it < steps; ++it) {
    const float* Xc_ = X[cur];
    float* Xn = X[cur ^ 1];
    float* Xtn = Xt[cur ^ 1];
    const float sa = it == 0 ? inv * inv : 1.f, sx = it == 0 ? inv : 1.f;
    if constexpr (LDSB) {  // A = X X^T, X staged through LDS
      static_assert((R / 32) * (R / 32 + 1) / 2 <= 2 * 8, "at most two tiles of A per wave");
      ns_xxt<R, NN>(Xc_, Am, bs, sa);
    } else {  // A = X X^T (symmetric: upper tiles, mirrored)
      Op<float> ops[1] = {{Xc_, NN, Xc_, NN, NN}};
      gemm_nt(R, R, ops, [&](int i, int j, const float* a) {
        const float v = sa * a[0];
        Am[i * R + j] = v;
        if ((i >> 5) != (j >> 5)) Am[j * R + i] = v;
      }, true);
    }
    __syncthreads();
    {  // B = b A + c A A  (A symmetric: A A = A A^T, and B is symmetric)
      Op<float> ops[1] = {{Am, R, Am, R, R}};
      float* Bd = LDSB ? bs : Bm;
      constexpr int BP = LDSB ? R + 4 : R;
      gemm_nt(R, R, ops, [&](int i, int j, const float* a) {
        const float v = cb * Am[i * R + j] + cc * a[0];
        Bd[i * BP + j] = v;
        if ((i >> 5) != (j >> 5)) Bd[j * BP + i] = v;
      }, true);
    }
    __syncthreads();
    if constexpr (LDSB) {  // X <- a X + B X
      ns_bx<R, NN>(bs, Xc_, Xn, ca, sx);
    } else {  // X <- a X + B X, also transposed for the next step's B X
      Op<float> ops[1] = {{Bm, R, Xt[cur], R, R}};
      gemm_nt(R, NN, ops, [&](int i, int j, const float* a) {
        const float y = sx * (ca * Xc_[i * NN + j] + a[0]);
        Xn[i * NN + j] = y;
        Xtn[j * R + i] = y;
      });
    }
    __syncthreads();
    cur ^= 1;
  }

  // W <- (1 - alpha) W - theta O
  const float* O = X[cur];
  const float keep = 1.f - alpha;
  for (int e = threadIdx.x; e < ROWS * COLS; e += blockDim.x) {
    const int r = e / COLS, q = e % COLS;
    const float o = TR ? O[q * NN + r] : O[r * NN + q];
    Wm[e] = keep * Wm[e] - theta * o;
  }
  __syncthreads();
}

}  // namespace atlas
