"""fp64 CPU oracle of the fused prologue that produces the memory's inputs.

TEST INFRASTRUCTURE ONLY: the plain, slow reference the GPU prologue is
checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the GPU library.

What it computes, per sequence b and token t (Titans review, sec. 4.4
"Architectural Details": SiLU on the query/key/value computation, L2-norm of
queries and keys, a 1D depthwise convolution after the q/k/v projections;
Miras review, "Training": depthwise convolution across tokens after q, k, v,
L2-normalised q and k, gates as per-token values from low-rank projections):

  P_t        = W x_t                  W = [Wq; Wk; Wv; U_alpha; U_eta; U_theta; U_gamma]
  c_t        = sum_{j=0}^{K-1} w_conv[ch, j] * P_{t-(K-1)+j}[ch]     (q, k, v channels;
               rows before the sequence's first token count as zero)
  q, k, v    = SiLU(c), SiLU(z) = z * sigmoid(z)
  q, k       <- q / max(|q|_2, 1e-12), likewise k, per head (over its d channels)
  gate_g     = sigmoid(V_g (U_g x_t) + b_g) per head, g in alpha, eta, theta, gamma

Shapes: x [B][N][d_model]; W [3*H*d + 4*r][d_model]; w_conv [3*H*d][K];
V [4][H][r]; b [4][H].  Outputs q, k, v [B][H][N][d], gates [4][B][H][N].
"""
from __future__ import annotations

import numpy as np


def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def prologue(x, W, w_conv, V, b, heads: int, d_head: int, rank: int):
    """Returns (q, k, v, gates) in fp64, following the steps above literally."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    w_conv = np.asarray(w_conv, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    B, N, _ = x.shape
    H, d, r = heads, d_head, rank
    C = 3 * H * d
    K = w_conv.shape[1]
    P = x @ W.T                                      # [B][N][C + 4r]
    conv = np.zeros((B, N, C))
    for t in range(N):
        for j in range(K):
            src = t - (K - 1) + j
            if src >= 0:
                conv[:, t, :] += w_conv[:, j] * P[:, src, :C]
    act = silu(conv)
    q = act[..., 0 * H * d:1 * H * d].reshape(B, N, H, d)
    k = act[..., 1 * H * d:2 * H * d].reshape(B, N, H, d)
    v = act[..., 2 * H * d:3 * H * d].reshape(B, N, H, d)
    q = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-12)
    k = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-12)
    gates = np.zeros((4, B, H, N))
    for g in range(4):
        u = P[..., C + g * r:C + (g + 1) * r]        # [B][N][r]
        gates[g] = sigmoid((u @ V[g].T).transpose(0, 2, 1) + b[g][None, :, None])
    to_bhnd = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    return to_bhnd(q), to_bhnd(k), to_bhnd(v), gates
