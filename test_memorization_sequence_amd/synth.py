"""Seeded synthetic inputs for the test-time memory.

This module only draws random numbers; it holds none of the memory's
arithmetic.  Both the GPU library's tests/benchmark and the CPU oracle are
fed from it, so they see bit-identical inputs.

Recipe (one numpy Generator, default_rng(seed), draws in this order):
  q, k ~ N(0, 1)  [B, H, N, d_k], L2-normalised over the last dim in fp32
         (the architecture normalises queries and keys: Titans review sec. 4.4,
         Miras review "Training"), then rounded to bf16 for bf16 workloads;
  v    ~ N(0, 1)  [B, H, N, d_v], rounded to bf16 for bf16 workloads;
  u_alpha, u_eta, u_theta, u_gamma ~ U(lo, hi) [B, H, N]; gate = sigmoid(u)
         stored as fp32 (eta = 0 without momentum, gamma = 1 when constant);
  initial MLP weights ~ N(0, init_std^2), one draw per head, shared by every
         batch entry (W1 [H, hidden, D] then W2 [H, d_v, hidden]); zero for a
         linear memory;
  Huber bias only, drawn after those: delta_t = m_t * |v_t|_2 [B, H, N] fp32
         with m_t = 1/4 or 4, each with probability 1/2 (a threshold per token
         that depends on the input, far from the token's error norm either way);
  gated MLP memory only, drawn last: W3 [H, hidden, D] ~ N(0, init_std^2).
bf16 values are held in float32 arrays whose low 16 bits are zero.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float64).astype(np.float32)


def _gate(rng, shape, rng_range, const):
    if rng_range is None:
        return np.full(shape, const, dtype=np.float32)
    u = rng.uniform(rng_range[0], rng_range[1], size=shape)
    return (1.0 / (1.0 + np.exp(-u))).astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """Returns float32 numpy arrays q, k, v, alpha, eta, theta, gamma and the
    initial weights (w1, w2 for an MLP, per head; m for a linear memory)."""
    rng = np.random.default_rng(seed)
    B, H, N = wl.batch, wl.heads, wl.seq_len
    q = _normal(rng, (B, H, N, wl.d_k))
    k = _normal(rng, (B, H, N, wl.d_k))
    if wl.normalize_qk:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)
    v = _normal(rng, (B, H, N, wl.d_v))
    if wl.normalize_v:
        v = v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)
    if wl.io_dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    g = (B, H, N)
    alpha = _gate(rng, g, wl.alpha_u, 0.0)
    eta = _gate(rng, g, wl.eta_u if wl.momentum else None, 0.0)
    theta = _gate(rng, g, wl.theta_u, 0.0)
    if wl.theta_div != 1.0:
        theta = (theta / np.float32(wl.theta_div)).astype(np.float32)
    gamma = _gate(rng, g, wl.gamma_u, 1.0)
    out = dict(q=np.ascontiguousarray(q), k=np.ascontiguousarray(k), v=np.ascontiguousarray(v),
               alpha=alpha, eta=eta, theta=theta, gamma=gamma)
    D = wl.feature_dim
    if wl.memory == "mlp":
        if wl.init_std > 0:
            out["w1"] = (_normal(rng, (H, wl.hidden, D)) * np.float32(wl.init_std)).astype(np.float32)
            out["w2"] = (_normal(rng, (H, wl.d_v, wl.hidden)) * np.float32(wl.init_std)).astype(np.float32)
        else:
            out["w1"] = np.zeros((H, wl.hidden, D), np.float32)
            out["w2"] = np.zeros((H, wl.d_v, wl.hidden), np.float32)
    else:
        out["m"] = np.zeros((H, wl.d_v, D), np.float32)
    if wl.bias == "huber":
        vn = np.sqrt(np.sum(v.astype(np.float64) ** 2, axis=-1))
        m = np.where(rng.uniform(size=g) < 0.5, 0.25, 4.0)
        out["delta"] = (m * vn).astype(np.float32)
    if wl.memory == "mlp" and wl.gated:
        out["w3"] = (_normal(rng, (H, wl.hidden, D)) * np.float32(wl.init_std)).astype(np.float32)
    return out


def initial_weights_flat(wl: Workload, inputs: dict) -> np.ndarray:
    """[B*H, P] float32: each sequence's initial weights in the order W1 then W2
    (MLP, both row-major; then W3 for the gated memory) or M (linear,
    row-major [d_v][D])."""
    B, H = wl.batch, wl.heads
    if wl.memory == "mlp":
        parts = [inputs["w1"].reshape(H, -1), inputs["w2"].reshape(H, -1)]
        if wl.gated:
            parts.append(inputs["w3"].reshape(H, -1))
        per_head = np.concatenate(parts, axis=1)
    else:
        per_head = inputs["m"].reshape(H, -1)
    return np.ascontiguousarray(np.broadcast_to(per_head[None], (B, H, per_head.shape[1]))
                                .reshape(B * H, -1))


def make_prologue_inputs(batch, seq_len, d_model, heads, d_head, conv_taps=4, gate_rank=16, seed=0) -> dict:
    """Seeded inputs of the fused prologue (float32 arrays; x and w hold bf16
    values): x ~ N(0, 1) [B, N, d_model]; w ~ N(0, 1/d_model) [3*H*d + 4*r,
    d_model]; w_conv ~ N(0, 1/K) [3*H*d, K]; gate_v ~ N(0, 1/r) [4, H, r];
    gate_b ~ N(0, 1) [4, H]; drawn in that order."""
    rng = np.random.default_rng(seed)
    C = 3 * heads * d_head
    x = round_to_bf16(_normal(rng, (batch, seq_len, d_model)))
    w = round_to_bf16((_normal(rng, (C + 4 * gate_rank, d_model)) / np.float32(np.sqrt(d_model))).astype(np.float32))
    w_conv = (_normal(rng, (C, conv_taps)) / np.float32(np.sqrt(conv_taps))).astype(np.float32)
    gate_v = (_normal(rng, (4, heads, gate_rank)) / np.float32(np.sqrt(gate_rank))).astype(np.float32)
    gate_b = _normal(rng, (4, heads))
    return dict(x=x, w=w, w_conv=w_conv, gate_v=gate_v, gate_b=gate_b)
