"""Workload presets for the test-time memory (update + retrieval).

Each preset fixes the memory form, the feature map, the Omega window c, the
chunk b, the shapes and the recipe of the synthetic inputs.  The memory forms
follow the Titans review (sec. 3.1 "Memory Architecture": matrix or MLP
memory) and the ATLAS review (sec. 3.1 "Polynomial Feature Mapping", sec. 3.2
"Omega Rule", sec. 3.3 chunking).

Gate recipes are (lo, hi) ranges of U(lo, hi) pushed through a sigmoid; None
means the gate is constant (eta = 0 without momentum, gamma = 1 when c = 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    d_k: int
    d_v: int
    memory: str            # "linear" | "mlp"
    hidden: int            # MLP hidden width (0 for linear)
    residual: bool         # MLP: y = r + W2 gelu(W1 phi(x)), r the raw key/query
    feature_map: str       # "identity" | "poly2" | "raw_poly2"
    poly_dims: int         # leading key dims fed to the degree-2 map
    window: int            # Omega window c
    chunk: int             # chunk b
    momentum: bool
    io_dtype: str          # "bf16" | "f32" for q, k, v, out
    bias: str = "l2"       # "l2" | "dot" | "lp" | "huber"
    grad_scale: float = 1.0
    bias_p: float = 2.0    # p of the l_p bias
    sign_alpha: float = 0.0  # l_p / Huber: 0 exact sign(e), > 0 tanh(sign_alpha * e)
    layernorm: bool = False  # MLP: f = r + LN(W2 gelu(W1 x))
    ln_eps: float = 1e-5
    gated: bool = False    # MLP: f = r + W2 (gelu(W1 x) .* (W3 x))
    optimizer: str = "gd"  # "gd": momentum + decay; "muon": Newton-Schulz on the momentum
    ns_steps: int = 5      # Muon: Newton-Schulz steps
    alpha_u: tuple | None = (-4.0, 0.0)
    theta_u: tuple | None = (-4.0, 0.0)
    eta_u: tuple | None = (0.0, 3.0)
    gamma_u: tuple | None = (-2.0, 2.0)
    init_std: float = 0.0  # std of the initial MLP weights (0: zero init)
    normalize_qk: bool = True
    normalize_v: bool = False
    theta_div: float = 1.0  # theta = sigmoid(u) / theta_div
    note: str = field(default="", compare=False)

    @property
    def feature_dim(self) -> int:
        p = self.poly_dims
        if self.feature_map == "identity":
            return self.d_k
        if self.feature_map == "poly2":
            return self.d_k + self.d_k * (self.d_k + 1) // 2
        return self.d_k + p + p * (p + 1) // 2

    @property
    def n_seq(self) -> int:
        return self.batch * self.heads

    def with_shape(self, batch=None, heads=None, seq_len=None) -> "Workload":
        return replace(self, batch=batch or self.batch, heads=heads or self.heads,
                       seq_len=seq_len if seq_len is not None else self.seq_len)


WORKLOADS = {
    # matrix memory 64x64, delta rule (c = 1), no momentum, fp32 io
    "linear64_delta": Workload(
        "linear64_delta", 1, 1, 1024, 64, 64, "linear", 0, False, "identity", 0,
        window=1, chunk=64, momentum=False, io_dtype="f32", eta_u=None, gamma_u=None,
        note="linear 64x64, c=1, no momentum, fp32"),
    # matrix memory on phi(k) = [k, upper-tri(k k^T)] (32 -> 560), c = 16, momentum
    "linear_poly2": Workload(
        "linear_poly2", 2, 8, 4096, 32, 32, "linear", 0, False, "poly2", 32,
        window=16, chunk=64, momentum=True, io_dtype="bf16", theta_div=16.0,
        note="linear 560x32 poly2, c=16, momentum, bf16"),
    # 2-layer residual MLP 64-256-64, c = 1, momentum + decay
    "mlp64": Workload(
        "mlp64", 4, 16, 8192, 64, 64, "mlp", 256, True, "identity", 0,
        window=1, chunk=64, momentum=True, io_dtype="bf16", gamma_u=None, init_std=0.02,
        note="MLP 64-256-64 residual, c=1, momentum, bf16"),
    # ATLAS-style: [k, poly2(k[:32])] (688) -> 512 -> 128 residual MLP, c = 64, N = 32768
    "atlas_long": Workload(
        "atlas_long", 1, 8, 32768, 128, 128, "mlp", 512, True, "raw_poly2", 32,
        window=64, chunk=64, momentum=True, io_dtype="bf16", init_std=0.02, theta_div=64.0,
        note="MLP 688-512-128 residual, raw+poly2 map, c=64, N=32768, bf16"),
    # layer scale: d_model 1536 = 12 heads x 128, MLP 128-512-128, c = 32, B = 8, N = 16384
    "layer_scale": Workload(
        "layer_scale", 8, 12, 16384, 128, 128, "mlp", 512, True, "identity", 0,
        window=32, chunk=64, momentum=True, io_dtype="bf16", init_std=0.02, theta_div=32.0,
        note="MLP 128-512-128 residual, c=32, 8x12 heads, N=16384, bf16"),
}

# Gate recipes under which the memory changes a lot over a few hundred tokens
# and stays finite (small decay).  Used by the parity tests next to each
# preset's own recipe, because several presets decay to the W = 0 fixed point
# of the MLP memory within a few chunks.
LIVELY = {
    "linear64_delta": dict(alpha_u=(-8.0, -4.0)),
    "linear_poly2": dict(alpha_u=(-8.0, -4.0), theta_div=16.0),
    "mlp64": dict(alpha_u=(-8.0, -4.0), theta_u=(-6.0, -2.0)),
    "atlas_long": dict(alpha_u=(-8.0, -4.0), theta_div=128.0),
    "layer_scale": dict(alpha_u=(-8.0, -4.0), theta_div=64.0),
}


def lively(wl: Workload) -> Workload:
    return replace(wl, **LIVELY[wl.name])


# the order the five workloads are listed in
ORDER = ["linear64_delta", "linear_poly2", "mlp64", "atlas_long", "layer_scale"]
