"""ctypes binding of the fp64 CPU oracle (atlas_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  It imports nothing
from the GPU library's package and the GPU library imports nothing from here.

All arrays are numpy float64 (count: int64), C-contiguous.  The oracle's
state is kept as separate arrays (weights, momentum, halo keys/values/gammas,
token count); see atlas_oracle.h for their shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "atlas_oracle.c")
LIB_PATH = os.environ.get("ATLAS_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

LINEAR, MLP = 0, 1
PHI = {"identity": 0, "poly2": 1, "raw_poly2": 2}
BIAS = {"l2": 0, "dot": 1, "lp": 2, "huber": 3}
OPTIMIZER = {"gd": 0, "muon": 1}


def build(src: str = SRC, out: str | None = None) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) into a shared library."""
    out = out or LIB_PATH
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class OracleConfig(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int),
        ("seq_len", ctypes.c_int),
        ("d_k", ctypes.c_int),
        ("d_v", ctypes.c_int),
        ("memory", ctypes.c_int),
        ("hidden", ctypes.c_int),
        ("residual", ctypes.c_int),
        ("feature_map", ctypes.c_int),
        ("poly_dims", ctypes.c_int),
        ("window", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("momentum", ctypes.c_int),
        ("bias", ctypes.c_int),
        ("grad_scale", ctypes.c_double),
        ("bias_p", ctypes.c_double),
        ("sign_alpha", ctypes.c_double),
        ("layernorm", ctypes.c_int),
        ("ln_eps", ctypes.c_double),
        ("gated", ctypes.c_int),
        ("optimizer", ctypes.c_int),
        ("ns_steps", ctypes.c_int),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        cp = ctypes.POINTER(OracleConfig)
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_feature_dim.argtypes = [cp]
        L.oracle_feature_dim.restype = ctypes.c_int
        L.oracle_param_count.argtypes = [cp]
        L.oracle_param_count.restype = ctypes.c_long
        L.oracle_phi.argtypes = [cp, dp, dp]
        L.oracle_memory_apply.argtypes = [cp, dp, dp, dp, dp]
        L.oracle_token_grad.argtypes = [cp, dp, dp, dp, dp, ctypes.c_double, dp]
        L.oracle_token_grad_ex.argtypes = [cp, dp, dp, dp, dp, ctypes.c_double, ctypes.c_double, dp]
        L.oracle_forward.argtypes = [cp] + [dp] * 7 + [dp] * 5 + [ctypes.POINTER(ctypes.c_int64), dp]
        L.oracle_forward.restype = ctypes.c_int
        L.oracle_forward_ex.argtypes = [cp] + [dp] * 8 + [dp] * 6 + [ctypes.POINTER(ctypes.c_int64), dp]
        L.oracle_forward_ex.restype = ctypes.c_int
        L.oracle_newton_schulz.argtypes = [dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp]
        _lib = L
    return _lib


def make_config(*, n_seq=1, seq_len=0, d_k, d_v, memory="linear", hidden=0, residual=False,
                feature_map="identity", poly_dims=0, window=1, chunk=1, momentum=False,
                bias="l2", grad_scale=1.0, bias_p=2.0, sign_alpha=0.0, layernorm=False,
                ln_eps=1e-5, gated=False, optimizer="gd", ns_steps=5) -> OracleConfig:
    return OracleConfig(
        n_seq=n_seq, seq_len=seq_len, d_k=d_k, d_v=d_v,
        memory=MLP if memory == "mlp" else LINEAR, hidden=hidden, residual=int(bool(residual)),
        feature_map=PHI[feature_map], poly_dims=poly_dims, window=window, chunk=chunk,
        momentum=int(bool(momentum)), bias=BIAS[bias], grad_scale=float(grad_scale),
        bias_p=float(bias_p), sign_alpha=float(sign_alpha), layernorm=int(bool(layernorm)),
        ln_eps=float(ln_eps), gated=int(bool(gated)), optimizer=OPTIMIZER[optimizer],
        ns_steps=int(ns_steps))


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"] and a.dtype == np.float64
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def feature_dim(cfg: OracleConfig) -> int:
    return lib().oracle_feature_dim(ctypes.byref(cfg))


def param_count(cfg: OracleConfig) -> int:
    return lib().oracle_param_count(ctypes.byref(cfg))


def phi(cfg: OracleConfig, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(feature_dim(cfg))
    lib().oracle_phi(ctypes.byref(cfg), _p(x), _p(out))
    return out


def newton_schulz(G, steps: int = 5) -> np.ndarray:
    """Muon's orthogonalisation of one matrix (atlas_oracle.c)."""
    G = np.ascontiguousarray(G, dtype=np.float64)
    out = np.zeros_like(G)
    lib().oracle_newton_schulz(_p(G), G.shape[0], G.shape[1], int(steps), _p(out))
    return out


def memory_apply(cfg: OracleConfig, theta, x, r) -> np.ndarray:
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    x = np.ascontiguousarray(x, dtype=np.float64)
    r = np.ascontiguousarray(r, dtype=np.float64)
    y = np.zeros(cfg.d_v)
    lib().oracle_memory_apply(ctypes.byref(cfg), _p(theta), _p(x), _p(r), _p(y))
    return y


def token_grad(cfg: OracleConfig, theta, x, r, v, gamma, delta=0.0) -> np.ndarray:
    """Gradient of one token's weighted loss; delta: its Huber threshold."""
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (theta, x, r, v)]
    g = np.zeros(param_count(cfg))
    lib().oracle_token_grad_ex(ctypes.byref(cfg), *[_p(a) for a in arrs], float(gamma), float(delta), _p(g))
    return g


def empty_state(cfg: OracleConfig) -> dict:
    """Zero state for cfg.n_seq sequences (weights, momentum, halo, count)."""
    P, S, c = param_count(cfg), cfg.n_seq, cfg.window
    return {
        "mem": np.zeros((S, P)),
        "mom": np.zeros((S, P)),
        "halo_k": np.zeros((S, max(c - 1, 0), cfg.d_k)),
        "halo_v": np.zeros((S, max(c - 1, 0), cfg.d_v)),
        "halo_g": np.zeros((S, max(c - 1, 0))),
        "halo_d": np.zeros((S, max(c - 1, 0))),
        "count": np.zeros(S, dtype=np.int64),
    }


def forward(cfg: OracleConfig, q, k, v, alpha, eta, theta, gamma, state: dict,
            threads: int | None = None, delta=None):
    """Runs one call.  q,k: [S,N,d_k]; v: [S,N,d_v]; gates (and delta, the
    Huber thresholds, needed by that bias only): [S,N].
    `state` (from empty_state or a previous call) is updated in place.
    Returns (out [S,N,d_v], threads_used)."""
    S, N = q.shape[0], q.shape[1]
    cfg = OracleConfig.from_buffer_copy(cfg)
    cfg.n_seq, cfg.seq_len = S, N
    if delta is None:
        delta = np.zeros((S, N))
    ins = [np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, alpha, eta, theta, gamma, delta)]
    state.setdefault("halo_d", np.zeros((S, max(cfg.window - 1, 0))))
    for key in ("mem", "mom", "halo_k", "halo_v", "halo_g", "halo_d"):
        assert state[key].dtype == np.float64 and state[key].flags["C_CONTIGUOUS"], key
        assert state[key].shape[0] == S, key
    assert state["count"].dtype == np.int64
    out = np.zeros((S, N, cfg.d_v))
    if threads:
        lib().oracle_set_threads(int(threads))
    used = lib().oracle_forward_ex(
        ctypes.byref(cfg), *[_p(a) for a in ins],
        _p(state["mem"]), _p(state["mom"]), _p(state["halo_k"]), _p(state["halo_v"]),
        _p(state["halo_g"]), _p(state["halo_d"]), state["count"].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        _p(out))
    if used < 0:
        raise ValueError("oracle rejected the configuration")
    return out, used


def config_for(wl) -> OracleConfig:
    """Oracle configuration for a workload description (any object with the
    workload fields: d_k, d_v, memory, hidden, residual, feature_map,
    poly_dims, window, chunk, momentum, bias, grad_scale; bias_p if present)."""
    return make_config(d_k=wl.d_k, d_v=wl.d_v, memory=wl.memory, hidden=wl.hidden,
                       residual=wl.residual, feature_map=wl.feature_map, poly_dims=wl.poly_dims,
                       window=wl.window, chunk=wl.chunk, momentum=wl.momentum, bias=wl.bias,
                       grad_scale=wl.grad_scale, bias_p=getattr(wl, "bias_p", 2.0),
                       sign_alpha=getattr(wl, "sign_alpha", 0.0), layernorm=getattr(wl, "layernorm", False),
                       ln_eps=getattr(wl, "ln_eps", 1e-5), gated=getattr(wl, "gated", False),
                       optimizer=getattr(wl, "optimizer", "gd"), ns_steps=getattr(wl, "ns_steps", 5))


def run_workload(wl, inputs: dict, weights0, seqs=None, n_tokens=None, state=None, threads=None):
    """Runs the oracle on generator inputs ([B,H,N,...] float32 arrays).
    weights0: [B*H, P] initial weights.  seqs: flat sequence indices to run
    (default all); n_tokens: prefix length (default all).  Returns
    (out [S, n, d_v] float64, state dict)."""
    S_all = wl.batch * wl.heads
    seqs = list(range(S_all)) if seqs is None else list(seqs)
    n = wl.seq_len if n_tokens is None else n_tokens

    def take(a):
        a = a.reshape(S_all, a.shape[2], *a.shape[3:])
        return np.ascontiguousarray(a[seqs, :n], dtype=np.float64)

    cfg = config_for(wl)
    cfg.n_seq = len(seqs)
    if state is None:
        state = empty_state(cfg)
        state["mem"][:] = np.asarray(weights0, dtype=np.float64)[seqs]
    delta = take(inputs["delta"]) if "delta" in inputs else None
    out, used = forward(cfg, *(take(inputs[key]) for key in ("q", "k", "v", "alpha", "eta", "theta", "gamma")),
                        state, threads=threads, delta=delta)
    return out, state, used
