"""Python binding of libatlas_mem.so (include/atlas_mem.h): argument
marshalling only.  Every step of the memory update and retrieval runs in the
library's HIP kernels; torch provides device memory and the stream.

The library is loaded after torch so that both use the one HIP runtime
already in the process.  There is no fallback: if the library is missing
the import of this module raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from .configs import Workload

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libatlas_mem.so")
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "atlas_mem.h")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_OOM, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4, 5
MEM = {"linear": 0, "mlp": 1}
PHI = {"identity": 0, "poly2": 1, "raw_poly2": 2}
BIAS = {"l2": 0, "dot": 1, "lp": 2, "huber": 3}
IO = {"bf16": 0, "f32": 1}
KERNEL = {"auto": 0, "per_sequence": 1, "sharded": 2, "streamed": 3, "grouped": 4}
OPTIMIZER = {"gd": 0, "muon": 1}
TORCH_IO = {"bf16": torch.bfloat16, "f32": torch.float32}


class AtlasMemConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "batch", "heads", "seq_len", "d_k", "d_v", "memory", "mlp_layers", "mlp_hidden",
        "mlp_residual", "feature_map", "poly_dims", "window", "chunk", "momentum", "bias",
        "io_dtype")] + [("grad_scale", ctypes.c_float), ("kernel", ctypes.c_int), ("bias_p", ctypes.c_float),
                       ("sign_alpha", ctypes.c_float), ("mlp_layernorm", ctypes.c_int), ("ln_eps", ctypes.c_float),
                       ("mlp_gated", ctypes.c_int), ("optimizer", ctypes.c_int), ("ns_steps", ctypes.c_int)]


class StateLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "seq_stride", "weights", "momentum", "halo_k", "halo_v", "halo_g", "count")] + [
        ("feature_dim", ctypes.c_int), ("param_count", ctypes.c_long), ("halo_d", ctypes.c_size_t)]


class PrologueConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "batch", "seq_len", "d_model", "heads", "d_head", "conv_taps", "gate_rank")]


class AtlasError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = f"{what}: {lib().atlas_mem_error_string(code).decode()}"
        if code == ERR_HIP:
            msg += f" ({lib().atlas_mem_last_hip_error().decode()})"
        super().__init__(msg)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        cp = ctypes.POINTER(AtlasMemConfig)
        vp = ctypes.c_void_p
        L.atlas_mem_init.argtypes = [cp, ctypes.POINTER(vp)]
        L.atlas_mem_init.restype = ctypes.c_int
        L.atlas_mem_supported.argtypes = [cp]
        L.atlas_mem_supported.restype = ctypes.c_int
        L.atlas_mem_state_bytes.argtypes = [vp]
        L.atlas_mem_state_bytes.restype = ctypes.c_size_t
        L.atlas_mem_state_layout_of.argtypes = [vp, ctypes.POINTER(StateLayout)]
        L.atlas_mem_state_layout_of.restype = ctypes.c_int
        L.atlas_mem_forward.argtypes = [vp] * 11
        L.atlas_mem_forward.restype = ctypes.c_int
        L.atlas_mem_forward_ex.argtypes = [vp] * 12
        L.atlas_mem_forward_ex.restype = ctypes.c_int
        L.atlas_mem_forward_noalloc.argtypes = [cp] + [vp] * 12
        L.atlas_mem_forward_noalloc.restype = ctypes.c_int
        L.atlas_mem_set_kernel_events.argtypes = [vp, vp, vp]
        L.atlas_mem_set_kernel_events.restype = ctypes.c_int
        L.atlas_mem_kernel_family.argtypes = [vp]
        L.atlas_mem_kernel_family.restype = ctypes.c_int
        L.atlas_mem_device_errors.argtypes = [vp, ctypes.POINTER(ctypes.c_uint)]
        L.atlas_mem_device_errors.restype = ctypes.c_int
        L.atlas_mem_free.argtypes = [vp]
        L.atlas_mem_free.restype = ctypes.c_int
        L.atlas_mem_error_string.argtypes = [ctypes.c_int]
        L.atlas_mem_error_string.restype = ctypes.c_char_p
        L.atlas_mem_last_hip_error.argtypes = []
        L.atlas_mem_last_hip_error.restype = ctypes.c_char_p
        pc = ctypes.POINTER(PrologueConfig)
        L.atlas_prologue_init.argtypes = [pc, ctypes.POINTER(vp)]
        L.atlas_prologue_init.restype = ctypes.c_int
        L.atlas_prologue_forward.argtypes = [vp] * 14
        L.atlas_prologue_forward.restype = ctypes.c_int
        L.atlas_prologue_set_events.argtypes = [vp] * 4
        L.atlas_prologue_set_events.restype = ctypes.c_int
        L.atlas_prologue_set_fused.argtypes = [vp, ctypes.c_int]
        L.atlas_prologue_set_fused.restype = ctypes.c_int
        L.atlas_prologue_free.argtypes = [vp]
        L.atlas_prologue_free.restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            names |= set(re.findall(r"\b(atlas_(?:mem|prologue)_\w+)\s*\(", open(os.path.join(INCLUDE, f)).read()))
    return sorted(names)


def config_of(wl: Workload, kernel: str = "auto") -> AtlasMemConfig:
    return AtlasMemConfig(kernel=KERNEL[kernel],
        batch=wl.batch, heads=wl.heads, seq_len=wl.seq_len, d_k=wl.d_k, d_v=wl.d_v,
        memory=MEM[wl.memory], mlp_layers=2 if wl.memory == "mlp" else 0, mlp_hidden=wl.hidden,
        mlp_residual=int(wl.residual), feature_map=PHI[wl.feature_map], poly_dims=wl.poly_dims,
        window=wl.window, chunk=wl.chunk, momentum=int(wl.momentum), bias=BIAS[wl.bias],
        io_dtype=IO[wl.io_dtype], grad_scale=wl.grad_scale, bias_p=getattr(wl, "bias_p", 2.0),
        sign_alpha=getattr(wl, "sign_alpha", 0.0), mlp_layernorm=int(getattr(wl, "layernorm", False)),
        ln_eps=getattr(wl, "ln_eps", 1e-5), mlp_gated=int(getattr(wl, "gated", False)),
        optimizer=OPTIMIZER[getattr(wl, "optimizer", "gd")], ns_steps=getattr(wl, "ns_steps", 5))


def supported(cfg: AtlasMemConfig) -> int:
    return lib().atlas_mem_supported(ctypes.byref(cfg))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class AtlasMem:
    """One library handle (one workload shape, one stream at a time)."""

    def __init__(self, wl: Workload | AtlasMemConfig, kernel: str = "auto"):
        self.cfg = config_of(wl, kernel) if isinstance(wl, Workload) else wl
        self.io_dtype = torch.float32 if self.cfg.io_dtype == IO["f32"] else torch.bfloat16
        h = ctypes.c_void_p()
        rc = lib().atlas_mem_init(ctypes.byref(self.cfg), ctypes.byref(h))
        if rc != OK:
            raise AtlasError(rc, "atlas_mem_init")
        self.handle = h
        lay = StateLayout()
        rc = lib().atlas_mem_state_layout_of(h, ctypes.byref(lay))
        if rc != OK:
            raise AtlasError(rc, "atlas_mem_state_layout_of")
        self.layout = lay
        self.n_seq = self.cfg.batch * self.cfg.heads
        self.state_bytes = lib().atlas_mem_state_bytes(h)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().atlas_mem_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- state buffer ---------------------------------------------------------------
    def new_state(self, weights: torch.Tensor, device="cuda") -> torch.Tensor:
        """Zeroed state with the given initial weights ([n_seq, P] float32)."""
        st = torch.zeros(self.state_bytes, dtype=torch.uint8, device=device)
        self.view(st, "weights").copy_(weights.to(device=device, dtype=torch.float32))
        return st

    def view(self, state: torch.Tensor, field: str) -> torch.Tensor:
        """[n_seq, ...] view of one field of the state buffer."""
        L, c = self.layout, self.cfg
        rows = state.view(self.n_seq, L.seq_stride)
        halo = c.window - 1
        sizes = {"weights": L.param_count, "momentum": L.param_count if c.momentum else 0,
                 "halo_k": halo * c.d_k, "halo_v": halo * c.d_v, "halo_g": halo,
                 "halo_d": halo if c.bias == BIAS["huber"] else 0}
        if field == "count":
            return rows[:, L.count:L.count + 8].view(torch.int64)[:, 0]
        off = getattr(L, field)
        return rows[:, off:off + 4 * sizes[field]].view(torch.float32)

    def set_kernel_events(self, before=None, after=None):
        """Record two torch.cuda.Event (created with enable_timing=True) around
        the recurrent kernel of every later forward; None clears."""
        raw = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
        rc = lib().atlas_mem_set_kernel_events(self.handle, raw(before), raw(after))
        if rc != OK:
            raise AtlasError(rc, "atlas_mem_set_kernel_events")

    def family(self) -> str:
        """Kernel family this handle runs ("per_sequence", "sharded", "streamed", "grouped")."""
        code = lib().atlas_mem_kernel_family(self.handle)
        return {v: k for k, v in KERNEL.items()}[code]

    def device_errors(self) -> int:
        """Error word of the last call (synchronises the device)."""
        f = ctypes.c_uint(0)
        rc = lib().atlas_mem_device_errors(self.handle, ctypes.byref(f))
        if rc != OK:
            raise AtlasError(rc, "atlas_mem_device_errors")
        return f.value

    # -- forward --------------------------------------------------------------------
    def forward(self, q, k, v, alpha, eta, theta, gamma, state, out, stream=None, delta=None):
        """Enqueues one call on `stream` (default: torch's current stream).
        delta: the per-token Huber thresholds (that bias only)."""
        if stream is None:
            stream = torch.cuda.current_stream()
        if delta is None and self.cfg.bias != BIAS["huber"]:
            rc = lib().atlas_mem_forward(
                self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(theta),
                _ptr(gamma), _ptr(state), _ptr(out), ctypes.c_void_p(stream.cuda_stream))
            what = "atlas_mem_forward"
        else:
            rc = lib().atlas_mem_forward_ex(
                self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(theta),
                _ptr(gamma), _ptr(delta), _ptr(state), _ptr(out), ctypes.c_void_p(stream.cuda_stream))
            what = "atlas_mem_forward_ex"
        if rc != OK:
            raise AtlasError(rc, what)
        return out


def forward_noalloc(wl: Workload | AtlasMemConfig, q, k, v, alpha, eta, theta, gamma, state, out,
                    errors=None, stream=None, delta=None, kernel: str = "auto") -> None:
    """atlas_mem_forward_noalloc: the call of AtlasMem.forward without a
    handle, on the library's static scratch buffer.  errors: optional int32
    device tensor of one element that receives the call's error word."""
    cfg = config_of(wl, kernel) if isinstance(wl, Workload) else wl
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().atlas_mem_forward_noalloc(
        ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(theta), _ptr(gamma),
        _ptr(delta), _ptr(state), _ptr(out), _ptr(errors), ctypes.c_void_p(stream.cuda_stream))
    if rc != OK:
        raise AtlasError(rc, "atlas_mem_forward_noalloc")


class AtlasPrologue:
    """The fused prologue (include/atlas_prologue.h): x -> q, k, v and the
    four gates in the layouts AtlasMem.forward takes."""

    def __init__(self, batch, seq_len, d_model, heads, d_head, conv_taps=4, gate_rank=16):
        self.cfg = PrologueConfig(batch=batch, seq_len=seq_len, d_model=d_model, heads=heads, d_head=d_head,
                                  conv_taps=conv_taps, gate_rank=gate_rank)
        h = ctypes.c_void_p()
        rc = lib().atlas_prologue_init(ctypes.byref(self.cfg), ctypes.byref(h))
        if rc != OK:
            raise AtlasError(rc, "atlas_prologue_init")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().atlas_prologue_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_events(self, gemm_before=None, before=None, after=None):
        raw = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
        rc = lib().atlas_prologue_set_events(self.handle, raw(gemm_before), raw(before), raw(after))
        if rc != OK:
            raise AtlasError(rc, "atlas_prologue_set_events")

    def set_fused(self, fused: bool):
        rc = lib().atlas_prologue_set_fused(self.handle, 1 if fused else 0)
        if rc != OK:
            raise AtlasError(rc, "atlas_prologue_set_fused")

    def forward(self, x, w, w_conv, gate_v, gate_b, q, k, v, alpha, eta, theta, gamma, stream=None):
        if stream is None:
            stream = torch.cuda.current_stream()
        rc = lib().atlas_prologue_forward(
            self.handle, *[_ptr(t) for t in (x, w, w_conv, gate_v, gate_b, q, k, v, alpha, eta, theta, gamma)],
            ctypes.c_void_p(stream.cuda_stream))
        if rc != OK:
            raise AtlasError(rc, "atlas_prologue_forward")
