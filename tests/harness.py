"""Shared helpers of the GPU tests: run the library and the oracle on the
same seeded inputs and compare."""
import numpy as np

from oracle import oracle as O
from test_memorization_sequence_amd import synth


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def tol_of(wl):
    """Output/state tolerance: rel. L2 2e-2 for bf16 io, 1e-4 for fp32 io."""
    return 1e-4 if wl.io_dtype == "f32" else 2e-2


def to_device(wl, inputs, device="cuda"):
    import torch
    io = torch.float32 if wl.io_dtype == "f32" else torch.bfloat16
    d = {}
    for key in ("q", "k", "v"):
        d[key] = torch.from_numpy(inputs[key]).to(device=device, dtype=io).contiguous()
    for key in ("alpha", "eta", "theta", "gamma", "delta"):
        if key in inputs:
            d[key] = torch.from_numpy(inputs[key]).to(device=device).contiguous()
    return d


def gpu_run(mem, wl, dev_inputs, state, out=None):
    import torch
    if out is None:
        out = torch.empty(wl.batch, wl.heads, wl.seq_len, wl.d_v, dtype=mem.io_dtype, device="cuda")
    mem.forward(dev_inputs["q"], dev_inputs["k"], dev_inputs["v"], dev_inputs["alpha"],
                dev_inputs["eta"] if wl.momentum else None, dev_inputs["theta"], dev_inputs["gamma"],
                state, out, delta=dev_inputs.get("delta"))
    return out


def gpu_state_np(mem, state):
    return {f: mem.view(state, f).cpu().numpy().astype(np.float64 if f != "count" else np.int64)
            for f in ("weights", "momentum", "halo_k", "halo_v", "halo_g", "halo_d", "count")}


def compare(wl, inputs, out_gpu, st_gpu, out_or, st_or, seqs=None, n_tokens=None):
    """Returns a dict of relative errors and exact-match flags."""
    S = wl.batch * wl.heads
    seqs = list(range(S)) if seqs is None else list(seqs)
    n = wl.seq_len if n_tokens is None else n_tokens
    y = np.asarray(out_gpu, dtype=np.float64).reshape(S, wl.seq_len, wl.d_v)[seqs, :n]
    res = {"out": rel_l2(y, out_or)}
    if wl.memory == "mlp" and wl.residual:
        # The memory's own contribution y - r.  y is returned in the io dtype,
        # so even an exact computation is off by the rounding of y; that part
        # (twice the oracle's own rounding error, in L2) is not charged.
        r = inputs["q"].reshape(S, wl.seq_len, wl.d_k)[seqs, :n].astype(np.float64)
        quant = 0.0
        if wl.io_dtype == "bf16":
            quant = np.linalg.norm(synth.round_to_bf16(out_or.astype(np.float32)).astype(np.float64) - out_or)
        den = max(np.linalg.norm(out_or - r), 1e-300)
        res["memory_part"] = max(0.0, np.linalg.norm(y - out_or) - 2.0 * quant) / den
        res["memory_part_raw"] = rel_l2(y - r, out_or - r)
    if st_gpu is not None:
        res["weights"] = rel_l2(st_gpu["weights"][seqs], st_or["mem"])
        if wl.momentum:
            res["momentum"] = rel_l2(st_gpu["momentum"][seqs], st_or["mom"])
        res["halo_exact"] = bool(np.array_equal(st_gpu["halo_k"][seqs].reshape(st_or["halo_k"].shape), st_or["halo_k"])
                                 and np.array_equal(st_gpu["halo_v"][seqs].reshape(st_or["halo_v"].shape), st_or["halo_v"])
                                 and np.array_equal(st_gpu["halo_g"][seqs], st_or["halo_g"])
                                 and (wl.bias != "huber" or np.array_equal(st_gpu["halo_d"][seqs], st_or["halo_d"])))
        res["count_exact"] = bool(np.array_equal(st_gpu["count"][seqs], st_or["count"]))
    return res


def prepare(wl, seed=0):
    inputs = synth.make_inputs(wl, seed)
    w0 = synth.initial_weights_flat(wl, inputs)
    return inputs, w0
