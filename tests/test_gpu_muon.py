"""Parity of the library's Muon memory optimizer with the fp64 oracle (needs
an MI355X).

Muon (ATLAS summary sec. 5, "Memory Optimization") replaces gradient descent
on the memory: per token, S = eta S + grad, each weight matrix moves by
-theta NS(S) after the decay, NS the quintic Newton-Schulz iteration of the
published Muon optimizer.  It runs on the per-sequence family.  Same inputs,
same tolerances as the gradient-descent parity tests: relative L2 2e-2 for
bf16 io, 1e-4 for fp32 io, on the outputs, the memory's own contribution,
the final weights and the final momentum; halo and count exact.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

from test_memorization_sequence_amd.configs import WORKLOADS, lively

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_memorization_sequence_amd import binding
    import harness
    return binding, harness


def _muon(name, n, recipe="preset", **kw):
    wl = WORKLOADS[name].with_shape(batch=1, heads=2, seq_len=n)
    if recipe == "lively":
        wl = lively(wl)
    return replace(wl, optimizer="muon", **kw)


def _parity(B, wl):
    binding, H = B
    inputs, w0 = H.prepare(wl)
    mem = binding.AtlasMem(wl)
    assert mem.family() == "per_sequence"
    dev = H.to_device(wl, inputs)
    st = mem.new_state(torch.from_numpy(w0))
    out = H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert mem.device_errors() == 0   # the pair's waits all completed
    st_g = H.gpu_state_np(mem, st)
    out_g = out.float().cpu().numpy()
    from oracle import oracle as O
    out_o, st_o, _ = O.run_workload(wl, inputs, w0)
    r = H.compare(wl, inputs, out_g, st_g, out_o, st_o)
    assert np.isfinite(out_g).all()
    tol = H.tol_of(wl)
    for key in ("out", "memory_part", "weights", "momentum"):
        if key in r:
            assert r[key] <= tol, (key, r)
    assert r["halo_exact"] and r["count_exact"], r
    return r


# three full chunks and a ragged tail where the oracle is quick; the
# 128-512-128 memory (about 0.15 s of oracle time per token) over one full
# chunk and a ragged tail
MUON_CASES = [("linear64_delta", 3 * 64 + 17, {}), ("linear_poly2", 3 * 64 + 17, {}), ("mlp64", 3 * 64 + 17, {}),
              ("mlp64", 2 * 64 + 5, {"momentum": False}), ("mlp64", 2 * 64 + 5, {"bias": "dot"}),
              ("mlp64", 2 * 64 + 5, {"window": 8}), ("mlp64", 2 * 64 + 5, {"ns_steps": 2}),
              ("mlp64", 2 * 64 + 5, {"bias": "lp", "bias_p": 3.0}),
              ("mlp64", 2 * 64 + 5, {"bias": "huber", "sign_alpha": 16.0}),
              ("layer_scale", 64 + 9, {}),
              # shapes beyond the workloads': hidden width 2 d, and the window c = 1
              ("layer_scale", 64 + 9, {"hidden": 256}), ("layer_scale", 64 + 9, {"window": 1})]


@pytest.mark.parametrize("recipe", ["preset", "lively"])
@pytest.mark.parametrize("name,n,kw", MUON_CASES)
def test_muon_parity(B, name, n, kw, recipe):
    wl = _muon(name, n, recipe, **kw)
    _say(f"[muon] {name} {kw} {recipe} B=1 H=2 N={n}")
    r = _parity(B, wl)
    _say(f"[muon] {name} {kw} {recipe}: {r}")


def test_muon_wide_feature_map(B):
    """The 688-512-128 memory on [k, poly2(k[:32])] (c = 64): W1's orientation
    has 512 rows, past the LDS path, so Newton-Schulz keeps B and a transposed
    copy of X in the workspace.  One sequence, ten tokens: the oracle needs
    about 4 s per token of this memory."""
    wl = replace(lively(WORKLOADS["atlas_long"]).with_shape(batch=1, heads=1, seq_len=10), optimizer="muon")
    _say("[muon] atlas_long B=1 H=1 N=10")
    r = _parity(B, wl)
    _say(f"[muon] atlas_long: {r}")


def test_muon_split_is_bitwise_equal(B):
    """Two calls with a chunk-aligned split equal one call, bit for bit: the
    Muon momentum lives in the state's momentum slot."""
    binding, H = B
    n = 2 * 64 + 5
    wl = _muon("mlp64", n, "lively")
    _say("[muon split] mlp64")
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    one = binding.AtlasMem(wl)
    st1 = one.new_state(torch.from_numpy(w0))
    out1 = H.gpu_run(one, wl, dev, st1)
    n1 = 64
    wa, wb = wl.with_shape(seq_len=n1), wl.with_shape(seq_len=n - n1)
    ma, mb = binding.AtlasMem(wa), binding.AtlasMem(wb)
    st2 = ma.new_state(torch.from_numpy(w0))
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    da = {k_: part(t, 0, n1) for k_, t in dev.items()}
    db = {k_: part(t, n1, n) for k_, t in dev.items()}
    oa = H.gpu_run(ma, wa, da, st2)
    ob = H.gpu_run(mb, wb, db, st2)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=2), out1)
    assert torch.equal(st1, st2)


def test_muon_theta_zero_keeps_weights_and_alpha_one_erases(B):
    """alpha = theta = 0: the weights never move (the momentum still
    accumulates); alpha = 1, theta = 0: the weights are zero after the first
    token, so y is the residual alone."""
    binding, H = B
    wl = _muon("mlp64", 64 + 7, "lively")
    inputs, w0 = H.prepare(wl)
    inputs = dict(inputs)
    inputs["theta"] = np.zeros_like(inputs["theta"])
    inputs["alpha"] = np.zeros_like(inputs["alpha"])
    dev = H.to_device(wl, inputs)
    mem = binding.AtlasMem(wl)
    st = mem.new_state(torch.from_numpy(w0))
    H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert torch.equal(mem.view(st, "weights").cpu(), torch.from_numpy(w0).float())
    inputs["alpha"] = np.ones_like(inputs["alpha"])
    dev = H.to_device(wl, inputs)
    st = mem.new_state(torch.from_numpy(w0))
    out = H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert not mem.view(st, "weights").any()
    assert torch.equal(out.cpu(), dev["q"].cpu())



def test_muon_bench_shape_sampled(B):
    """The benchmark's Muon launch: all 96 sequences of the 128-512-128
    memory (8 x 12 heads, c = 32) in one call, here of one chunk and a
    ragged tail; the oracle replays three sequences (first, middle, last),
    outputs and final weights and momentum."""
    binding, H = B
    n = 64 + 9
    wl = replace(WORKLOADS["layer_scale"].with_shape(seq_len=n), optimizer="muon")
    _say(f"[muon full grid] layer_scale B={wl.batch} H={wl.heads} N={n}")
    inputs, w0 = H.prepare(wl)
    mem = binding.AtlasMem(wl)
    dev = H.to_device(wl, inputs)
    st = mem.new_state(torch.from_numpy(w0))
    out = H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert mem.device_errors() == 0
    seqs = [0, 47, 95]
    from oracle import oracle as O
    out_o, st_o, _ = O.run_workload(wl, inputs, w0, seqs=seqs)
    r = H.compare(wl, inputs, out.float().cpu().numpy(), H.gpu_state_np(mem, st), out_o, st_o, seqs=seqs)
    _say(f"[muon full grid] {r}")
    for key in ("out", "memory_part", "weights", "momentum"):
        assert r[key] <= H.tol_of(wl), (key, r)
    assert r["halo_exact"] and r["count_exact"], r


@pytest.mark.parametrize("n", [0, 1, 37])
def test_muon_short_and_empty_calls(B, n):
    """Calls shorter than one chunk (and the empty call, which leaves the
    state as it is) on the pair of workgroups (64-256-64) and on the linear
    memory."""
    binding, H = B
    for name in ("mlp64", "linear_poly2"):
        wl = _muon(name, n, "lively")
        _say(f"[muon short] {name} N={n}")
        if n == 0:
            inputs, w0 = H.prepare(wl.with_shape(seq_len=1))
            mem = binding.AtlasMem(wl)
            st = mem.new_state(torch.from_numpy(w0))
            before = st.clone()
            dev = H.to_device(wl.with_shape(seq_len=1), inputs)
            out = torch.empty(wl.batch, wl.heads, 0, wl.d_v, dtype=mem.io_dtype, device="cuda")
            mem.forward(dev["q"][:, :, :0], dev["k"][:, :, :0], dev["v"][:, :, :0], dev["alpha"][:, :, :0],
                        dev["eta"][:, :, :0], dev["theta"][:, :, :0], dev["gamma"][:, :, :0], st, out)
            torch.cuda.synchronize()
            assert torch.equal(st, before)
            continue
        _parity(B, wl)
