"""The linear memory on the precomputed-phi family (one recurrence workgroup
per sequence, the retrieval of every chunk at once), against the fp64 oracle
(needs an MI355X).

Shapes: the poly2 map on 32-dim keys (560 features, the linear_poly2 preset)
with windows c = 16 (96 window rows) and c = 40 (128 rows), and the identity
map on 64-dim keys in bf16 with c = 1 (64 rows).  Tolerance: relative L2
2e-2 (bf16 io) on the outputs, final weights and momentum; halo and count
exact.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

from test_memorization_sequence_amd.configs import WORKLOADS, lively

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SMALL_N = 3 * 64 + 17


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


def _wl(shape, **kw):
    if shape == "poly2":
        wl = WORKLOADS["linear_poly2"]
    elif shape == "poly2_c40":
        wl = replace(WORKLOADS["linear_poly2"], window=40, theta_div=40.0)
    else:   # identity 64x64 in bf16, c = 1
        wl = replace(WORKLOADS["linear64_delta"], io_dtype="bf16")
    return replace(wl, **kw)


def _run(B, wl, kernel="grouped", seqs=None, n_tokens=None):
    binding, H = B
    inputs, w0 = H.prepare(wl)
    mem = binding.AtlasMem(wl, kernel)
    assert mem.family() == kernel
    dev = H.to_device(wl, inputs)
    st = mem.new_state(torch.from_numpy(w0))
    out = H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert mem.device_errors() == 0
    from oracle import oracle as O
    out_o, st_o, _ = O.run_workload(wl, inputs, w0, seqs=seqs, n_tokens=n_tokens)
    return inputs, out.float().cpu().numpy(), H.gpu_state_np(mem, st), out_o, st_o


def _check(B, wl, r):
    binding, H = B
    tol = H.tol_of(wl)
    for key in ("out", "weights", "momentum"):
        if key in r:
            assert r[key] <= tol, (key, r)
    assert r["halo_exact"] and r["count_exact"], r


CASES = [(s, rcp, kw) for s in ("poly2", "poly2_c40", "id64") for rcp in ("preset", "lively")
         for kw in ("", "dot", "no_momentum")]


@pytest.mark.parametrize("shape,recipe,variant", CASES)
def test_parity_linear_grouped(B, shape, recipe, variant):
    kw = {"dot": dict(bias="dot"), "no_momentum": dict(momentum=False, eta_u=None), "": {}}[variant]
    wl = _wl(shape, **kw).with_shape(batch=1, heads=3, seq_len=SMALL_N)
    if recipe == "lively":
        wl = replace(wl, alpha_u=(-8.0, -4.0))
    _say(f"[linear] {shape} {recipe} {variant or 'l2'} B=1 H=3 N={SMALL_N}")
    inputs, out_g, st_g, out_o, st_o = _run(B, wl)
    r = B[1].compare(wl, inputs, out_g, st_g, out_o, st_o)
    _say(f"[linear] {shape} {recipe} {variant or 'l2'}: {r}")
    assert np.isfinite(out_g).all()
    _check(B, wl, r)


@pytest.mark.parametrize("n", [0, 1, 37, 64, 65])
@pytest.mark.parametrize("shape", ["poly2", "id64"])
def test_short_and_empty_calls_linear(B, shape, n):
    wl = lively(_wl(shape)).with_shape(batch=1, heads=2, seq_len=n) if shape == "poly2" else \
        replace(_wl(shape), alpha_u=(-8.0, -4.0)).with_shape(batch=1, heads=2, seq_len=n)
    _say(f"[linear short] {shape} N={n}")
    inputs, out_g, st_g, out_o, st_o = _run(B, wl)
    if n == 0:
        assert out_g.size == 0
        np.testing.assert_array_equal(st_g["weights"], st_o["mem"])
        assert (st_g["count"] == 0).all()
        return
    _check(B, wl, B[1].compare(wl, inputs, out_g, st_g, out_o, st_o))


@pytest.mark.parametrize("shape", ["poly2", "poly2_c40", "id64"])
def test_split_is_bitwise_equal_linear(B, shape):
    """Two calls with a chunk-aligned split equal one call, bit for bit (the
    second call's window reaches into the first through the halo)."""
    binding, H = B
    wl = replace(_wl(shape), alpha_u=(-8.0, -4.0)).with_shape(batch=1, heads=2, seq_len=SMALL_N)
    _say(f"[linear split] {shape}")
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    one = binding.AtlasMem(wl, "grouped")
    st1 = one.new_state(torch.from_numpy(w0))
    out1 = H.gpu_run(one, wl, dev, st1)
    n1 = 128
    wa, wb = wl.with_shape(seq_len=n1), wl.with_shape(seq_len=SMALL_N - n1)
    ma, mb = binding.AtlasMem(wa, "grouped"), binding.AtlasMem(wb, "grouped")
    st2 = ma.new_state(torch.from_numpy(w0))
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    oa = H.gpu_run(ma, wa, {k: part(t, 0, n1) for k, t in dev.items()}, st2)
    ob = H.gpu_run(mb, wb, {k: part(t, n1, SMALL_N) for k, t in dev.items()}, st2)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=2), out1)
    assert torch.equal(st1, st2)


def test_deterministic_linear(B):
    binding, H = B
    wl = lively(_wl("poly2")).with_shape(batch=2, heads=3, seq_len=SMALL_N)
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    mem = binding.AtlasMem(wl, "grouped")
    outs, sts = [], []
    for _ in range(2):
        st = mem.new_state(torch.from_numpy(w0))
        outs.append(H.gpu_run(mem, wl, dev, st).clone())
        sts.append(st)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(sts[0], sts[1])


def test_alpha_one_theta_zero_erases_exactly_linear(B):
    """alpha = 1, theta = 0: the memory is exactly zero after the first token
    and every output is exactly zero."""
    binding, H = B
    wl = _wl("poly2").with_shape(batch=1, heads=2, seq_len=SMALL_N)
    inputs, w0 = H.prepare(wl)
    inputs["alpha"][:] = 1.0
    inputs["theta"][:] = 0.0
    dev = H.to_device(wl, inputs)
    mem = binding.AtlasMem(wl, "grouped")
    st = mem.new_state(torch.from_numpy(np.random.default_rng(5).normal(size=w0.shape).astype(np.float32)))
    out = H.gpu_run(mem, wl, dev, st)
    torch.cuda.synchronize()
    assert not out.any()
    assert not mem.view(st, "weights").any()


def test_families_agree_linear(B):
    """The per-sequence and the precomputed-phi kernels give the same result up
    to bf16 rounding order."""
    binding, H = B
    wl = lively(_wl("poly2")).with_shape(batch=2, heads=2, seq_len=SMALL_N)
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    res = {}
    for kernel in ("per_sequence", "grouped"):
        mem = binding.AtlasMem(wl, kernel)
        st = mem.new_state(torch.from_numpy(w0))
        res[kernel] = (H.gpu_run(mem, wl, dev, st).float().cpu().numpy(), mem.view(st, "weights").cpu().numpy())
    torch.cuda.synchronize()
    assert H.rel_l2(res["grouped"][0], res["per_sequence"][0]) <= 2e-2
    assert H.rel_l2(res["grouped"][1], res["per_sequence"][1]) <= 2e-2


def test_full_size_sampled_linear(B):
    """linear_poly2 at its full shape (16 sequences x 4096 tokens) in the
    benchmark's launch; the oracle replays two chunks of the first and last
    sequence."""
    binding, H = B
    wl = WORKLOADS["linear_poly2"]
    S = wl.batch * wl.heads
    seqs, n = [0, S - 1], 2 * wl.chunk
    _say(f"[linear full] linear_poly2 seqs={seqs} n={n}")
    inputs, out_g, _, out_o, _ = _run(B, wl, seqs=seqs, n_tokens=n)
    assert np.isfinite(out_g).all()
    r = B[1].compare(wl, inputs, out_g, None, out_o, None, seqs=seqs, n_tokens=n)
    _say(f"[linear full] {r}")
    assert r["out"] <= B[1].tol_of(wl), r
