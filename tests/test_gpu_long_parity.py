"""Parity over the workloads' full lengths (needs an MI355X).

The chunk chain is sequential (ATLAS review, sec. 3.3 "Parallelizing Omega
Rule": every chunk starts from the state the previous chunk left), so the bf16
rounding of each chunk's operands feeds every later chunk.  These tests run
each workload at its full shape, in the launch configuration the benchmark
times (AUTO family, all sequences in one call), and replay sampled sequences
on the fp64 oracle over the whole call (atlas_long: over its first 8192
tokens, with the GPU call split there; a chunk-aligned split equals one call
bit for bit).  Checked, against the same tolerance as every other parity test
(relative L2 2e-2 for bf16 io, 1e-4 for fp32 io):

  * the outputs, as one tensor, per sequence (the maximum), and per chunk of
    every sampled sequence (the curve is printed; its maximum is asserted);
  * the memory's own contribution y - r (residual MLPs): as one tensor with
    the bf16 rounding of y not charged, and per chunk without that discount
    wherever the contribution is at least 100 times that rounding;
  * the final weights and momentum of the sampled sequences.

Both recipes run: the workload's own gates, and the lively ones (small decay)
under which the memory keeps changing over the whole sequence.
"""
import sys

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


# workload -> (sampled sequences, tokens the oracle replays: None = all)
LONG = {
    "linear64_delta": (None, None),
    "linear_poly2": (None, None),
    "mlp64": ([0, 9, 22, 37, 41, 50, 58, 63], None),
    "layer_scale": ([0, 95], None),
    "atlas_long": ([5], 8192),
}


def chunk_curve(y, y_or, chunk):
    """[n_seq, n_chunks] relative L2 of every chunk of every sequence."""
    S, n, dv = y_or.shape
    nc = -(-n // chunk)
    out = np.zeros((S, nc))
    for j in range(nc):
        a = y[:, j * chunk:(j + 1) * chunk].reshape(S, -1)
        b = y_or[:, j * chunk:(j + 1) * chunk].reshape(S, -1)
        den = np.linalg.norm(b, axis=1)
        out[:, j] = np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)
    return out


@pytest.mark.parametrize("recipe", ["preset", "lively"])
@pytest.mark.parametrize("name", list(LONG))
def test_full_length_parity(B, name, recipe):
    binding, H = B
    from oracle import oracle as O
    wl = WORKLOADS[name]
    if recipe == "lively":
        wl = lively(wl)
    seqs, n_or = LONG[name]
    S, N = wl.batch * wl.heads, wl.seq_len
    seqs = list(range(S)) if seqs is None else seqs
    n_or = N if n_or is None else n_or
    _say(f"[long] {name} {recipe}: B={wl.batch} H={wl.heads} N={N}; oracle replays seqs {seqs} x {n_or} tokens")
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    # one call over all N tokens, or two chunk-aligned calls split at n_or
    parts = [(0, N)] if n_or == N else [(0, n_or), (n_or, N)]
    st = None
    outs, snap = [], None
    for a, b in parts:
        wp = wl.with_shape(seq_len=b - a)
        mem = binding.AtlasMem(wp)
        if st is None:
            st = mem.new_state(torch.from_numpy(w0))
        d = {k_: t[:, :, a:b].contiguous() for k_, t in dev.items()}
        outs.append(H.gpu_run(mem, wp, d, st))
        torch.cuda.synchronize()
        assert mem.device_errors() == 0
        if b == n_or:
            snap = H.gpu_state_np(mem, st)
        family = mem.family()
    out_g = torch.cat(outs, dim=2).float().cpu().numpy().reshape(S, N, wl.d_v)
    assert np.isfinite(out_g).all()
    del dev, outs
    _say(f"[long] {name} {recipe}: GPU done ({family}); oracle ...")
    out_o, st_o, used = O.run_workload(wl, inputs, w0, seqs=seqs, n_tokens=n_or)
    _say(f"[long] {name} {recipe}: oracle done on {used} threads")
    y = out_g[seqs, :n_or].astype(np.float64)
    tol = H.tol_of(wl)
    r = H.compare(wl, inputs, out_g, snap, out_o, st_o, seqs=seqs, n_tokens=n_or)
    per_seq = [H.rel_l2(y[i], out_o[i]) for i in range(len(seqs))]
    curve = chunk_curve(y, out_o, wl.chunk)
    worst = np.unravel_index(np.argmax(curve), curve.shape)
    _say(f"[long] {name} {recipe}: {r}")
    _say(f"[long] {name} {recipe}: per-sequence max {max(per_seq):.3e}; per-chunk max {curve.max():.3e} "
         f"(sequence {seqs[worst[0]]}, chunk {worst[1]} of {curve.shape[1]})")
    _say(f"[long] {name} {recipe}: per-chunk curve of sequence {seqs[0]} (every 8th chunk): "
         + " ".join(f"{x:.1e}" for x in curve[0, ::8]))
    assert r["out"] <= tol, r
    assert max(per_seq) <= tol, per_seq
    assert curve.max() <= tol, (curve.max(), worst)
    for key in ("memory_part", "weights", "momentum"):
        if key in r:
            assert r[key] <= tol, (key, r)
    assert r["halo_exact"] and r["count_exact"], r
    if wl.memory == "mlp" and wl.residual:
        # per chunk, no rounding discount, where the memory's own part is
        # at least 100 times the bf16 rounding of y
        from test_memorization_sequence_amd import synth
        rr = inputs["q"].reshape(S, N, wl.d_k)[seqs, :n_or].astype(np.float64)
        checked, worst_mp = 0, 0.0
        for i in range(len(seqs)):
            for j in range(0, n_or, wl.chunk):
                sl = slice(j, j + wl.chunk)
                m = out_o[i, sl] - rr[i, sl]
                quant = np.linalg.norm(synth.round_to_bf16(out_o[i, sl].astype(np.float32)) - out_o[i, sl])
                if quant > 0 and np.linalg.norm(m) >= 100.0 * quant:
                    checked += 1
                    e = H.rel_l2(y[i, sl] - rr[i, sl], m)
                    worst_mp = max(worst_mp, e)
        _say(f"[long] {name} {recipe}: memory part checked raw on {checked} chunks, worst {worst_mp:.3e}")
        assert worst_mp <= tol
        if recipe == "lively":
            assert checked > 0, "the lively recipe keeps the memory's part well above the rounding of y"
