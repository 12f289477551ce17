"""Parity over the workloads' full lengths (needs an MI355X).

The chunk chain is sequential (ATLAS review, sec. 3.3 "Parallelizing Omega
Rule": every chunk starts from the state the previous chunk left), so the bf16
rounding of each chunk's operands feeds every later chunk.  These tests run
each workload at its full shape, in the launch configuration the benchmark
times (AUTO family, all sequences in one call), and replay sampled sequences
on the fp64 oracle over the whole call (atlas_long: over a prefix, with the
GPU call split there; a chunk-aligned split equals one call bit for bit).
Checked, against the same tolerance as every other parity test (relative L2
2e-2 for bf16 io, 1e-4 for fp32 io):

  * the outputs, as one tensor, per sequence (the maximum), and per chunk of
    every sampled sequence (the curve is printed; its maximum is asserted);
  * the memory's own contribution y - r (residual MLPs): as one tensor with
    the bf16 rounding of y not charged, and per chunk without that discount
    wherever the contribution is at least 100 times that rounding;
  * the final weights and momentum of the sampled sequences.  Under the
    workloads' own gates the MLP memories decay towards the W = 0 fixed point
    (by about 27 orders of magnitude over mlp64's 8192 tokens), where the
    relative error of the remainder is ill-conditioned: half a bf16 ulp of
    noise on the keys moves the fp64 oracle's own final weights by up to
    4 % (tests/test_decay_conditioning.py measures it).  The state is
    therefore judged against max(|W_oracle|, 1e-3 |W_0|): relative while the
    weights keep at least a thousandth of their initial size, and as an
    absolute error at that level once they have decayed below it.

Both recipes run: the workloads' own gates, and the lively ones (small decay)
under which the MLP memory keeps learning.  Over long horizons the lively MLP
memory is dynamically unstable: its weights grow until the step overshoots,
and the fp64 oracle itself diverges to inf/NaN on 5 of mlp64's 64 sequences,
71 of layer_scale's 96 and all 8 of atlas_long's within their lengths, while
a bounded trajectory amplifies any perturbation steadily.  A replay from the
first token then compares two chaotic trajectories, not two implementations.
So the lively MLP runs are checked by shadowing: the GPU call is split into
segments of 16 chunks (a chunk-aligned split equals one call bit for bit),
and every segment is replayed by the oracle from the GPU's own state at the
segment's start.  Each segment is judged over the chunks on which the oracle
is conditioned at the GPU's precision: a second oracle replay, with its state
multiplied by 1 + u 2^-6 (u uniform in [-1, 1]) at every chunk boundary, must
agree with the first to within half the tolerance (the end state is compared where they agree to
within a quarter of it over the whole segment).  The GPU rounds about a
dozen operand tensors of every chunk to bf16 (keys, queries, weight and
momentum images, activations, errors, gate products), each by up to half an
ulp (2^-9); state noise of eight half-ulps reproduces the size of the GPU's
error both on ordinary segments (measured 2-5e-3 against 4-8e-3 for the
model) and at the onset of a divergence (5e-2 against 6e-2).
Segments that start after the GPU trajectory has left the bounded regime
(non-finite, or weights above 100 times their initial norm) are not replayed;
the coverage is printed and must include every segment of the sequences
sampled from those the GPU keeps bounded.
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


# workload -> recipe -> (sampled sequences (None: all), tokens the oracle replays (None: all))
LONG = {
    "linear64_delta": {"preset": (None, None), "lively": (None, None)},
    "linear_poly2": {"preset": (None, None), "lively": (None, None)},
    "mlp64": {"preset": (None, None)},
    "layer_scale": {"preset": ([0, 95], None)},
    "atlas_long": {"preset": ([5], 8192)},
}
FULL_CASES = [(n, r) for n in LONG for r in LONG[n]]

# lively MLP runs, shadowed: workload -> (sampled sequences (None: all), tokens per call)
SHADOW = {
    "mlp64": (None, None),
    "layer_scale": ([1, 6, 12], None),
    "atlas_long": ([4, 7], 8192),
}
SEG_CHUNKS = 16


def chunk_curve(y, y_or, chunk):
    """[n_seq, n_chunks] relative L2 of every chunk of every sequence."""
    S, n, dv = y_or.shape
    nc = -(-n // chunk)
    out = np.zeros((S, nc))
    for j in range(nc):
        a = y[:, j * chunk:(j + 1) * chunk].reshape(S, -1)
        b = y_or[:, j * chunk:(j + 1) * chunk].reshape(S, -1)
        with np.errstate(all="ignore"):
            den = np.linalg.norm(b, axis=1)
            out[:, j] = np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)
    return np.where(np.isfinite(out), out, np.inf)


@pytest.mark.parametrize("name,recipe", FULL_CASES)
def test_full_length_parity(B, name, recipe):
    binding, H = B
    from oracle import oracle as O
    wl = WORKLOADS[name]
    if recipe == "lively":
        wl = lively(wl)
    seqs, n_or = LONG[name][recipe]
    S, N = wl.batch * wl.heads, wl.seq_len
    seqs = list(range(S)) if seqs is None else seqs
    n_or = N if n_or is None else n_or
    nch = -(-n_or // wl.chunk)
    _say(f"[long] {name} {recipe}: B={wl.batch} H={wl.heads} N={N}; oracle replays seqs {seqs[:16]} x {n_or} tokens")
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
    n_bad_gpu = int((~np.isfinite(out_g).all(axis=(1, 2))).sum())
    del dev, outs
    _say(f"[long] {name} {recipe}: GPU done ({family}), {n_bad_gpu} of {S} sequences non-finite; oracle ...")
    out_o, st_o, used = O.run_workload(wl, inputs, w0, seqs=seqs, n_tokens=n_or)
    _say(f"[long] {name} {recipe}: oracle done on {used} threads")
    tol = H.tol_of(wl)

    horizon = np.full(len(seqs), nch)
    full = list(range(len(seqs)))

    y = out_g[seqs, :n_or].astype(np.float64)
    curve = chunk_curve(y, out_o, wl.chunk)
    mask = np.arange(nch)[None, :] < horizon[:, None]
    judged = np.where(mask, curve, 0.0)
    worst = np.unravel_index(np.argmax(judged), judged.shape)
    # whole tensor and per sequence over the conditioned chunks
    sel = np.repeat(mask, wl.chunk, axis=1)[:, :n_or]
    dif = np.where(sel[..., None], y - out_o, 0.0)
    ref = np.where(sel[..., None], out_o, 0.0)
    rel_all = float(np.linalg.norm(dif) / np.linalg.norm(ref))
    per_seq = np.linalg.norm(dif.reshape(len(seqs), -1), axis=1) / np.linalg.norm(ref.reshape(len(seqs), -1), axis=1)
    _say(f"[long] {name} {recipe}: out rel {rel_all:.3e}; per-sequence max {per_seq.max():.3e}; per-chunk max "
         f"{judged.max():.3e} (sequence {seqs[worst[0]]}, chunk {worst[1]} of {nch})")
    _say(f"[long] {name} {recipe}: per-chunk curve of sequence {seqs[0]} (every 8th chunk): "
         + " ".join(f"{x:.1e}" for x in curve[0, ::8]))
    assert np.isfinite(y[sel]).all()
    assert rel_all <= tol and per_seq.max() <= tol and judged.max() <= tol

    # state, on the sequences conditioned over the whole call
    if full:
        fs = [seqs[i] for i in full]
        st_f = {key: val[full] for key, val in st_o.items()}
        r = H.compare(wl, inputs, out_g, snap, out_o[full], st_f, seqs=fs, n_tokens=n_or)
        w0s = np.asarray(w0, dtype=np.float64)[fs]
        floor = 1e-3 * np.linalg.norm(w0s, axis=1)
        for key, g_key in (("mem", "weights"), ("mom", "momentum")):
            if g_key not in r:
                continue
            num = np.linalg.norm(snap[g_key][fs] - st_f[key], axis=1)
            den = np.maximum(np.linalg.norm(st_f[key], axis=1), floor)
            r[g_key + "_floored"] = float(np.sqrt(np.sum(num ** 2)) / max(np.sqrt(np.sum(den ** 2)), 1e-300))
        decay = (" |W_oracle| / |W_0| = " + " ".join(f"{x:.1e}" for x in (np.linalg.norm(st_f["mem"], axis=1)
                                                                          / np.linalg.norm(w0s, axis=1))[:8])
                 if np.linalg.norm(w0s) > 0 else "")
        _say(f"[long] {name} {recipe}: state of {len(fs)} sequences: {r};" + decay)
        for key in ("memory_part", "weights_floored", "momentum_floored"):
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
            for j in range(horizon[i]):
                sl = slice(j * wl.chunk, (j + 1) * wl.chunk)
                m = out_o[i, sl] - rr[i, sl]
                quant = np.linalg.norm(synth.round_to_bf16(out_o[i, sl].astype(np.float32)) - out_o[i, sl])
                if quant > 0 and np.linalg.norm(m) >= 100.0 * quant:
                    checked += 1
                    worst_mp = max(worst_mp, H.rel_l2(y[i, sl] - rr[i, sl], m))
        _say(f"[long] {name} {recipe}: memory part checked raw on {checked} chunks, worst {worst_mp:.3e}")
        assert worst_mp <= tol


def _segment_state(snap, i, wl):
    """The oracle's state dict (one sequence) from a GPU state snapshot row."""
    c1 = wl.window - 1
    st = {"mem": snap["weights"][i][None].copy(),
          "mom": snap["momentum"][i][None].copy() if wl.momentum else np.zeros_like(snap["weights"][i][None]),
          "halo_k": snap["halo_k"][i].reshape(1, c1, wl.d_k).copy(),
          "halo_v": snap["halo_v"][i].reshape(1, c1, wl.d_v).copy(),
          "halo_g": snap["halo_g"][i].reshape(1, c1).copy(),
          "halo_d": np.zeros((1, c1)),
          "count": snap["count"][i].reshape(1).astype(np.int64).copy()}
    return st


@pytest.mark.parametrize("name", list(SHADOW))
def test_lively_shadowed_segments(B, name):
    binding, H = B
    from oracle import oracle as O
    wl = lively(WORKLOADS[name])
    seqs, n_call = SHADOW[name]
    S, N = wl.batch * wl.heads, wl.seq_len
    n_call = N if n_call is None else n_call
    seqs = list(range(S)) if seqs is None else seqs
    L = SEG_CHUNKS * wl.chunk
    assert n_call % L == 0
    nseg = n_call // L
    tol = H.tol_of(wl)
    _say(f"[shadow] {name} lively: B={wl.batch} H={wl.heads}, {n_call} tokens in {nseg} segments of {L}; "
         f"sequences {seqs[:16]}")
    inputs, w0 = H.prepare(wl)
    dev = H.to_device(wl, inputs)
    ws = wl.with_shape(seq_len=L)
    mem = binding.AtlasMem(ws)
    st = mem.new_state(torch.from_numpy(w0))
    snaps, outs = [], []
    take = lambda snap: {key: val[seqs] for key, val in snap.items()}
    for j in range(nseg):
        snaps.append(take(H.gpu_state_np(mem, st)))
        outs.append(H.gpu_run(mem, ws, {k_: t[:, :, j * L:(j + 1) * L].contiguous() for k_, t in dev.items()}, st))
    torch.cuda.synchronize()
    assert mem.device_errors() == 0
    snaps.append(take(H.gpu_state_np(mem, st)))
    out_seg = torch.cat(outs, dim=2)
    # the segments are the trajectory of one call, bit for bit
    wo = wl.with_shape(seq_len=n_call)
    one = binding.AtlasMem(wo)
    st1 = one.new_state(torch.from_numpy(w0))
    out1 = H.gpu_run(one, wo, {k_: t[:, :, :n_call].contiguous() for k_, t in dev.items()}, st1)
    torch.cuda.synchronize()
    # (bitwise: diverged sequences hold NaN)
    assert torch.equal(out1.view(torch.int16), out_seg.view(torch.int16)) and torch.equal(st1, st)
    del dev, out1, outs
    y_all = out_seg.float().cpu().numpy().reshape(S, n_call, wl.d_v)[seqs].astype(np.float64)
    family = mem.family()

    # segments the GPU keeps in the bounded regime
    w0n = np.linalg.norm(np.asarray(w0, dtype=np.float64)[seqs], axis=1)
    jobs = []
    for i in range(len(seqs)):
        for j in range(nseg):
            wn = np.linalg.norm(snaps[j]["weights"][i])
            seg_y = y_all[i, j * L:(j + 1) * L]
            if np.isfinite(wn) and wn <= 100.0 * w0n[i] and np.isfinite(seg_y).all():
                jobs.append((i, j))
    _say(f"[shadow] {name}: GPU done ({family}); replaying {len(jobs)} of {len(seqs) * nseg} segments on the oracle")

    def replay(noisy):
        """Every job's segment on the oracle from the GPU's state at its start;
        noisy: the state is multiplied by 1 + u 2^-6 (u uniform in [-1, 1])
        at every chunk boundary, a perturbation of the size of the GPU's own
        rounding."""
        cfg = O.config_for(wl)
        flat = lambda a, i, j: a.reshape(S, N, *a.shape[3:])[seqs[i], j * L:(j + 1) * L]
        ins = {key: np.stack([flat(inputs[key], i, j) for i, j in jobs]).astype(np.float64)
               for key in ("q", "k", "v", "alpha", "eta", "theta", "gamma")}
        parts = [_segment_state(snaps[j], i, wl) for i, j in jobs]
        state = {key: np.ascontiguousarray(np.concatenate([p_[key] for p_ in parts])) for key in parts[0]}
        if not noisy:
            out, _ = O.forward(cfg, *(ins[key] for key in ("q", "k", "v", "alpha", "eta", "theta", "gamma")), state)
            return out, state
        rng = np.random.default_rng(1)
        outs = []
        for t in range(SEG_CHUNKS):
            for key in ("mem", "mom"):
                state[key] *= 1.0 + rng.uniform(-1.0, 1.0, state[key].shape) * 2.0 ** -6
            cut = {key: np.ascontiguousarray(a[:, t * wl.chunk:(t + 1) * wl.chunk]) for key, a in ins.items()}
            o, _ = O.forward(cfg, *(cut[key] for key in ("q", "k", "v", "alpha", "eta", "theta", "gamma")), state)
            outs.append(o)
        return np.concatenate(outs, axis=1), state

    out_o, st_o = replay(False)
    out_p, _ = replay(True)
    _say(f"[shadow] {name}: oracle done")

    from test_memorization_sequence_amd import synth
    judged_chunks, state_checked, worst, worst_at, worst_state, mp_checked, worst_mp = 0, 0, 0.0, None, 0.0, 0, 0.0
    horizons = []
    for n_job, (i, j) in enumerate(jobs):
        yg = y_all[i, j * L:(j + 1) * L][None]
        yo, yp = out_o[n_job][None], out_p[n_job][None]
        sens = chunk_curve(yp, yo, wl.chunk)[0]
        over = np.nonzero(sens > tol / 2)[0]
        h = int(over[0]) if over.size else SEG_CHUNKS
        horizons.append(h)
        cur = chunk_curve(yg, yo, wl.chunk)[0][:h]
        judged_chunks += h
        if h and cur.max() > worst:
            worst, worst_at = float(cur.max()), (seqs[i], j * SEG_CHUNKS + int(np.argmax(cur)))
        r_ = inputs["q"].reshape(S, N, wl.d_k)[seqs[i], j * L:(j + 1) * L].astype(np.float64)
        for t in range(h):
            sl = slice(t * wl.chunk, (t + 1) * wl.chunk)
            m = yo[0, sl] - r_[sl]
            quant = np.linalg.norm(synth.round_to_bf16(yo[0, sl].astype(np.float32)) - yo[0, sl])
            if quant > 0 and np.linalg.norm(m) >= 100.0 * quant:
                mp_checked += 1
                worst_mp = max(worst_mp, H.rel_l2(yg[0, sl] - r_[sl], m))
        floor = 1e-3 * w0n[i]
        keys = (("mem", "weights"), ("mom", "momentum")) if wl.momentum else (("mem", "weights"),)
        rel_state = lambda a, o: float(np.linalg.norm(a - o) / max(np.linalg.norm(o), floor))
        # the end state where the whole segment is well inside its conditioning
        if h == SEG_CHUNKS and sens.max() <= tol / 4:
            state_checked += 1
            for key, g_key in keys:
                worst_state = max(worst_state, rel_state(snaps[j + 1][g_key][i], st_o[key][n_job]))
    total = len(jobs) * SEG_CHUNKS
    _say(f"[shadow] {name}: segment horizons (chunks of {SEG_CHUNKS}): " + " ".join(str(h) for h in horizons[:128]))
    _say(f"[shadow] {name}: judged {judged_chunks} of {total} replayed chunks; outputs per chunk worst {worst:.3e} "
         f"at (sequence, chunk) {worst_at}; end-of-segment state on {state_checked} segments, worst {worst_state:.3e}; "
         f"memory part raw on {mp_checked} chunks, worst {worst_mp:.3e}")
    assert worst <= tol and worst_state <= tol and worst_mp <= tol
    assert judged_chunks >= 0.5 * total and mp_checked > 0
