"""The Huber bias makes a discrete choice per token (|e|_2 <= delta).  The
GPU takes it on bf16/fp32 arithmetic, the oracle in fp64; they agree when no
token's error norm lies near its threshold.  The synthetic thresholds
(delta_t = 1/4 or 4 times |v_t|_2) keep every choice of the parity cases at
least a factor 2 away from the boundary; this replays those cases on the
oracle chunk by chunk and checks it, and that both branches occur."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import oracle as O
from test_memorization_sequence_amd import synth
from test_memorization_sequence_amd.configs import WORKLOADS, lively

N = 3 * 64 + 17


@pytest.mark.parametrize("recipe", ["preset", "lively"])
@pytest.mark.parametrize("name", ["linear_poly2", "mlp64", "layer_scale"])
def test_huber_choices_are_far_from_the_threshold(name, recipe):
    wl = replace(WORKLOADS[name], bias="huber").with_shape(batch=1, heads=2, seq_len=N)
    if recipe == "lively":
        wl = lively(wl)
    inp = synth.make_inputs(wl, 0)
    w0 = synth.initial_weights_flat(wl, inp)
    cfg = O.config_for(wl)
    cfg.n_seq = 1
    worst, small, large = np.inf, 0, 0
    for s in range(2):
        st = O.empty_state(cfg)
        st["mem"][0] = w0[s]
        g = lambda key: np.ascontiguousarray(inp[key].reshape(2, N, *inp[key].shape[3:])[s:s + 1], dtype=np.float64)
        q, k, v, al, et, th, ga, dl = (g(x) for x in ("q", "k", "v", "alpha", "eta", "theta", "gamma", "delta"))
        for t0 in range(0, N, wl.chunk):
            te = min(N, t0 + wl.chunk)
            W = st["mem"][0].copy()
            for i in range(max(0, t0 - wl.window + 1), te):
                f = O.memory_apply(cfg, W, O.phi(cfg, k[0, i]), k[0, i])
                ratio = np.linalg.norm(f - v[0, i]) / dl[0, i]
                worst = min(worst, abs(np.log(ratio)))
                small += ratio <= 1
                large += ratio > 1
            sl = slice(t0, te)
            O.forward(cfg, q[:, sl], k[:, sl], v[:, sl], al[:, sl], et[:, sl], th[:, sl], ga[:, sl], st,
                      delta=dl[:, sl])
    assert worst > np.log(2.0), worst
    assert small > 50 and large > 50, (small, large)
