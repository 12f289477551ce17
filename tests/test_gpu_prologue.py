"""Parity of the fused prologue (GPU, through the C ABI) with its fp64
oracle.  Relative L2 <= 2e-2 on q, k, v (bf16 outputs) and on the gates."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    return np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b)


def _run(B, N, dm, H, d, K=4, r=16, seed=0):
    from test_memorization_sequence_amd import binding, synth
    inp = synth.make_prologue_inputs(B, N, dm, H, d, K, r, seed)
    dev = lambda a, dt: torch.from_numpy(a).to("cuda", dtype=dt).contiguous()
    x, w = dev(inp["x"], torch.bfloat16), dev(inp["w"], torch.bfloat16)
    wc, gv, gb = dev(inp["w_conv"], torch.float32), dev(inp["gate_v"], torch.float32), dev(inp["gate_b"], torch.float32)
    q, k, v = [torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    gates = [torch.empty(B, H, N, dtype=torch.float32, device="cuda") for _ in range(4)]
    pro = binding.AtlasPrologue(B, N, dm, H, d, K, r)
    pro.forward(x, w, wc, gv, gb, q, k, v, *gates)
    torch.cuda.synchronize()
    outs = [t.float().cpu().numpy() for t in (q, k, v)] + [np.stack([g.cpu().numpy() for g in gates])]
    return inp, outs


@pytest.mark.parametrize("B,N,dm,H,d,K,r", [(2, 37, 256, 2, 128, 4, 16), (3, 70, 192, 3, 64, 3, 8),
                                            (1, 5, 512, 2, 256, 8, 4), (2, 1, 128, 1, 128, 4, 1)])
def test_prologue_parity_small(B, N, dm, H, d, K, r):
    from oracle import prologue as PR
    _say(f"[prologue] B={B} N={N} d_model={dm} H={H} d={d} K={K} r={r}")
    inp, outs = _run(B, N, dm, H, d, K, r)
    want = PR.prologue(inp["x"], inp["w"], inp["w_conv"], inp["gate_v"], inp["gate_b"], H, d, r)
    errs = [rel_l2(o, w_) for o, w_ in zip(outs, want)]
    _say(f"[prologue] relL2 q,k,v,gates = {errs}")
    assert all(e <= 2e-2 for e in errs), errs


def test_prologue_parity_layer_scale_shape_sampled():
    """The layer-scale shape (8 x 16384 tokens, d_model 1536 = 12 heads x 128),
    checked on the first 64 tokens of the first and the last sequence: the
    prologue is causal and keeps sequences apart, so the oracle on those
    prefixes alone gives the exact expected values."""
    from oracle import prologue as PR
    B, N, dm, H, d = 8, 16384, 1536, 12, 128
    _say(f"[prologue] layer-scale shape B={B} N={N}")
    inp, outs = _run(B, N, dm, H, d)
    n = 64
    for b in (0, B - 1):
        want = PR.prologue(inp["x"][b:b + 1, :n], inp["w"], inp["w_conv"], inp["gate_v"], inp["gate_b"], H, d, 16)
        got = [o[b:b + 1, :, :n] for o in outs[:3]] + [outs[3][:, b:b + 1, :, :n]]
        errs = [rel_l2(o, w_) for o, w_ in zip(got, want)]
        _say(f"[prologue] sequence {b}: relL2 q,k,v,gates = {errs}")
        assert all(e <= 2e-2 for e in errs), errs
    assert all(np.isfinite(o).all() for o in outs)
