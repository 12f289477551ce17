"""Throughput of the test-time memory update + retrieval on one MI355X.

One step = one atlas_mem_forward over the whole batch: every (batch, head)
sequence, all seq_len tokens, through the gate-coefficient kernel and the
recurrent chunk kernel.  Inputs are seeded synthetic tensors already resident
in HBM; each step continues the memory from the previous step's state (the
state is a stream, so no reset is needed and the work per step is fixed).

Prints one JSON line.  `roofline` refers to the recurrent chunk kernel (the
dominant kernel); its duration is measured live with HIP events recorded by
the library around that kernel on the call's stream.  `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "test_memorization_sequence_amd", "csrc")

# HBM bytes per launch of the chunk kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes scaled by a plain-copy calibration (fetch x2.0, write
# x1.0), keyed by the hash of the kernel sources they were taken on.  A
# changed kernel reports null until it is measured again.
MEASURED_TRAFFIC = {
    # (workload, kernel, optimizer, tokens per sequence), l2 bias, plain memory
    ("layer_scale", "stream_mlp_kernel", "gd", 16384): {"src": "c1bb50a4302709b0", "bytes": 76.59e9},
    ("atlas_long", "grouped_kernel", "gd", 32768): {"src": "f796b652af5fe317", "bytes": 27.73e9},
    ("layer_scale", "chunk_kernel", "muon", 64): {"src": "fc044794f9a08d4f", "bytes": 91.9e9},
    ("linear64_delta", "chunk_kernel", "gd", 1024): {"src": "fc044794f9a08d4f", "bytes": 1.67e6},
    # the recurrence and the retrieval after it (the pair the kernel events bracket)
    ("linear_poly2", "linear_rec_kernel", "gd", 4096): {"src": "420997f0416615d7", "bytes": 0.344e9},
    ("mlp64", "sharded_mlp_kernel", "gd", 8192): {"src": "a93810f9f3be7fb4", "bytes": 1.779e9},
}


# translation unit of each recurrent kernel
KERNEL_SOURCE = {"stream_mlp_kernel": "atlas_mem_stream.hip", "sharded_mlp_kernel": "atlas_mem_sharded.hip",
                 "chunk_kernel": "atlas_mem_kernels.hip", "grouped_kernel": "atlas_mem_grouped.hip",
                 "linear_rec_kernel": "atlas_mem_linear.hip"}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the source file that holds the kernel and of every local header
    it includes, directly or not."""
    import hashlib
    import re
    seen, todo = [], [KERNEL_SOURCE[kernel]]
    while todo:
        f = todo.pop(0)
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.append(f)
        with open(os.path.join(CSRC, f)) as fh:
            todo += re.findall(r'#include "([^"]+)"', fh.read())
    m = hashlib.sha1()
    for f in sorted(seen):
        m.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()[:16]


def alg_flops_per_chunk(wl) -> float:
    """FLOPs the method must do per chunk of one sequence (the chunked form;
    per-token weights are never materialised): forward over the window,
    backward, momentum+decay update, the state side of the retrieval and the
    intra-chunk (token x token) terms."""
    b, W, D, dv, h = wl.chunk, wl.chunk + wl.window - 1, wl.feature_dim, wl.d_v, wl.hidden
    f = 2 if wl.momentum else 1
    if wl.memory == "linear":
        return 2 * W * D * dv + f * 2 * W * D * dv + f * 2 * b * D * dv + 2 * b * W * (D + dv)
    P = h * D + dv * h
    return (2 * W * (h * D + dv * h) + 2 * W * dv * h + f * 2 * W * P + f * 2 * b * P
            + 2 * b * W * (D + 2 * h + dv))


def weight_matrices(wl):
    """(rows, cols) of each weight matrix of the memory."""
    D, dv, h = wl.feature_dim, wl.d_v, wl.hidden
    return [(dv, D)] if wl.memory == "linear" else [(h, D), (dv, h)]


def alg_flops_muon(wl, n_tokens: int) -> float:
    """FLOPs of one sequence under the Muon optimizer over n_tokens: the
    window forward and backward at each chunk-start state, and per token the
    window gradient of every matrix (one rank-one term for c = 1, else the
    running sum's entering and leaving terms: 2 or 4 rows cols), ns_steps
    Newton-Schulz steps on the r x n orientation (the symmetric A = X X^T:
    r r n, the symmetric A A: r^3, B X: 2 r r n), the update and the
    retrieval (2 P)."""
    b, W, D, dv, h, c = wl.chunk, wl.chunk + wl.window - 1, wl.feature_dim, wl.d_v, wl.hidden, wl.window
    nch = -(-n_tokens // b)
    if wl.memory == "linear":
        per_chunk = 2 * W * D * dv
    else:
        per_chunk = 2 * W * (h * D + dv * h) + 2 * W * dv * h
    per_token = 0.0
    for rows, cols in weight_matrices(wl):
        r, n = min(rows, cols), max(rows, cols)
        per_token += 2 * min(c, 2) * rows * cols + wl.ns_steps * (3 * r * r * n + r ** 3) + 2 * rows * cols
    return nch * per_chunk + n_tokens * per_token


def alg_bytes_per_head_token(wl) -> int:
    """q, k, v in, out back (io dtype), four fp32 gates."""
    es = 4 if wl.io_dtype == "f32" else 2
    return es * (2 * wl.d_k + 2 * wl.d_v) + 4 * 4


def cpu_baseline(wl, inputs, w0, budget_s: float):
    """The fp64 oracle on a bounded sample: one sequence per thread, the first
    n tokens, n chunk-aligned and sized for about budget_s seconds."""
    from oracle import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(16, os.cpu_count() or 1)
    S = wl.batch * wl.heads
    n_seq = min(S, threads)
    P = wl.hidden * wl.feature_dim + wl.d_v * wl.hidden if wl.memory == "mlp" else wl.d_v * wl.feature_dim
    cost = 2.0 * (wl.window + 8) * P            # flops per head-token, direct window sums
    if wl.optimizer == "muon":                   # plus the per-token Newton-Schulz steps
        cost += sum(wl.ns_steps * (4 * min(r, c) ** 2 * max(r, c) + 2 * min(r, c) ** 3) for r, c in weight_matrices(wl))
    n = int(budget_s * 3.0e9 / cost) // wl.chunk * wl.chunk
    n = max(wl.chunk, min(n, wl.seq_len))
    seqs = [int(s) for s in range(0, S, max(1, S // n_seq))][:n_seq]
    t = time.perf_counter()
    _, _, used = O.run_workload(wl, inputs, w0, seqs=seqs, n_tokens=n, threads=threads)
    dt = time.perf_counter() - t
    head_tokens = len(seqs) * n
    return {
        "value": head_tokens / wl.heads / dt,
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"{len(seqs)} of {S} (batch, head) sequences x first {n} tokens of {wl.name}, "
                  f"fp64, {dt:.1f} s; value counts tokens as positions (head-tokens / {wl.heads})",
        "head_tokens_per_s": head_tokens / dt,
    }


def kernel_name(binding, wl, family):
    """Name of the recurrent kernel a call runs for this workload and family."""
    if family == "auto":
        family = binding.AtlasMem(wl, "auto").family()
    if family == "grouped" and wl.memory == "linear":
        # the events bracket the recurrence and the retrieval that follows it
        return "linear_rec_kernel"
    return {"sharded": "sharded_mlp_kernel", "streamed": "stream_mlp_kernel", "per_sequence": "chunk_kernel",
            "grouped": "grouped_kernel"}[family]


def bench_prologue(args, wl):
    """The prologue on the workload's shape: d_model = heads * d_k, K = 4 taps,
    gate rank 16.  One JSON line.  The default path is one kernel (the
    projection GEMM with the per-token steps applied to each tile on chip),
    timed with HIP events on the call's stream; it is bound by the bf16
    MFMA work of the projections.  The two-kernel path (GEMM into a
    workspace, then the per-token kernel) is timed beside it for reference."""
    import numpy as np
    import torch
    from test_memorization_sequence_amd import binding, synth
    B, N, H, d, K, r = wl.batch, wl.seq_len, wl.heads, wl.d_k, 4, 16
    dm = H * d
    print(f"[bench] prologue of {wl.name}: B={B} N={N} d_model={dm} H={H} d={d}", file=sys.stderr, flush=True)
    inp = synth.make_prologue_inputs(B, N, dm, H, d, K, r, 0)
    dev = lambda a, dt: torch.from_numpy(a).to("cuda", dtype=dt).contiguous()
    x, w = dev(inp["x"], torch.bfloat16), dev(inp["w"], torch.bfloat16)
    wc, gv, gb = dev(inp["w_conv"], torch.float32), dev(inp["gate_v"], torch.float32), dev(inp["gate_b"], torch.float32)
    q, k, v = [torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    gates = [torch.empty(B, H, N, dtype=torch.float32, device="cuda") for _ in range(4)]
    pro = binding.AtlasPrologue(B, N, dm, H, d, K, r)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in evs:
        e.record(stream)
    pro.set_events(*evs)

    def run(steps):
        gemm_ms, kern_ms = [], []
        t0 = time.perf_counter()
        for _ in range(steps):
            pro.forward(x, w, wc, gv, gb, q, k, v, *gates, stream=stream)
            evs[2].synchronize()
            gemm_ms.append(evs[0].elapsed_time(evs[1]))
            kern_ms.append(evs[1].elapsed_time(evs[2]))
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, float(np.mean(gemm_ms)), float(np.mean(kern_ms))

    # the two-kernel path, for reference (a few calls)
    pro.set_fused(False)
    run(1)
    two_ms, two_gemm, two_kern = run(3)
    pro.set_fused(True)
    for _ in range(args.warmup):
        pro.forward(x, w, wc, gv, gb, q, k, v, *gates, stream=stream)
    torch.cuda.synchronize()
    ms, _, k_ms = run(args.steps)
    rows, ncol = B * N, 3 * H * d + 4 * r
    flops = 2.0 * rows * ncol * dm
    hbm_bytes = rows * dm * 2 + ncol * dm * 2 + 3 * rows * H * d * 2 + 4 * rows * H * 4
    res = {
        "metric": "prologue tokens/sec (1 GPU): x -> q, k, v, gates",
        "value": rows / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy)",
        "config": {"workload": f"prologue of {wl.name}", "batch": B, "seq_len": N, "d_model": dm, "heads": H,
                   "d_head": d, "conv_taps": K, "gate_rank": r},
        "roofline": {"bound": "mfma", "kernel": "fused_prologue_kernel", "achieved": flops / (k_ms * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "traffic": None,
                     "alg_flops_per_launch": flops, "kernel_ms": k_ms,
                     "alg_hbm_bytes_per_launch": hbm_bytes, "hbm_GBps": hbm_bytes / (k_ms * 1e-3) / 1e9},
        "two_kernel_path": {"ms_per_step": two_ms, "gemm_ms": two_gemm, "kernel_ms": two_kern,
                            "gemm_tflops": flops / (two_gemm * 1e-3) / 1e12},
    }
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer_scale")
    ap.add_argument("--kernel", default="auto", choices=["auto", "per_sequence", "sharded", "streamed", "grouped"])
    ap.add_argument("--bias", default=None, choices=["l2", "dot", "lp", "huber"],
                    help="attentional bias (default: the workload's own)")
    ap.add_argument("--bias-p", type=float, default=3.0, help="p of the l_p bias")
    ap.add_argument("--sign-alpha", type=float, default=0.0, help="l_p / Huber: 0 exact sign, > 0 tanh(alpha e)")
    ap.add_argument("--layernorm", action="store_true", help="MLP memory r + LN(W2 gelu(W1 x))")
    ap.add_argument("--gated", action="store_true", help="MLP memory r + W2 (gelu(W1 x) .* (W3 x))")
    ap.add_argument("--muon", action="store_true",
                    help="Muon memory optimizer (per-token Newton-Schulz; per-sequence family)")
    ap.add_argument("--ns-steps", type=int, default=5, help="Muon: Newton-Schulz steps")
    ap.add_argument("--seq-len", type=int, default=None, help="override the workload's tokens per sequence")
    ap.add_argument("--theta-as-stated", action="store_true",
                    help="theta = sigmoid(U(-4, 0)) without the division by the window c (the recipe as "
                         "stated, whose memory diverges to inf/NaN within a few chunks); throughput only")
    ap.add_argument("--prologue", action="store_true",
                    help="time the fused prologue (x -> q, k, v, gates) on the workload's shape instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0, help="seconds of oracle work (estimated)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only copy a buffer of this many bytes 3 times (HBM counter calibration)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: every (batch, head) sequence is independent, "
              "so a multi-GPU run is N copies of this one on a share of the sequences; "
              "no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from test_memorization_sequence_amd import binding, synth
    from test_memorization_sequence_amd.configs import WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.prologue:
        return bench_prologue(args, wl)
    if args.bias is not None:
        from dataclasses import replace
        wl = replace(wl, bias=args.bias, bias_p=args.bias_p, sign_alpha=args.sign_alpha)
    if args.layernorm or args.gated:
        from dataclasses import replace
        wl = replace(wl, layernorm=wl.layernorm or args.layernorm, gated=args.gated)
    if args.muon:
        from dataclasses import replace
        wl = replace(wl, optimizer="muon", ns_steps=args.ns_steps)
    if args.seq_len is not None:
        wl = wl.with_shape(seq_len=args.seq_len)
    if args.theta_as_stated:
        from dataclasses import replace
        wl = replace(wl, theta_div=1.0)
    print(f"[bench] {wl.name} bias={wl.bias}: B={wl.batch} H={wl.heads} N={wl.seq_len} ({wl.note})", file=sys.stderr, flush=True)
    inputs = synth.make_inputs(wl, 0)
    w0 = synth.initial_weights_flat(wl, inputs)
    dev = torch.device("cuda:0")
    io = torch.float32 if wl.io_dtype == "f32" else torch.bfloat16
    t_in = {k: torch.from_numpy(inputs[k]).to(dev, dtype=io) for k in ("q", "k", "v")}
    g_in = {k: torch.from_numpy(inputs[k]).to(dev) for k in ("alpha", "eta", "theta", "gamma", "delta") if k in inputs}
    mem = binding.AtlasMem(wl, args.kernel)
    state = mem.new_state(torch.from_numpy(w0), device=dev)
    out = torch.empty(wl.batch, wl.heads, wl.seq_len, wl.d_v, dtype=io, device=dev)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    ev1.record(stream)
    mem.set_kernel_events(ev0, ev1)

    def step():
        mem.forward(t_in["q"], t_in["k"], t_in["v"], g_in["alpha"], g_in["eta"] if wl.momentum else None,
                    g_in["theta"], g_in["gamma"], state, out, stream, delta=g_in.get("delta"))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    kernel_ms = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
        ev1.synchronize()
        kernel_ms.append(ev0.elapsed_time(ev1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mem.set_kernel_events(None, None)
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    flags = mem.device_errors()
    finite = bool(torch.isfinite(out.float()).all())
    if flags != 0:
        print(f"[bench] error: device error word {flags:#x} (a group barrier timed out; outputs invalid)",
              file=sys.stderr)
        sys.exit(3)
    if not finite and not args.theta_as_stated:
        print("[bench] error: non-finite outputs", file=sys.stderr)
        sys.exit(3)

    S = wl.batch * wl.heads
    nch = -(-wl.seq_len // wl.chunk)
    muon = wl.optimizer == "muon"
    flops = alg_flops_muon(wl, wl.seq_len) * S if muon else alg_flops_per_chunk(wl) * nch * S
    k_ms = float(np.mean(kernel_ms))
    achieved = flops / (k_ms * 1e-3) / 1e12
    # Muon's Newton-Schulz GEMMs run as fp32 MFMA
    peak = PEAK_FP32_TFLOPS if wl.io_dtype == "f32" or muon else PEAK_BF16_TFLOPS
    meas = (MEASURED_TRAFFIC.get((wl.name, kernel_name(binding, wl, args.kernel), wl.optimizer, wl.seq_len))
            if wl.bias == "l2" and not wl.layernorm and not wl.gated else None)
    traffic = meas["bytes"] if meas and meas["src"] == kernel_source_hash(kernel_name(binding, wl, args.kernel)) else None
    tokens = wl.batch * wl.seq_len
    res = {
        "metric": "memory update+retrieve tokens/sec (1 GPU); MFMA util % of bf16 peak",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.io_dtype == "f32" else "bf16",
        "data": "synthetic (seeded numpy: L2-normalised q,k; N(0,1) v; sigmoid gates"
                + (", theta as stated: the memory diverges, outputs non-finite)" if args.theta_as_stated
                   else f", theta / {wl.theta_div:g})" if wl.theta_div != 1.0 else ")"),
        "config": {"workload": wl.name, "kernel_family": args.kernel, "batch": wl.batch, "heads": wl.heads, "seq_len": wl.seq_len,
                   "d_k": wl.d_k, "d_v": wl.d_v, "memory": wl.memory, "hidden": wl.hidden,
                   "feature_dim": wl.feature_dim, "window": wl.window, "chunk": wl.chunk,
                   "momentum": wl.momentum, "bias": wl.bias, "layernorm": wl.layernorm, "gated": wl.gated,
                   **({"optimizer": "muon", "ns_steps": wl.ns_steps} if muon else {}),
                   **({"bias_p": wl.bias_p} if wl.bias == "lp" else {}),
                   **({"sign_alpha": wl.sign_alpha} if wl.bias in ("lp", "huber") else {})},
        "head_tokens_per_s": S * wl.seq_len / (ms_per_step * 1e-3),
        "mfma_util_pct": 100.0 * (flops / (ms_per_step * 1e-3) / 1e12) / peak,
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_name(binding, wl, args.kernel),
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
            "traffic_unit": "bytes per launch",
            "alg_flops_per_launch": flops,
            "kernel_ms": k_ms,
        },
        "hbm_alg_gbs": alg_bytes_per_head_token(wl) * S * wl.seq_len / (ms_per_step * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, inputs, w0, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
