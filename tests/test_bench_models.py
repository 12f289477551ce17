"""The benchmark's work models (CPU): the algorithmic FLOPs per chunk of the
gradient-descent path and of the Muon path, and the algorithmic bytes per
head-token, against the per-chunk breakdown worked out for each workload and
against plain counting of the GEMMs they stand for."""
import importlib.util
import os
import subprocess
import sys
from dataclasses import replace

import pytest

from test_memorization_sequence_amd.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# MFLOP per chunk of one sequence (forward + backward + update + retrieval
# state side + intra-chunk), at b = 64
PER_CHUNK_MFLOP = {"linear64_delta": 2.62, "linear_poly2": 19.07, "mlp64": 28.31, "atlas_long": 471.9,
                   "layer_scale": 136.3}


@pytest.mark.parametrize("name", list(PER_CHUNK_MFLOP))
def test_flops_per_chunk(bench, name):
    assert bench.alg_flops_per_chunk(WORKLOADS[name]) / 1e6 == pytest.approx(PER_CHUNK_MFLOP[name], rel=2e-3)


def test_layer_scale_launch_flops(bench):
    wl = WORKLOADS["layer_scale"]
    assert bench.alg_flops_per_chunk(wl) * 256 * 96 == 3349269184512


def test_bytes_per_head_token(bench):
    assert bench.alg_bytes_per_head_token(WORKLOADS["layer_scale"]) == 1040
    assert bench.alg_bytes_per_head_token(WORKLOADS["linear64_delta"]) == 1040
    assert bench.alg_bytes_per_head_token(WORKLOADS["linear_poly2"]) == 272
    assert bench.alg_bytes_per_head_token(WORKLOADS["mlp64"]) == 528


def test_muon_flops_by_counting(bench):
    """128-512-128 MLP, c = 32, 64 tokens: one chunk's window forward and
    backward, then per token and matrix (both 128 x 512 in the orientation
    with fewer rows) the running window gradient (4 per weight), five
    Newton-Schulz steps (symmetric X X^T and A A at half cost, B X in full),
    the update and the retrieval."""
    wl = replace(WORKLOADS["layer_scale"], optimizer="muon", ns_steps=5)
    W, D, dv, h = 64 + 32 - 1, 128, 128, 512
    chunk = 2 * W * (h * D + dv * h) + 2 * W * dv * h
    r, n = 128, 512
    step = r * r * n + r ** 3 + 2 * r * r * n
    per_matrix = 4 * r * n + 5 * step + 2 * r * n
    assert bench.alg_flops_muon(wl, 64) == chunk + 64 * 2 * per_matrix
    assert bench.alg_flops_muon(wl, 64) * 96 == pytest.approx(1.683455e12, rel=1e-6)
    # ns_steps and c enter as counted
    assert bench.alg_flops_muon(replace(wl, ns_steps=1), 64) < bench.alg_flops_muon(wl, 64)
    assert bench.alg_flops_muon(replace(wl, window=1), 64) < bench.alg_flops_muon(wl, 64)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The product path has no fallback: with the library absent, the first
    call into the binding raises."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from test_memorization_sequence_amd import binding\n"
            "binding.LIB_PATH = %r\n"
            "binding._lib = None\n"
            "try:\n    binding.lib()\nexcept ImportError as e:\n    print('raised', e)\n") % (ROOT, str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert "raised" in r.stdout, r.stdout + r.stderr
