"""Builds libatlas_mem.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libatlas_mem.so")
SOURCES = ["atlas_mem_kernels.hip", "atlas_mem_sharded.hip", "atlas_mem_stream.hip", "atlas_mem_grouped.hip",
           "atlas_mem_linear.hip",
           "atlas_mem_api.hip", "atlas_prologue.hip", "atlas_prologue_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels read every accumulator back
    # into vector arithmetic, and accumulation registers only add copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + INCLUDE, "-I" + CSRC,
]


# The projection GEMM keeps its 64 accumulator tiles per wave in the
# accumulation registers for the whole K loop, so it is built without the
# VGPR form of the MFMA results.
NO_VGPR_FORM = {"atlas_prologue_gemm.hip"}


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(CSRC, src.replace(".hip", ".o"))
    flags = FLAGS
    if src in NO_VGPR_FORM:
        flags = [f for i, f in enumerate(FLAGS)
                 if f != "-amdgpu-mfma-vgpr-form=1" and not (f == "-mllvm" and FLAGS[i + 1] == "-amdgpu-mfma-vgpr-form=1")]
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops' is not a recognized" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose: bool = False) -> str:
    # one hipcc per translation unit, run side by side
    from concurrent.futures import ThreadPoolExecutor
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
