"""Builds liba8w8.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m w8a8_quantized_decode_amd.build`` (or ``build()`` from Python).
Every source in ``csrc/`` is compiled with hipcc as HIP for gfx950 and linked into
``w8a8_quantized_decode_amd/liba8w8.so``; the measurement aid in ``measure/`` (the
streaming-read ceiling that bench.py reports) becomes ``libmeasure.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "liba8w8.so")
MEASURE = os.path.join(PKG, "measure")
MEASURE_LIB = os.path.join(PKG, "libmeasure.so")
OBJ_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # exact FP32 semantics: no contraction of a*b+c into FMA; IEEE division / sqrt
    "-ffp-contract=off",
    "-fno-fast-math",
    # keep the compiler from emitting packed FP32 ALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}",
]


# Per-source additions.  The prefill GEMM keeps its MFMA accumulators in architectural
# VGPRs: its operand stages fill the accumulation registers, and with accumulators there
# too the allocator rotates them through copies every loop iteration.
FILE_FLAGS = {
    "gemm_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liba8w8)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(os.path.dirname(src)) + "_" +
                       os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + FLAGS + FILE_FLAGS.get(
        os.path.basename(src), [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compiles every source and links liba8w8.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    msrcs = sorted(os.path.join(MEASURE, f) for f in os.listdir(MEASURE) if f.endswith(".hip"))
    mobjs = [_compile(f) for f in msrcs]
    tmp = MEASURE_LIB + ".tmp"
    r = subprocess.run([hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + mobjs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, MEASURE_LIB)
    if verbose:
        print(f"built {LIB} and {MEASURE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
