"""Build libsvdq.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with IEEE-exact fp32
division and denormals (no fast-math), no floating-point contraction (the
packed codes must be bit-identical to their definition; kernels that want a
fused multiply-add write fmaf explicitly), and without packed-fp32
instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsvdq.so")
# measurement aid used only by the benchmark (not part of the layer's ABI)
PROBE_LIB = os.path.join(HERE, "libsvdq_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["svdq_api.cpp", "quantize_act.hip", "pack_weight.hip", "images.hip", "gemm_int4.hip",
           "gemm_fp4.hip", "gemm_int4_gelu.hip", "lowrank_up.hip", "awq.hip", "lowrank_factors.hip", "qk_norm_rope.hip",
           "nvfp4.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-ffp-contract=off",
    "-fconstexpr-steps=50000000",  # the GELU table is evaluated at compile time
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    pobjs = [_compile(src) for src in PROBE_SOURCES]
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *pobjs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
