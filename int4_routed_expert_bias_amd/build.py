"""Build libcoli_moe.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcoli_moe.so")

SOURCES = ["coli_moe.cpp", "route.hip", "union.hip", "expert_f32.hip", "expert_i8.hip", "place.hip",
           "expert_i8v.hip", "combine.hip", "mla.hip", "noalloc.hip",
           "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # IEEE fp32 divide/sqrt (the int8 quantiser must round exactly like the oracle)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-file flags.  The router's fp64 MFMA accumulators stay in VGPRs (the
# default AGPR form copies them across the loop every iteration).  The
# streaming kernels' register rings are indexed by unrolled loop counters:
# the unroll limit for loops marked "#pragma unroll" is raised so that the
# largest instantiations (four tokens, the accumulator-dump variants) are
# still fully unrolled.
_UNROLL = ["-mllvm", "-pragma-unroll-threshold=100000"]
EXTRA = {"route.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "expert_i8v.hip": _UNROLL, "expert_f32.hip": _UNROLL}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + lang + ["-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
