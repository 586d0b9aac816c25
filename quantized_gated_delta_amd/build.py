"""Compile the HIP library ``libsq.so`` for gfx950 in-tree.

hipcc cross-compiles without a GPU.  Flags:
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
  -fno-gpu-flush-denormals-to-zero                   keep fp32 subnormals (IEEE)
  -fhip-fp32-correctly-rounded-divide-sqrt           correctly rounded 1/x, x/y
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsq.so")
# the instrumented timeline build (-DSQ_TIMELINE): decode kernels that store
# per-wave phase timestamps; loaded instead of libsq.so when SQ_LIBRARY names it
LIB_TIMELINE = os.path.join(HERE, "libsq_timeline.so")
ARCH = "gfx950"

SOURCES = ["sq_kernels.hip", "sq_probe.hip", "sq_api.cpp"]

HIP_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra=(), timeline: bool = False) -> str:
    """Compile every source and link libsq.so (always rebuilds); timeline:
    the instrumented build libsq_timeline.so instead."""
    objs = []
    build_dir = os.path.join(HERE, "_build_timeline" if timeline else "_build")
    os.makedirs(build_dir, exist_ok=True)
    flags = HIP_FLAGS + (["-DSQ_TIMELINE"] if timeline else [])
    out = LIB_TIMELINE if timeline else LIB
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + flags + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
