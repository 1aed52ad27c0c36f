"""Build the gfx950 paged-attention library (libpaged_attn.so) with hipcc.

Every kernel is compiled for gfx950 only, with packed-fp32 instruction
selection switched off and IEEE-correct fp32 division (the fp8 store
quantiser divides).  The library is built in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpaged_attn.so")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "write_kv.hip", "pages.hip", "noalloc.hip",
           "verify.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]

# Per-source flags for prefill.hip (the row-tile kernel):
#  * it never tests for NaN (masked keys are replaced by a select before any
#    max, and rejected pages are flagged with NaN bit patterns written as
#    integers), so NaN canonicalisation of max inputs is dropped;
#  * its MFMA accumulators are selected in VGPR form.  In AGPR form the
#    compiler kept a VGPR copy of every O^T accumulator for the (rare) VALU
#    rescale and moved all of them between the two files on every step
#    (about 300 v_accvgpr moves per 64 MFMAs); in VGPR form the accumulators
#    stay put and only the loop-invariant Q^T operands overflow into AGPRs,
#    which the MFMAs read directly.
EXTRA = {"prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile and link; returns the path of the shared library."""
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(HERE, "_build", src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + COMMON + lang + EXTRA.get(src, []) + ["-c", path, "-o", obj]
        if resource_usage and src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--usage" in sys.argv))
