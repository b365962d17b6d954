"""Builds libkivi.so in-tree with hipcc for gfx950.

Usage: ``python -m kv_cache_quantization_codec_amd.build`` (or call
:func:`build`).  The library is placed next to this file, where the binding
loads it from.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkivi.so")

SOURCES = [os.path.join(CSRC, "kivi_api.cpp"), os.path.join(CSRC, "kivi_kernels.hip"),
           os.path.join(CSRC, "kivi_attention.hip"), os.path.join(CSRC, "kivi_copy.hip"),
           os.path.join(CSRC, "kivi_fp8.hip")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # min/max of fp16 values skip NaN quieting (inputs are finite by contract);
    # fp32 division stays correctly rounded (no fast-math flags).
    "-fno-honor-nans",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkivi")


def build(verbose: bool = False) -> str:
    """Compile every source into ``libkivi.so`` (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
