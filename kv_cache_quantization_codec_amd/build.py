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

# flags for every compile step; "-shared" goes on the link line only
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # min/max of fp16 values skip NaN quieting (inputs are finite by contract);
    # fp32 division stays correctly rounded (no fast-math flags).
    "-fno-honor-nans",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]

OBJ_DIR = os.path.join(HERE, "_build")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkivi")


def _filtered(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source into ``libkivi.so`` (always recompiles).

    The sources compile in parallel, one hipcc process each (the attention
    kernels' templates dominate the time), and are linked in one step."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                text=True)))
    failed = []
    for cmd, obj, proc in jobs:
        _, err = proc.communicate()
        err = _filtered(err)
        if proc.returncode != 0:
            failed.append(f"{cmd[-3]} ({proc.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-fPIC", "-shared", *(obj for _, obj, _ in jobs), "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filtered(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
