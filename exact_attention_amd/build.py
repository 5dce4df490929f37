"""Build libmfa.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m exact_attention_amd.build`` (or ``build()`` from Python).  Always
recompiles.  The library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmfa.so")

SOURCES = ["mfa_api.cpp", "mfa_fwd.hip", "mfa_decode.hip", "mfa_bwd.hip"]

# Packed-fp32 VALU instructions are disabled for the device code (hipcc would
# otherwise form them from ordinary float code).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


# Per-source extra flags (none at present).
SOURCE_FLAGS: dict = {}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (ROCm is required to build libmfa)")
    return cand


def build(verbose: bool = False, extra_flags=None) -> str:
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *(extra_flags or []), "-I", INCLUDE,
               "-I", CSRC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, cmd, r

    # the sources compile independently (the forward kernel's file takes the longest)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = []
    for src, obj, cmd, r in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(_filter_warnings(r.stderr), file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def _filter_warnings(text: str) -> str:
    # the host pass does not know the device-only target feature; that note is harmless
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    return "\n".join(lines)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
