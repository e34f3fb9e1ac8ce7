"""Build the HIP library ``libqrw.so`` in-tree for gfx950.

Compiled with hipcc -O3 and no fast-math; packed-fp32 instruction generation
is switched off (``-packed-fp32-ops``) so binary32 math is emitted as scalar
VALU ops.  The library's only runtime dependency is the HIP runtime
(``libamdhip64.so.7``); its RUNPATH points at the copy that ships with torch,
so the library and torch share one runtime whichever is loaded first.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqrw.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def torch_lib_dir():
    import importlib.util

    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        return None
    return os.path.join(os.path.dirname(spec.origin), "lib")


def hipcc():
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", INCLUDE, "-o", LIB + ".tmp"] + sources()
    tl = torch_lib_dir()
    if tl:
        cmd += [f"-Wl,-rpath,{tl}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
    sys.exit(0)
