"""Build the HIP library ``libqrw.so`` in-tree for gfx950, and beside it
``libqrw_probe.so`` (csrc/probe: the benchmark's same-traffic copy, empty-grid
and timeline kernels, and the GPU tests' exhaustive arithmetic sweeps).

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
PROBE_LIB = os.path.join(PKG, "libqrw_probe.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def probe_sources():
    return sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))


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


FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall"]


def _link(objs, out, verbose):
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    tl = torch_lib_dir()
    if tl:
        cmd += [f"-Wl,-rpath,{tl}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile each source to an object in parallel (bounded by ``jobs``, default
    the CPU count, at most 16), then link the operator library and the probe
    library.  Returns the operator library's path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    psrcs = probe_sources()
    objs = [os.path.join(objdir, os.path.basename(f)[:-4] + ".o") for f in srcs]
    pobjs = [os.path.join(objdir, "probe_" + os.path.basename(f)[:-4] + ".o") for f in psrcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc(), f"--offload-arch={ARCH}"] + FLAGS + ["-I", INCLUDE, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True)

    n = jobs or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        results = list(ex.map(compile_one, zip(srcs + psrcs, objs + pobjs)))
    failed = False
    for src, r in zip(srcs + psrcs, results):
        out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in line)
        if out.strip():
            print(out, file=sys.stderr)
        if r.returncode != 0:
            print(f"compiling {os.path.basename(src)} failed", file=sys.stderr)
            failed = True
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc")
    _link(objs, LIB, verbose)
    _link(pobjs, PROBE_LIB, verbose)
    build_host_cost(verbose)
    return LIB


HOST_COST = os.path.join(PKG, "qrw_host_cost")


def build_host_cost(verbose: bool = False) -> str:
    """The C host-cost harness (csrc/probe/host_cost.c), linked against both
    libraries and the system HIP runtime."""
    rocm_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "probe", "host_cost.c"), "-o", HOST_COST + ".tmp",
           "-L", PKG, "-lqrw", "-lqrw_probe", "-L", rocm_lib, "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{rocm_lib}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(HOST_COST + ".tmp", HOST_COST)
    return HOST_COST


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
    sys.exit(0)
