"""Build libaggemm.so (the HIP kernels and the C ABI) in-tree for gfx950,
and libaggprobe.so, the benchmark's register-only matrix-core probe.

    python communication_gemm_amd/build.py   (run by path: importing the
                                             package would load the library)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libaggemm.so")
PROBE_LIB = os.path.join(PKG, "libaggprobe.so")

SOURCES = ["api.cpp", "plan.cpp", "producer.hip", "consumer.hip", "scratch.hip"]
PROBE_SOURCES = ["probe.hip"]

# Packed fp32 instructions are switched off for every HIP translation unit.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libaggemm.so and
    libaggprobe.so atomically."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cc = hipcc()
    procs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("HIP build failed")
    n = len(SOURCES)
    for lib, part in ((LIB, objs[:n]), (PROBE_LIB, objs[n:])):
        tmp = lib + f".tmp{os.getpid()}"
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *part, "-o", tmp]
        subprocess.run(link, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
