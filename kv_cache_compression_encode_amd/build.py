"""Builds libcg.so (the gfx950 codec library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-ffp-contract=off",
    # packed fp32 instructions stay off: the compiler emits none of them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "--offload-arch=" + ARCH,
]
SOURCES = ["cg_kernels.hip", "cg_api.cpp"]


def build(verbose: bool = False, save_temps_dir: str | None = None) -> str:
    """Compiles every source and links libcg.so; always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if save_temps_dir:
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd, cwd=save_temps_dir or objdir)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
