"""Build libnvfp4.so (gfx950) in-tree with hipcc.

Every HIP source is compiled with -ffp-contract=off (the quantizer's arithmetic is fixed in
binary32 with one rounding per operation) and without packed-FP32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnvfp4.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["nvfp4_kernels.hip", "nvfp4_gemm.hip", "nvfp4_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", INCLUDE,
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append((src, [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    for src, cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, cwd=BUILD_DIR, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        for src, out in failed:
            sys.stderr.write(f"--- hipcc failed on {src}\n{out}\n")
        raise RuntimeError("libnvfp4 build failed: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                          cwd=BUILD_DIR)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
