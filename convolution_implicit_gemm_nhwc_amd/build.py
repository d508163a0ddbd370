"""Build libfconv.so (the C-ABI library with its gfx950 kernels) in-tree.

    python -m convolution_implicit_gemm_nhwc_amd.build

Kernels are compiled ahead of time for gfx950 only.  Flags:
  -ffp-contract=off   the int8 epilogue is specified operation by operation;
                      no multiply-add may be formed that the source does not
                      write (the side-input step calls fmaf explicitly);
  -fno-fast-math      IEEE semantics for the epilogues;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 VALU instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfconv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "conv.hip", "wgrad.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, src + ".o")
        cmd = [HIPCC, *COMMON]
        if src.endswith(".hip"):
            cmd += DEVICE
        cmd += ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
