"""Builds libstepq.so (HIP, gfx950) in the package directory.

hipcc compiles for gfx950 only, with packed-FP32 instruction selection
turned off, -O3 and IEEE division / square root (no fast-math).
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libstepq.so"
INCLUDE = PKG.parent / "include"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}"]
SOURCES = ["stepq_kernels.hip", "stepq_api.cpp"]


def build(verbose: bool = False) -> Path:
    """Compile every source and link libstepq.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="stepq_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = Path(tmp) / (src + ".o")
            cmd = [HIPCC, *FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(str(obj))
        out = Path(tmp) / "libstepq.so"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", str(out)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
