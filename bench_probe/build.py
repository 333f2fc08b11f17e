"""Builds libstreamprobe.so (HIP, gfx950) beside this file: the benchmark's
plain streaming-bandwidth probe (read-only, write-only and copy kernels).  It is
measurement harness for bench.py, not part of the decode library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "stream_probe.hip"
LIB = HERE / "libstreamprobe.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> Path:
    """Compile and link libstreamprobe.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="streamprobe_build_") as tmp:
        out = Path(tmp) / LIB.name
        cmd = [HIPCC, *FLAGS, str(SRC), "-o", str(out)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
