"""Compile libmsa.so (all HIP sources, gfx950) in-tree with hipcc."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libmsa.so")
SOURCES = sorted(glob.glob(os.path.join(_HERE, "csrc", "*.hip")))
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def build(verbose: bool = True, extra=()) -> str:
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:])
