"""Compile the generator's host (gcc/OpenMP) and device (hipcc, gfx950) libraries in-tree."""

from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = True) -> None:
    src = os.path.join(_HERE, "csrc")
    host_cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared",
                os.path.join(src, "gen_host.c"), "-o", os.path.join(_HERE, "libsynth_host.so")]
    dev_cmd = ["/opt/rocm/bin/hipcc", *HIP_FLAGS, os.path.join(src, "fill.hip"),
               "-o", os.path.join(_HERE, "libsynth_fill.so")]
    for cmd in (host_cmd, dev_cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=subprocess.PIPE if not verbose else None)


if __name__ == "__main__":
    build()
    sys.exit(0)
