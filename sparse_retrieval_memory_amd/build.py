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


def build_sanitized(out: str, verbose: bool = False) -> str:
    """The same library with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged), for checking the C ABI's
    host-side validation; load it with the ASan runtime preloaded."""
    flags = [f for f in FLAGS if f != "-O3"]
    cmd = ["/opt/rocm/bin/hipcc", *flags, "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           *SOURCES, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return out


if __name__ == "__main__":
    if sys.argv[1:2] == ["--sanitized"]:
        build_sanitized(sys.argv[2], verbose=True)
    else:
        build(extra=sys.argv[1:])
