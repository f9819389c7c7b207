"""Compile the oracle's C helper (gcc, OpenMP) in-tree: test infrastructure only."""

from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = True) -> None:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", os.path.join(_HERE, "csrc", "pool_means.c"),
           "-o", os.path.join(_HERE, "liboracle_pool.so")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build()
