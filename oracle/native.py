"""ctypes access to the oracle's C helper (test infrastructure only).

``pool_means_bf16`` is ``msa_oracle.pool_means`` on bf16 bits, in C with
OpenMP, for pooling whole corpora; it is pinned against the numpy version in
tests/test_oracle_pins.py.  Build with ``python -m oracle.build``
(``__graft_entry__.build()`` does it too).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle_pool.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"oracle helper not built: {LIB} (run python -m oracle.build)")
        lib = ctypes.CDLL(LIB)
        lib.oracle_pool_means_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_pool_means_bf16.restype = ctypes.c_int64
        _lib = lib
    return _lib


def pool_means_bf16(bits: np.ndarray, doc_len, chunk: int) -> np.ndarray:
    """Chunk means (float64 [n_chunks, ...]) of bf16 bit rows ``bits`` [n_tok, ...] in document order."""
    x = np.ascontiguousarray(bits).view(np.uint16)
    L = np.ascontiguousarray(doc_len, dtype=np.int64)
    row = int(np.prod(x.shape[1:])) if x.ndim > 1 else 1
    assert x.shape[0] >= int(L.sum())
    n_chunks = int(((L + chunk - 1) // chunk).sum())
    out = np.empty((n_chunks,) + x.shape[1:], dtype=np.float64)
    rc = _load().oracle_pool_means_bf16(x.ctypes.data, row, L.ctypes.data, len(L), chunk, out.ctypes.data)
    if rc != n_chunks:
        raise RuntimeError(f"oracle_pool_means_bf16 returned {rc}")
    return out
