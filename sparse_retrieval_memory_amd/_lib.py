"""ctypes loader for libmsa.so: argument marshalling only, no computation.

The library is built in-tree (``python -m sparse_retrieval_memory_amd.build``).
There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
# MSA_LIBRARY names another build of the same library (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(_HERE, "libmsa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "msa.h")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4

c_p = ctypes.c_void_p
c_i = ctypes.c_int
c_i64 = ctypes.c_int64
c_sz = ctypes.c_size_t
c_d = ctypes.c_double
c_f = ctypes.c_float

SIGNATURES = {
    "msa_version": (c_i, []),
    "msa_status_string": (ctypes.c_char_p, [c_i]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_pool_chunks": (c_i, [c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i, c_i, c_i, c_d,
                              c_p, c_p, c_p, c_p]),
    "msa_encode_workspace_bytes": (c_sz, [c_i64, c_i]),
    "msa_encode_router_keys": (c_i, [c_p, c_i64, c_i, c_p, c_i, c_i, c_p, c_p, c_i64, c_i64, c_i, c_p, c_p,
                                     c_sz, c_p]),
    "msa_store_delete_workspace_bytes": (c_sz, [c_i64]),
    "msa_store_delete": (c_i, [c_p, c_p, c_p, c_i64, c_i64, c_i, c_i, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz,
                               c_p]),
    "msa_store_append": (c_i, [c_p, c_p, c_p, c_i64, c_i64, c_i, c_i, c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_p]),
    "msa_route_workspace_bytes": (c_sz, [c_i, c_i, c_i, c_i, c_i64, c_i64]),
    "msa_route_scores": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_i64, c_p, c_p, c_p,
                               c_p, c_sz, c_p]),
    "msa_krbar_inv_norms": (c_i, [c_p, c_i64, c_i, c_i, c_p, c_p]),
    "msa_route_backward_workspace_bytes": (c_sz, [c_i, c_i, c_i, c_i, c_i64]),
    "msa_sparse_attn_backward_workspace_bytes": (c_sz, [c_i, c_i, c_i, c_i, c_i, c_i, c_i]),
    "msa_sparse_attn_backward": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_i, c_p, c_p, c_i64, c_i, c_p,
                                       c_i, c_d, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "msa_route_scores_backward": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_i64, c_p, c_p, c_p,
                                        c_p, c_p, c_p, c_p, c_sz, c_p]),
    "msa_topk_workspace_bytes": (c_sz, [c_i, c_i64, c_i]),
    "msa_topk_docs": (c_i, [c_p, c_i, c_i64, c_i, c_p, c_p, c_p, c_sz, c_p]),
    "msa_route_topk_workspace_bytes": (c_sz, [c_i, c_i, c_i, c_i, c_i64, c_i64, c_i]),
    "msa_route_topk": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_i64, c_p, c_i, c_p, c_p, c_p, c_p, c_p,
                             c_sz, c_p]),
    "msa_route_topk_noalloc": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_i64, c_p, c_i, c_p, c_p, c_p,
                                     c_p, c_p]),
    "msa_route_scan": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_sz, c_p]),
    "msa_route_select": (c_i, [c_i, c_i64, c_p, c_i64, c_p, c_i, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "msa_route_workspace_clear": (c_i, [c_p, c_sz, c_p]),
    "msa_fetch_docs": (c_i, [c_p, c_i, c_i, c_p, c_p, c_i64, c_i, c_i, c_p, c_i, c_p, c_p, c_p]),
    "msa_gather_docs": (c_i, [c_p, c_i, c_i, c_p, c_p, c_i64, c_i, c_i, c_p, c_i, c_p, c_p]),
    "msa_append_router_rows": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_p, c_i, c_i, c_p, c_p, c_p, c_p]),
    "msa_sparse_attn_decode": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_i, c_p, c_p, c_i64,
                                     c_i, c_p, c_i, c_d, c_f, c_p, c_p]),
    "msa_sparse_attn_local_partial": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_i, c_i, c_d, c_f, c_p, c_p,
                                            c_p]),
    "msa_sparse_attn_memory_merge": (c_i, [c_p, c_i, c_i, c_i, c_i, c_i, c_i, c_p, c_p, c_i64, c_i, c_p, c_i, c_d,
                                           c_f, c_p, c_p, c_p, c_p, c_p]),
    "msa_sparse_attn_forward": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_i, c_p, c_p, c_i64,
                                      c_i, c_p, c_i, c_d, c_f, c_p, c_p, c_p]),
    "msa_sparse_attn_backward_saved": (c_i, [c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_i, c_p, c_p, c_i64, c_i,
                                             c_p, c_i, c_d, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                             c_sz, c_p]),
}


class MSAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmsa.so is not built ({LIB_PATH}); run "
                               "python -m sparse_retrieval_memory_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def declared_symbols() -> list:
    """Names of the functions declared in include/msa.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(msa_\w+)\s*\(", text, re.M)))


def call(name: str, *args) -> int:
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != MSA_OK:
        raise MSAError(name, rc, lib.msa_last_error().decode())
    return rc


def raw(name: str, *args):
    """Call without raising (for error-path tests)."""
    return getattr(load(), name)(*args)
