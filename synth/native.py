"""ctypes access to the compiled generator (host C and device HIP versions).

Both produce exactly the bits of ``synth.splitmix.normal_bf16``; they exist for
speed.  Build them with ``python -m synth.build`` (``__graft_entry__.build()``
does it too).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import splitmix as sm

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_fill.so")

_host = None
_dev = None
_dev_tables = {}


def available() -> bool:
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB) or os.environ.get("SYNTH_NO_NATIVE") == "1":
            _host = False
        else:
            lib = ctypes.CDLL(HOST_LIB)
            lib.synth_normal_bf16_host.argtypes = [ctypes.c_uint64] * 4 + [
                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
            lib.synth_normal_bf16_host.restype = None
            _host = lib
    return _host is not False


def normal_bf16(seed, tid, layer, start, count) -> np.ndarray:
    assert available()
    out = np.empty(count, dtype=np.uint16)
    if count:
        _host.synth_normal_bf16_host(seed, tid, layer, start, count,
                                     sm.NORMAL_TABLE.ctypes.data, out.ctypes.data)
    return out


def _device_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run python -m synth.build)")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill_normal_bf16.argtypes = [ctypes.c_uint64] * 4 + [
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill_normal_bf16.restype = ctypes.c_int
        _dev = lib
    return _dev


def fill_normal_bf16_device(out, seed, tid, layer, start, stream=None):
    """Fill the contiguous int16/uint16 CUDA tensor ``out`` on its device."""
    import torch
    lib = _device_lib()
    dev = out.device
    if dev not in _dev_tables:
        _dev_tables[dev] = torch.from_numpy(sm.NORMAL_TABLE.view(np.int16).copy()).to(dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    assert out.is_contiguous() and out.element_size() == 2
    rc = lib.synth_fill_normal_bf16(seed, tid, layer, start, out.numel(),
                                    _dev_tables[dev].data_ptr(), out.data_ptr(),
                                    ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_bf16 failed: {rc}")
    return out
