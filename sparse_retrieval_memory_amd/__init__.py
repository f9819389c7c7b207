"""MI355X-native Memory Sparse Attention (MSA) routing + sparse-attention hot path.

The compute lives in libmsa.so (hand-written HIP for gfx950, C ABI declared in
include/msa.h).  This package is its thin binding (``ops``: same names as the
C calls, taking torch tensors) plus the host-side driver of the Memory
Interleave rounds (``interleave``).  Importing it does not load the library; the first call
does, and raises if it is not built -- there is no CPU fallback.
"""

from . import _lib, ops  # noqa: F401
from ._lib import MSAError  # noqa: F401

__all__ = ["ops", "MSAError"]
