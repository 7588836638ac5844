"""VeriCache draft/verify hot path on AMD MI355X.

The compute lives in libvc.so (HIP kernels for gfx950, C ABI in include/vc.h);
this package is the Python binding over it (ctypes; PyTorch supplies device
memory and streams) plus the host-side scheduler that interleaves requests'
drafting and verification.
"""
from . import _vc  # noqa: F401  (raises ImportError when the library is not built)
from .binding import *  # noqa: F401,F403
