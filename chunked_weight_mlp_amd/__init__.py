"""MI355X (gfx950) fast-weight prefill of In-Place Test-Time Training.

The compute path is libipttt.so (hand-written HIP kernels behind a C ABI,
include/ipttt.h); `ipttt` is its ctypes binding. Importing the binding does not
load the library; the first call does, and fails loudly if it is not built.
"""
from . import ipttt  # noqa: F401
from .ipttt import Layer, IptttError  # noqa: F401
