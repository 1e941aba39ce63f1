"""ctypes binding of libipttt_probe (include/ipttt_probe.h): micro-benchmarks of
the chip's achievable rates, for measurement only (the benchmark reports the
layer's kernels against them). Loading fails loudly if the library is missing."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libipttt_probe.so")

IPTTT_PROBE_MFMA16 = 0
IPTTT_PROBE_MFMA32 = 1
IPTTT_PROBE_READ = 2
IPTTT_PROBE_LDS = 3
IPTTT_PROBE_COPY = 4
EXPORTS = ("ipttt_probe",)

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with chunked_weight_mlp_amd/build.py")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.ipttt_probe.argtypes = [ctypes.c_int32, ctypes.c_int64, vp, ctypes.c_size_t, vp,
                                ctypes.c_size_t, ctypes.POINTER(ctypes.c_double), vp]
    lib.ipttt_probe.restype = ctypes.c_int
    _lib = lib
    return lib


def ipttt_probe(kind: int, n: int, src, src_bytes: int, dst, dst_bytes: int, stream=None) -> float:
    """Enqueues one launch; returns its FLOPs (MFMA kinds) or bytes (the others)."""
    work = ctypes.c_double(0.0)
    s = load().ipttt_probe(kind, n, src, src_bytes, dst, dst_bytes, ctypes.byref(work), stream)
    if s != 0:
        raise RuntimeError(f"ipttt_probe(kind={kind}) failed with status {s}")
    return work.value
