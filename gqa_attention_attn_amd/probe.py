"""Python binding of libgqa_probe.so (include/gqa_probe.h): the HBM read and
copy probes and the empty kernel that bench.py times beside the attention
kernels.  Argument marshalling only; raises if the library is not built."""

from __future__ import annotations

import ctypes
import os

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_probe.so")
EXPORTS = ("gqa_probe_read", "gqa_probe_copy", "gqa_probe_empty")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built (python -m gqa_attention_attn_amd.build)")
        import torch  # noqa: F401  (bind to torch's HIP runtime, as the attention library does)
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp = ctypes.c_void_p
        L.gqa_probe_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.gqa_probe_read.restype = ctypes.c_int32
        L.gqa_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.gqa_probe_copy.restype = ctypes.c_int32
        L.gqa_probe_empty.argtypes = [vp]
        L.gqa_probe_empty.restype = ctypes.c_int32
        _lib = L
    return _lib


def read(src: int, nbytes: int, sink: int, stream: int) -> int:
    return int(lib().gqa_probe_read(src, int(nbytes), sink, stream))


def copy(src: int, dst: int, nbytes: int, stream: int) -> int:
    return int(lib().gqa_probe_copy(src, dst, int(nbytes), stream))


def empty(stream: int) -> int:
    return int(lib().gqa_probe_empty(stream))
