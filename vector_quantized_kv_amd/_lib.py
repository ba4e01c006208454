"""ctypes declarations of libvq.so (the C ABI in include/vq.h)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvq.so")

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

SIGNATURES = {
    "vq_status_string": (ctypes.c_char_p, [c_int]),
    "vq_last_error": (ctypes.c_char_p, []),
    "vq_version": (c_int, []),
    "vq_supports_shape": (c_int, [c_int, c_int, c_int]),
    "vq_encode": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                          c_void_p, c_int, c_int, c_int,
                          c_void_p, c_int, c_int, c_void_p, c_void_p,
                          c_void_p, c_int, c_int, c_void_p,
                          c_void_p]),
    "vq_encode_kv": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                             c_void_p, c_int, c_int,
                             c_void_p, c_int, c_int, c_void_p, c_void_p,
                             c_void_p, c_int, c_int, c_int,
                             c_void_p, c_void_p, c_int, c_int, c_void_p,
                             c_void_p]),
    "vq_decode": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int,
                          c_void_p, c_int, c_int, c_int,
                          c_void_p, c_int, c_int, c_void_p, c_void_p, c_int,
                          c_void_p, c_int, c_void_p]),
    "vq_encode_decode": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                                 c_void_p, c_int, c_int, c_int,
                                 c_void_p, c_int, c_int, c_void_p, c_void_p,
                                 c_void_p, c_int, c_int, c_void_p,
                                 c_void_p, c_int, c_void_p]),
    "vq_transform": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_int, c_int,
                             c_void_p, c_void_p, c_void_p]),
    "vq_kmeans_workspace_bytes": (c_size_t, [ctypes.c_longlong, c_int, c_int]),
    "vq_kmeans": (c_int, [c_void_p, ctypes.c_longlong, c_int, c_void_p, c_int, c_int,
                          c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "vq_attend_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "vq_attend_path": (c_int, [c_int] * 12),
    "vq_attend": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                          c_void_p, c_void_p, c_int,
                          c_void_p, c_int, c_int, c_void_p, c_void_p,
                          c_void_p, c_void_p, c_int,
                          c_int, c_int, c_int, c_int, c_void_p,
                          c_float, c_int, c_int,
                          c_void_p, c_void_p, c_size_t, c_void_p]),
    "vq_decode_step": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                               c_void_p, c_void_p, c_int,
                               c_void_p, c_int, c_int,
                               c_void_p, c_void_p, c_int,
                               c_int, c_int, c_int, c_int, c_void_p,
                               c_float, c_int, c_int,
                               c_void_p, c_void_p, c_size_t, c_void_p]),
    "vq_attend_noalloc": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_int,
                                  c_void_p, c_int, c_int, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_int,
                                  c_int, c_int, c_int, c_int, c_void_p,
                                  c_float, c_int, c_int,
                                  c_void_p, c_void_p]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -m vector_quantized_kv_amd.build)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
