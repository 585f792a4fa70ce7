"""Loading libtcgemm.so.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process: device pointers and streams from
torch are then valid in the library).  There is no fallback: if the library
is missing the import of the product fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must be loaded before libtcgemm.so)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtcgemm.so")

_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LibraryMissing(
                    f"{LIB_PATH} is not built; run `python -m tensor_core_gemm_amd.build` "
                    "(hipcc --offload-arch=gfx950)")
            _lib = ctypes.CDLL(LIB_PATH)
    return _lib
