"""ctypes binding of libep_probe.so (include/ep_probe.h): the measurement
kernels a benchmark runs beside the library's operations as same-traffic
ceilings.  They are not part of the method; nothing in the package calls
them.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

from . import abi

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libep_probe.so")

EXPORTS = ("ep_probe_write", "ep_probe_pack", "ep_probe_reduce", "ep_probe_empty",
           "ep_probe_ll_copy", "ep_probe_ll_reduce")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python combine_get_dispatch_05_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "ep_probe_write": [vp, i64, vp],
            "ep_probe_pack": [vp, i32, i32, vp, i32, vp, vp],
            "ep_probe_reduce": [vp, i32, i32, vp, i32, vp, vp],
            "ep_probe_empty": [i32, i32, vp],
            "ep_probe_ll_copy": [vp, i32, i32, i32, vp, vp],
            "ep_probe_ll_reduce": [vp, vp, i32, i32, i32, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int, fn: str) -> None:
    abi.check(rc, fn)
