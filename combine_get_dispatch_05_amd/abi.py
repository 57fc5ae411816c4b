"""ctypes binding of libep.so (the C ABI declared in include/ep.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are passed as raw device pointers; streams as the raw
hipStream_t of torch's current stream.  If the library has not been built
this module raises at import time -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep.so")

EP_OK = 0
EP_ERR_INVALID = 1
EP_ERR_ALIGN = 2
EP_ERR_CAPACITY = 3
EP_ERR_HANDLE = 4
EP_ERR_HIP = 5
EP_ERR_NOMEM = 6
EP_ERR_TOO_LARGE = 7

# Every function include/ep.h declares (checked against the header by the tests).
EXPORTS = (
    "ep_max_recv_rows", "ep_get_dispatch_layout", "ep_dispatch", "ep_combine",
    "ep_ll_dispatch", "ep_ll_combine", "ep_handle_copy_layout", "ep_handle_num_recv",
    "ep_handle_dims", "ep_handle_nbytes", "ep_handle_free", "ep_pool_trim", "ep_status_str",
    "ep_last_hip_error", "ep_version", "ep_set_tuning", "ep_tuning_list", "ep_ll_dispatch_fp8",
    "ep_ll_combine_fp8", "ep_mask_update", "ep_mask_clean", "ep_mask_query", "ep_lb_prefetch_weights",
    "ep_lb_reduce_grads", "ep_pool_stats", "ep_get_dispatch_layout_noalloc",
)


class Dims(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32), ("num_channels", ctypes.c_int32)]


class LayoutOut(ctypes.Structure):
    _fields_ = [("num_tokens_per_rank", ctypes.c_void_p),
                ("num_tokens_per_expert", ctypes.c_void_p),
                ("is_token_in_rank", ctypes.c_void_p),
                ("rank_prefix_matrix", ctypes.c_void_p),
                ("channel_prefix_matrix", ctypes.c_void_p),
                ("recv_channel_prefix_matrix", ctypes.c_void_p),
                ("send_head", ctypes.c_void_p),
                ("recv_src_idx", ctypes.c_void_p),
                ("recv_src_cap", ctypes.c_int64)]


class EpError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        text = _lib.ep_status_str(code).decode()
        hip = _lib.ep_last_hip_error().decode() if code == EP_ERR_HIP else ""
        super().__init__(f"{fn} failed: {text} ({code}){': ' + hip if hip else ''}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python combine_get_dispatch_05_amd/build.py` (or __graft_entry__.build())")
    # torch ships its own HIP runtime.  Loading torch first makes libep.so
    # bind to that same runtime instance (its DT_NEEDED soname then matches
    # the already loaded copy), so the streams and device pointers torch hands
    # over are valid inside the library.  Loading libep.so first would pull
    # in a second, independent runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pdims, pout = ctypes.POINTER(Dims), ctypes.POINTER(LayoutOut)
    sig = {
        "ep_max_recv_rows": (i64, [pdims]),
        "ep_get_dispatch_layout": (ctypes.c_int, [pdims, vp, vp, pout, ctypes.POINTER(vp), vp]),
        "ep_get_dispatch_layout_noalloc": (ctypes.c_int, [pdims, vp, vp, pout, vp]),
        "ep_dispatch": (ctypes.c_int, [pdims, vp, vp, vp, vp, ctypes.POINTER(vp), vp, vp, vp, i64,
                                       ctypes.POINTER(i64), vp]),
        "ep_combine": (ctypes.c_int, [vp, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp]),
        "ep_ll_dispatch": (ctypes.c_int, [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "ep_ll_dispatch_fp8": (ctypes.c_int, [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "ep_ll_combine": (ctypes.c_int, [pdims, i32, vp, vp, vp, vp, vp, vp, vp]),
        "ep_ll_combine_fp8": (ctypes.c_int, [pdims, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "ep_mask_update": (ctypes.c_int, [vp, i32, i32, i32, vp]),
        "ep_mask_clean": (ctypes.c_int, [vp, i32, vp]),
        "ep_mask_query": (ctypes.c_int, [vp, i32, vp, vp]),
        "ep_lb_prefetch_weights": (ctypes.c_int, [vp, vp, vp, i32, i32, i64, vp]),
        "ep_lb_reduce_grads": (ctypes.c_int, [vp, vp, vp, i32, i32, i64, vp]),
        "ep_handle_copy_layout": (ctypes.c_int, [vp, pout, vp]),
        "ep_handle_num_recv": (ctypes.c_int, [vp, ctypes.POINTER(i64)]),
        "ep_handle_dims": (ctypes.c_int, [vp, pdims]),
        "ep_handle_nbytes": (ctypes.c_size_t, [vp]),
        "ep_handle_free": (None, [vp]),
        "ep_pool_trim": (ctypes.c_int, []),
        "ep_pool_stats": (ctypes.c_int, [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i32),
                                         ctypes.POINTER(ctypes.c_size_t)]),
        "ep_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "ep_last_hip_error": (ctypes.c_char_p, []),
        "ep_version": (ctypes.c_int, []),
        "ep_set_tuning": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int]),
        "ep_tuning_list": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def check(rc: int, fn: str) -> None:
    if rc != EP_OK:
        raise EpError(rc, fn)


def dims(T: int, H: int, K: int, E: int, R: int, C: int = 1) -> Dims:
    return Dims(int(T), int(H), int(K), int(E), int(R), int(C))


def ptr(t):
    """Raw device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def current_stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def tunings(op: str) -> list:
    """All compiled-in launch shapes of ``op`` ("dispatch" or "combine")."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    n = _lib.ep_tuning_list(op.encode(), -1, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    out = []
    for i in range(max(n, 0)):
        _lib.ep_tuning_list(op.encode(), i, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
        out.append((a.value, b.value, c.value))
    return out


def set_tuning(op: str, *shape: int) -> None:
    """Override the launch shape of ``op`` (no arguments: back to default)."""
    vals = list(shape) + [-1] * (3 - len(shape)) if shape else [-1, -1, -1]
    check(_lib.ep_set_tuning(op.encode(), *vals), "ep_set_tuning")


def pool_stats() -> tuple:
    """(bytes kept, arenas kept, byte cap) of the current device's handle pool."""
    kb, n, cap = ctypes.c_size_t(), ctypes.c_int32(), ctypes.c_size_t()
    check(_lib.ep_pool_stats(ctypes.byref(kb), ctypes.byref(n), ctypes.byref(cap)),
          "ep_pool_stats")
    return int(kb.value), int(n.value), int(cap.value)


def version() -> tuple:
    v = _lib.ep_version()
    return (v >> 16, v & 0xFFFF)
