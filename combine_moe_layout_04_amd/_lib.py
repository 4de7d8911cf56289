"""ctypes loader for libmoe_layout.so (the HIP library built in-tree).

There is no fallback: if the library is missing every call raises, so a
product path can never silently run anything but the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_layout.so")

c_int, c_int64, c_size_t, c_void_p = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
c_char_p = ctypes.c_char_p


class MoeTuning(ctypes.Structure):
    _fields_ = [("chunks_per_lane", c_int), ("nontemporal", c_int), ("waves_per_block", c_int),
                ("layout_pairs", c_int), ("gather_mode", c_int)]


# name -> (restype, argtypes); the functions declared in include/moe_layout.h and
# include/moe_bench.h (the measurement entry points)
SIGNATURES = {
    "moe_workspace_size": (c_int, [c_int64, c_int, c_int, c_int, ctypes.POINTER(c_size_t)]),
    "moe_handle_create": (c_int, [ctypes.POINTER(c_void_p), ctypes.POINTER(MoeTuning)]),
    "moe_workspace_size_padded": (c_int, [c_int64, c_int, c_int, c_int, c_int, ctypes.POINTER(c_size_t)]),
    "moe_handle_create_padded": (c_int, [ctypes.POINTER(c_void_p), ctypes.POINTER(MoeTuning), c_int]),
    "moe_recv_capacity": (c_int, [c_void_p, ctypes.POINTER(c_int64)]),
    "moe_handle_destroy": (c_int, [c_void_p]),
    "moe_layout": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int, c_int, c_int, c_void_p,
                           c_size_t, c_void_p]),
    "moe_layout_noalloc": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int, c_int, c_int, c_void_p,
                                   c_size_t, c_void_p]),
    "moe_dispatch": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_int, c_void_p,
                             c_void_p, c_void_p]),
    "moe_combine": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_void_p, c_void_p]),
    "moe_combine_bwd": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p]),
    "moe_dispatch_bwd": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p]),
    "moe_send_capacity": (c_int, [c_void_p, ctypes.POINTER(c_int64)]),
    "moe_send": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_int64, c_void_p]),
    "moe_expand": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int64, c_void_p, c_int, c_void_p,
                           c_void_p, c_void_p]),
    "moe_reduce_partitions": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_void_p, c_void_p,
                                      c_int64, c_void_p]),
    "moe_combine_partitions": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int64, c_void_p,
                                       c_void_p]),
    "moe_handle_field": (c_int, [c_void_p, c_int, ctypes.POINTER(c_void_p), ctypes.POINTER(c_size_t)]),
    "moe_handle_dims": (c_int, [c_void_p, ctypes.POINTER(c_int64), ctypes.POINTER(c_int),
                                ctypes.POINTER(c_int), ctypes.POINTER(c_int)]),
    "moe_handle_check": (c_int, [c_void_p, c_void_p, ctypes.POINTER(c_int)]),
    "moe_bench_copy": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_time_next_kernel": (c_int, [c_void_p, c_void_p, c_void_p]),
    "moe_stream_create_cu_budget": (c_int, [c_int, c_int, ctypes.POINTER(c_void_p)]),
    "moe_stream_destroy": (c_int, [c_void_p]),
    "moe_strerror": (c_char_p, [c_int]),
    "moe_version": (c_char_p, []),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB
