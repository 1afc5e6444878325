"""ctypes view of libfa.so (the C ABI declared in include/fa.h).

Loading never falls back to anything: a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

# the in-tree build of the library
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_ALIGN",
    5: "FA_ERR_SCALE", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP", 8: "FA_ERR_ALIAS",
}
FA_BF16 = 0
FA_FP16 = 1

# name -> (restype, argtypes); the order follows include/fa.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_lse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                           _P]),
    "fa_fwd_plan": (_I, [_I, _I, _I, _I, _I, _I, _I, _P]),
    "fa_fwd_planned": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "fa_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P, ctypes.c_size_t,
                       _P]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P,
                             ctypes.c_size_t, _P]),
    "fa_decode_multi_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "fa_decode_multi": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                             ctypes.c_size_t, _P]),
    "fa_decode_paged_multi": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _I, _I, _F,
                                   _I, _P, ctypes.c_size_t, _P]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                    ctypes.c_size_t, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
}


class FwdPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("work_items", ctypes.c_int), ("grid", ctypes.c_int),
                ("persistent", ctypes.c_int), ("hkv_major", ctypes.c_int),
                ("kv_tiles", ctypes.c_longlong), ("masked_tiles", ctypes.c_longlong),
                ("xcd_map", ctypes.c_int), ("split_tiles", ctypes.c_int),
                ("queue", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m flash_attention_forward_fwd_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().fa_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
