"""ctypes loader for libmoe_dc.so (the C ABI declared in include/moe_dc.h).

The shared library is built in-tree by ``combine_moe_route_topk_amd.build``.
There is no fallback: if the library is missing or cannot be loaded, importing
this module raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_dc.so")

MOE_F32, MOE_BF16, MOE_F8E4M3 = 0, 1, 2
MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_SORT_AUTO, MOE_SORT_OFF, MOE_SORT_ON = -1, 0, 1
MOE_NOALLOC_SCRATCH_BYTES = (1 << 20) + 256      # include/moe_dc.h
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
                4: "MOE_ERR_HIP"}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/moe_dc.h
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route_topk": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _p, _p]),
    "moe_resolve_sorted": (ctypes.c_int, [_i32, _i64, _i32, ctypes.POINTER(_i32)]),
    "moe_dispatch_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_dispatch": (ctypes.c_int, [_p, _p, _i32, _i64, _i64, _p, _i32, _i32, _i32, _i32, _i32,
                                    ctypes.POINTER(_i32), _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    _sz, _p]),
    "moe_route_dispatch_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_route_dispatch": (ctypes.c_int, [_p, _i32, _p, _p, _p, _p, _i32, _i64, _i64, _i32, _i32, _i32,
                                          _i32, _i32, ctypes.POINTER(_i32), _p, _p, _p, _p, _p, _p,
                                          _p, _p, _p, _sz, _p]),
    "moe_route_dispatch_noalloc": (ctypes.c_int, [_p, _i32, _p, _p, _p, _p, _i32, _i64, _i64, _i32,
                                                  _i32, _i32, _i32, _i32, ctypes.POINTER(_i32), _p,
                                                  _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_scatter_rows": (ctypes.c_int, [_p, _i64, _i64, _i32, _p, _p, _p]),
    "moe_gather_rows": (ctypes.c_int, [_p, _i64, _i64, _i32, _p, _i64, _p, _p]),
    "moe_combine": (ctypes.c_int, [_p, _i32, _i64, _i64, _i32, _p, _p, _p, _i32, _p]),
    "moe_dequant_rows": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p]),
    "moe_grouped_swiglu_workspace_bytes": (_sz, [_i64, _i32, _i64, _i64]),
    "moe_grouped_swiglu": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _p, _i64, _p, _p,
                                          _sz, _p]),
    "moe_gather_swiglu_workspace_bytes": (_sz, [_i64, _i32, _i64, _i64]),
    "moe_gather_swiglu": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _p, _i64, _p, _p,
                                         _sz, _p]),
    "moe_gather_swiglu_combine": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _i64, _i32, _i32, _p,
                                                 _p, _p, _i64, _p, _p, _sz, _p]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _i32, _p, _p, _i64, _p, _p]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python combine_moe_route_topk_amd/build.py`; "
            "there is no CPU fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib.moe_last_error().decode(errors="replace")
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
