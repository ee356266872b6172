"""ctypes declarations of libeagle31.so (the C ABI in include/eagle31.h).

Loading this module never touches the GPU: it only opens the shared library
and declares argument types.  If the library has not been built, importing
raises immediately; there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeagle31.so")

NORM_NONE = 0
NORM_LAYERNORM = 1
NORM_RMSNORM = 2

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_NORM_KIND = -3
ERR_EPS = -4
ERR_ALIGN = -5
ERR_HIP = -6
ERR_WORKSPACE = -7
ERR_ALIAS = -8
ERR_TOO_LARGE = -9

STATUS_NAMES = {
    OK: "EAGLE31_OK",
    ERR_NULL: "EAGLE31_ERR_NULL",
    ERR_SHAPE: "EAGLE31_ERR_SHAPE",
    ERR_NORM_KIND: "EAGLE31_ERR_NORM_KIND",
    ERR_EPS: "EAGLE31_ERR_EPS",
    ERR_ALIGN: "EAGLE31_ERR_ALIGN",
    ERR_HIP: "EAGLE31_ERR_HIP",
    ERR_WORKSPACE: "EAGLE31_ERR_WORKSPACE",
    ERR_ALIAS: "EAGLE31_ERR_ALIAS",
    ERR_TOO_LARGE: "EAGLE31_ERR_TOO_LARGE",
}

# Every symbol the header declares, with (restype, argtypes).
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_pp = ctypes.POINTER(ctypes.c_void_p)

SIGNATURES = {
    "eagle31_fuse": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _pp, _pp, _vp, _vp, _vp, _vp]),
    "eagle31_workspace_size": (_sz, [_i64, _i64, _int]),
    "eagle31_workspace_init": (_int, [_vp, _sz, _vp]),
    "eagle31_fuse_ws": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _pp, _pp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "eagle31_fold_prepare": (_int, [_i64, _int, _pp, _pp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "eagle31_fuse_folded": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp, _vp]),
    "eagle31_fuse_rows": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _f32, _pp, _pp, _vp, _vp, _vp,
                                 _i64, _vp]),
    "eagle31_fuse_folded_rows": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp,
                                        _i64, _vp]),
    "eagle31_fuse_folded_ws": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp, _vp, _sz,
                                      _vp]),
    "eagle31_fuse_folded_noalloc": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp, _vp]),
    "eagle31_noalloc_scratch_bytes": (_sz, []),
    "eagle31_row_stats": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _f32, _vp, _vp, _vp]),
    "eagle31_norm_output": (_int, [_vp, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp]),
    "eagle31_embed_concat": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "eagle31_verify_accept": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "eagle31_verify_chunking": (_int, [_i64, _i64, _i64, _vp, _vp]),
    "eagle31_status_string": (ctypes.c_char_p, [_int]),
    "eagle31_last_hip_error": (_int, []),
    "eagle31_release": (_int, []),
    "eagle31_debug_stats_recompute": (_int, [_int]),
    "eagle31_debug_fail_workspace_zero": (_int, [_int]),
}


class Eagle31Error(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} returned {STATUS_NAMES.get(status, status)}"
        try:
            msg += f": {lib().eagle31_status_string(status).decode()}"
        except Exception:
            pass
        if status == ERR_HIP:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python eagle_draft_feature_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def ptr_array3(ptrs):
    """const void* const[3] from three integers (or None entries); None -> NULL array."""
    if ptrs is None:
        return None
    arr = (ctypes.c_void_p * 3)(*[(p if p else None) for p in ptrs])
    return ctypes.cast(arr, _pp), arr  # keep arr alive alongside the pointer


def check(fn: str, status: int) -> None:
    if status != OK:
        raise Eagle31Error(fn, status, lib().eagle31_last_hip_error() if status == ERR_HIP else 0)
