"""ctypes view of libmgs.so (include/mgs.h)."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libmgs.so")

MGS_OK = 0
MGS_ERR_INVALID_ARG = 1
MGS_ERR_UNSUPPORTED = 2
MGS_ERR_HIP = 3
MGS_FLAG_POW2_SCALE = 1
MGS_FLAG_VALIDATE = 2
MGS_MX_FLOOR = 0
MGS_MX_RCEIL = 1
MGS_MAX_GROUPS = 1024
MGS_DIM1_MAX_K = 131072
MGS_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "mgs_quant_groups_dim0", "mgs_dim0_workspace_bytes", "mgs_quant_groups_dim0_ws",
    "mgs_quant_groups_dim0_noalloc",
    "mgs_quant_groups_dim0_t", "mgs_quant_experts_dim1",
    "mgs_quant_groups_dim1", "mgs_mx_quant_dim0",
    "mgs_mx_quant_dim1", "mgs_mx_dequant_dim0", "mgs_cast_e4m3",
    "mgs_copy", "mgs_test_quant_dim0", "mgs_status_string", "mgs_last_hip_error",
)

_lock = threading.Lock()
_lib = None


class MgsError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__("%s failed: %s (status %d)%s" % (fn, _status_text(status), status, detail))


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Loads libmgs.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "libmgs.so not found at %s: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` or `python group_scaling_fp8_amd/build.py`" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        for name in ("mgs_quant_groups_dim0", "mgs_quant_groups_dim0_noalloc", "mgs_quant_groups_dim1"):
            fn = getattr(L, name)
            fn.argtypes = [vp, i64, i64, vp, i32, u32, vp, vp, vp]
            fn.restype = ctypes.c_int
        for name in ("mgs_quant_groups_dim0_ws", "mgs_quant_groups_dim0_t"):
            fn = getattr(L, name)
            fn.argtypes = [vp, i64, i64, vp, i32, u32, vp, vp, vp, i64, vp]
            fn.restype = ctypes.c_int
        L.mgs_dim0_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(i64)]
        L.mgs_dim0_workspace_bytes.restype = ctypes.c_int
        L.mgs_mx_quant_dim0.argtypes = [vp, i64, i64, vp, i32, ctypes.c_int, vp, vp, vp]
        L.mgs_mx_quant_dim0.restype = ctypes.c_int
        L.mgs_quant_experts_dim1.argtypes = [vp, i64, i64, i64, u32, vp, vp, vp, i64, vp]
        L.mgs_quant_experts_dim1.restype = ctypes.c_int
        L.mgs_test_quant_dim0.argtypes = [vp, i64, i64, vp, i32, i64, u32, ctypes.c_int, vp, vp, vp,
                                          i64, i64, i32, vp]
        L.mgs_test_quant_dim0.restype = ctypes.c_int
        L.mgs_mx_quant_dim1.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp]
        L.mgs_mx_quant_dim1.restype = ctypes.c_int
        L.mgs_mx_dequant_dim0.argtypes = [vp, vp, i64, i64, vp, vp]
        L.mgs_mx_dequant_dim0.restype = ctypes.c_int
        L.mgs_cast_e4m3.argtypes = [vp, i64, vp, vp]
        L.mgs_cast_e4m3.restype = ctypes.c_int
        L.mgs_copy.argtypes = [vp, vp, i64, vp]
        L.mgs_copy.restype = ctypes.c_int
        L.mgs_status_string.argtypes = [ctypes.c_int]
        L.mgs_status_string.restype = ctypes.c_char_p
        L.mgs_last_hip_error.argtypes = []
        L.mgs_last_hip_error.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_text(status: int) -> str:
    try:
        return lib().mgs_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "status"


def check(fn: str, status: int) -> None:
    if status != MGS_OK:
        detail = ""
        if status == MGS_ERR_HIP:
            detail = ", hipError %d" % lib().mgs_last_hip_error()
        raise MgsError(fn, status, detail)
