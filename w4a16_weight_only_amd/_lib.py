"""ctypes loader for libawq_w4a16.so (the C ABI declared in include/awq_w4a16.h).

Argument marshalling only: every step of the linear runs in the HIP library.
If the library is missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libawq_w4a16.so")

AWQ_OK = 0
AWQ_ERR_NULL = -1
AWQ_ERR_SHAPE = -2
AWQ_ERR_GROUP = -3
AWQ_ERR_ALIGN = -4
AWQ_ERR_UNSUPPORTED = -5
AWQ_ERR_HIP = -6

# Every function include/awq_w4a16.h declares, with its ctypes signature.
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_validate_pack": (ctypes.c_int, [_i64] * 10),
    "awq_check_limits": (ctypes.c_int, [_i64] * 4),
    "awq_release_workspace": (ctypes.c_int, []),
    "awq_dequant": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "awq_dequant_f16": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "awq_quantize_rtn": (ctypes.c_int, [_vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp]),
    "awq_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp]),
    "awq_moe_tiles": (ctypes.c_int64, [_i64, _i64, _i64]),
    "awq_moe_align": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "awq_moe_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp]),
    "awq_gemm_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp]),
    "awq_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp]),
    "awq_gemm_plan": (ctypes.c_int, [_i64, _i64, _i64, _i64,
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)]),
    "awq_gemm_plan_tail": (ctypes.c_int, [_i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


class AwqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load the library once.  torch is imported first so that the library binds to
    the HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's libamdhip64 before ours)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4a16_weight_only_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().awq_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status == AWQ_OK:
        return
    if status in (AWQ_ERR_SHAPE, AWQ_ERR_GROUP, AWQ_ERR_UNSUPPORTED, AWQ_ERR_ALIGN, AWQ_ERR_NULL):
        raise ValueError(f"{where}: {status_string(status)} (status {status})")
    raise AwqError(status, where)
