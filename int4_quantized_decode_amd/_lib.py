"""ctypes view of libqdecode.so (the C ABI in include/qdecode.h).

Argument marshalling only.  The library is required: there is no fallback,
and importing this module fails loudly when the built library is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdecode.so")

QD_OK = 0
QD_FMT_INT8_B32 = 1
QD_FMT_INT4_G64 = 2
QD_FMT_FP16 = 3
QD_MAX_K = 24576
QD_MAX_M = 16

STATUS_NAMES = {0: "QD_OK", 1: "QD_EINVAL", 2: "QD_ESHAPE", 3: "QD_EALIGN", 4: "QD_ERANGE",
                5: "QD_ELAUNCH", 6: "QD_EFORMAT", 7: "QD_EDEVICE"}


class QDWeight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


QD_PRO_NONE, QD_PRO_RMSNORM, QD_PRO_GLU = 0, 1, 2
QD_EPI_NONE, QD_EPI_SILU = 0, 1


class QDLinearOp(ctypes.Structure):
    _fields_ = [("w", QDWeight), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("group", ctypes.c_int32), ("prologue", ctypes.c_int32),
                ("gamma", ctypes.c_void_p), ("eps", ctypes.c_float), ("epilogue", ctypes.c_int32)]


# name -> (restype, argtypes), mirroring include/qdecode.h
SIGNATURES = {
    "qd_packed_bytes": (ctypes.c_uint64, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]),
    "qd_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "qpack_int8_b32": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "qpack_int4_g64": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "qpack_fp16": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "qgemv_int8_b32": (ctypes.c_int32, [ctypes.POINTER(QDWeight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "qgemv_int4_g64": (ctypes.c_int32, [ctypes.POINTER(QDWeight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "qgemv_fp16": (ctypes.c_int32, [ctypes.POINTER(QDWeight), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "qgemm_small_m": (ctypes.c_int32, [ctypes.POINTER(QDWeight), ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "decode_linear_stack": (ctypes.c_int32, [ctypes.POINTER(QDLinearOp), ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p]),
    "qd_stack_plan_create": (ctypes.c_int32, [ctypes.POINTER(QDLinearOp), ctypes.c_int64,
                                              ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)]),
    "qd_stack_plan_run": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p]),
    "qd_stack_plan_error": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    "qd_stack_plan_is_persistent": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    "qd_stack_plan_set_spin_limit": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_uint32]),
    "qd_stack_plan_describe": (ctypes.c_int32, [ctypes.POINTER(QDLinearOp), ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                                ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "qd_read_probe": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p]),
    "qd_stack_plan_destroy": (None, [ctypes.c_void_p]),
    "qd_stack_run_noalloc": (ctypes.c_int32, [ctypes.POINTER(QDLinearOp), ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_void_p]),
}


class QDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({lib.qd_status_string(status).decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python int4_quantized_decode_amd/build.py)")
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


def check(status: int, where: str) -> None:
    if status != QD_OK:
        raise QDError(status, where)
