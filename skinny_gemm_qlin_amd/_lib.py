"""ctypes binding of libqlin.so (the C ABI declared in include/qlin.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  There is no fallback of any kind: if the library
is missing, or a call returns an error status, a QlinError is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlin.so")

QLIN_OK = 0
QLIN_ERR_NULL = -1
QLIN_ERR_SHAPE = -2
QLIN_ERR_STRIDE = -3
QLIN_ERR_ALIGN = -4
QLIN_ERR_WORKSPACE = -5
QLIN_ERR_ARG = -6
QLIN_ERR_LAUNCH = -7

EXPORTS = (
    "qlin_status_str", "qlin_version", "qlin_act_quant_i8", "qlin_gemv_i8", "qlin_gemv_fp8",
    "qlin_gemv_fp8_blk", "qlin_moe_mxfp4_workspace_bytes", "qlin_moe_mxfp4",
    "qlin_moe_ffn_mxfp4_workspace_bytes", "qlin_moe_ffn_mxfp4", "qlin_act_quant_fp8", "qlin_gemv_fp8_w8a8",
    "qlin_gemv_fp8_blk_ex", "qlin_moe_mxfp4_noalloc", "qlin_linear_i8",
)

QLIN_FMT_E4M3 = 0
QLIN_FMT_E5M2 = 1


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libqlin.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.qlin_status_str.argtypes = [I]
    lib.qlin_status_str.restype = ctypes.c_char_p
    lib.qlin_version.restype = I
    lib.qlin_act_quant_i8.argtypes = [P, I64, I64, I64, P, I64, P, P]
    lib.qlin_act_quant_i8.restype = I
    lib.qlin_gemv_i8.argtypes = [P, I64, P, I, I64, I64, P, I64, I64, P, I, P, P, I64, I, P]
    lib.qlin_gemv_i8.restype = I
    lib.qlin_linear_i8.argtypes = [P, I64, I64, I64, P, I64, I64, P, I, P, P, I64, P, P, I64, P]
    lib.qlin_linear_i8.restype = I
    lib.qlin_gemv_fp8.argtypes = [P, I64, I64, I64, P, I64, I64, P, I, P, I64, P]
    lib.qlin_gemv_fp8.restype = I
    lib.qlin_act_quant_fp8.argtypes = [P, I64, I64, I64, I, I, P, I64, P, P]
    lib.qlin_act_quant_fp8.restype = I
    lib.qlin_gemv_fp8_w8a8.argtypes = [P, I64, P, I, I, I64, I64, P, I64, I64, P, I, I, P, I64, P]
    lib.qlin_gemv_fp8_w8a8.restype = I
    lib.qlin_gemv_fp8_blk.argtypes = [P, I64, I64, I64, P, I64, I64, P, P, P, P, I64, P]
    lib.qlin_gemv_fp8_blk.restype = I
    lib.qlin_gemv_fp8_blk_ex.argtypes = [P, I64, I64, I64, P, I64, I64, P, I64, I64, P, P, P, I64, P]
    lib.qlin_gemv_fp8_blk_ex.restype = I
    lib.qlin_moe_mxfp4_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.qlin_moe_mxfp4_workspace_bytes.restype = SZ
    lib.qlin_moe_mxfp4.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, I64, P, I64, P, SZ, P]
    lib.qlin_moe_mxfp4.restype = I
    lib.qlin_moe_mxfp4_noalloc.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, I64, P, I64, P]
    lib.qlin_moe_mxfp4_noalloc.restype = I
    lib.qlin_moe_ffn_mxfp4_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
    lib.qlin_moe_ffn_mxfp4_workspace_bytes.restype = SZ
    F = ctypes.c_float
    lib.qlin_moe_ffn_mxfp4.argtypes = [P, I64, I64, I64, P, I64, I64, P, P, I64, P, P, F, F, P, P, P, I64,
                                       P, SZ, P]
    lib.qlin_moe_ffn_mxfp4.restype = I
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().qlin_status_str(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != QLIN_OK:
        raise QlinError(status, where)
