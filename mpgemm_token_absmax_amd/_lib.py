"""ctypes loader for libbitlinear.so (the C ABI in include/bitlinear.h).

Argument marshalling only: no computation happens here. The library must have
been built in-tree (mpgemm_token_absmax_amd/build.py); loading fails loudly
otherwise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitlinear.so")

BL_OK = 0
BL_ERR_NULL = -1
BL_ERR_SHAPE = -2
BL_ERR_ALIGN = -3
BL_ERR_DTYPE = -4
BL_ERR_WORKSPACE = -5
BL_ERR_HIP = -6
BL_ERR_ALIAS = -7

BL_W_F32 = 0
BL_W_TERNARY_I8 = 1

BL_OUT_I32 = 0
BL_OUT_F32 = 1
BL_OUT_BF16 = 2

EXPORTS = ("bl_abi_version", "bl_status_string", "bl_quantize_act",
           "bl_quantize_act_tensor_workspace", "bl_quantize_act_tensor", "bl_rmsnorm_quant",
           "bl_pack_i2s_workspace", "bl_pack_i2s", "bl_pack_t3_row_bytes", "bl_pack_t3",
           "bl_gemv", "bl_gemv_t3", "bl_gemm_workspace", "bl_gemm", "bl_gemm_group_workspace",
           "bl_gemm_group", "bl_gemm_group_noalloc",
           "bl_decode_group", "bl_decode_group_t3", "bl_decode_norm_group")

MAX_GROUP = 8
BL_GEMM_NOALLOC_SCRATCH_BYTES = 32 << 20     # include/bitlinear.h


class DecodeProblem(ctypes.Structure):
    """Mirror of bl_decode_problem (include/bitlinear.h)."""
    _fields_ = [("packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("ytype", ctypes.c_int)]


class GemmProblem(ctypes.Structure):
    """Mirror of bl_gemm_problem (include/bitlinear.h)."""
    _fields_ = [("packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("y", ctypes.c_void_p), ("ytype", ctypes.c_int)]


_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def _declare(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    INT = ctypes.c_int
    SZ = ctypes.c_size_t
    lib.bl_abi_version.restype = INT
    lib.bl_abi_version.argtypes = []
    lib.bl_status_string.restype = ctypes.c_char_p
    lib.bl_status_string.argtypes = [INT]
    lib.bl_quantize_act.restype = INT
    lib.bl_quantize_act.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.bl_pack_i2s_workspace.restype = SZ
    lib.bl_quantize_act_tensor_workspace.restype = SZ
    lib.bl_quantize_act_tensor_workspace.argtypes = [I64]
    lib.bl_quantize_act_tensor.restype = INT
    lib.bl_quantize_act_tensor.argtypes = [P, I64, I64, I64, P, P, P, P, SZ, P]
    lib.bl_pack_i2s_workspace.argtypes = [I64, I64]
    lib.bl_rmsnorm_quant.restype = INT
    lib.bl_rmsnorm_quant.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, P, P, P, P, P]
    lib.bl_pack_i2s.restype = INT
    lib.bl_pack_i2s.argtypes = [P, INT, I64, I64, P, P, P, SZ, P]
    lib.bl_pack_t3_row_bytes.restype = SZ
    lib.bl_pack_t3_row_bytes.argtypes = [I64]
    lib.bl_pack_t3.restype = INT
    lib.bl_pack_t3.argtypes = [P, INT, I64, I64, P, P, P, SZ, P]
    lib.bl_gemv_t3.restype = INT
    lib.bl_gemv_t3.argtypes = [P, P, I64, I64, P, P, I64, P, INT, P]
    lib.bl_gemv.restype = INT
    lib.bl_gemv.argtypes = [P, P, I64, I64, P, P, I64, P, INT, P]
    lib.bl_gemm_workspace.restype = SZ
    lib.bl_gemm_workspace.argtypes = [I64, I64, I64]
    lib.bl_gemm.restype = INT
    lib.bl_gemm.argtypes = [P, P, I64, I64, P, P, P, I64, P, INT, P, SZ, P]
    lib.bl_gemm_group_workspace.restype = SZ
    lib.bl_gemm_group_workspace.argtypes = [ctypes.POINTER(ctypes.c_int64), INT, I64, I64]
    lib.bl_gemm_group.restype = INT
    lib.bl_gemm_group.argtypes = [ctypes.POINTER(GemmProblem), INT, I64, P, P, P, I64, P, SZ, P]
    lib.bl_gemm_group_noalloc.restype = INT
    lib.bl_gemm_group_noalloc.argtypes = [ctypes.POINTER(GemmProblem), INT, I64, P, P, P, I64, P]
    lib.bl_decode_group.restype = INT
    lib.bl_decode_group.argtypes = [ctypes.POINTER(DecodeProblem), INT, I64, P]
    lib.bl_decode_group_t3.restype = INT
    lib.bl_decode_group_t3.argtypes = [ctypes.POINTER(DecodeProblem), INT, I64, P]
    lib.bl_decode_norm_group.restype = INT
    lib.bl_decode_norm_group.argtypes = [ctypes.POINTER(DecodeProblem), INT, P, P, ctypes.c_float,
                                         P, P]
    return lib


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mpgemm_token_absmax_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return lib().bl_status_string(int(status)).decode()


def check(fn: str, status: int):
    if status != BL_OK:
        raise BitLinearError(fn, status)
