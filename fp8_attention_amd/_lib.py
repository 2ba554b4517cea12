"""ctypes declarations of libdm's C ABI (include/dm_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdm.so")

DM_OK, DM_ERR_NULL, DM_ERR_SHAPE, DM_ERR_ALIGN, DM_ERR_ENUM, DM_ERR_HIP, DM_ERR_WORKSPACE = range(7)
DM_E4M3, DM_E5M2 = 0, 1
DM_BF16, DM_F32 = 0, 1
DM_AXIS_COLS, DM_AXIS_ROWS = 0, 1
DM_DELTA_STALE, DM_DELTA_DO_MATCHED, DM_DELTA_MATCHED = 0, 1, 2

# every symbol include/dm_attn.h declares
EXPORTS = ("dm_padded_len", "dm_status_string", "dm_quantize_blockfp8", "dm_attn_fwd", "dm_attn_delta",
           "dm_attn_bwd", "dm_attn_bwd_dkdv", "dm_attn_bwd_dkdv_workspace_size", "dm_attn_bwd_dkdv_ws",
           "dm_attn_bwd_dkdv_noalloc",
           "dm_attn_bwd_dkdv_probes", "dm_attn_bwd_dq", "dm_attn_bwd_dq_probes")
DM_MAX_SEQLEN = 1 << 24
DM_NOALLOC_SCRATCH_BYTES = 128 << 20


class Operand(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class DmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libdm.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python fp8_attention_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.dm_padded_len.argtypes = [i64]
    lib.dm_padded_len.restype = i64
    lib.dm_status_string.argtypes = [i32]
    lib.dm_status_string.restype = ctypes.c_char_p
    lib.dm_quantize_blockfp8.argtypes = [vp, i32, i64, i64, i64, i64, i32, i32, vp, vp, vp]
    lib.dm_quantize_blockfp8.restype = i32
    sp = ctypes.POINTER(Shape)
    lib.dm_attn_fwd.argtypes = [sp, Operand, Operand, Operand, vp, vp, vp]
    lib.dm_attn_fwd.restype = i32
    lib.dm_attn_delta.argtypes = [sp, i32, vp, vp, Operand, Operand, Operand, Operand, vp, vp, vp]
    lib.dm_attn_delta.restype = i32
    lib.dm_attn_bwd.argtypes = [sp] + [Operand] * 7 + [vp] * 7 + [vp]
    lib.dm_attn_bwd.restype = i32
    lib.dm_attn_bwd_dkdv.argtypes = [sp] + [Operand] * 6 + [vp] * 4 + [vp]
    lib.dm_attn_bwd_dkdv.restype = i32
    lib.dm_attn_bwd_dkdv_workspace_size.argtypes = [sp, ctypes.POINTER(i64)]
    lib.dm_attn_bwd_dkdv_workspace_size.restype = i32
    lib.dm_attn_bwd_dkdv_ws.argtypes = [sp] + [Operand] * 6 + [vp] * 5 + [i64, vp]
    lib.dm_attn_bwd_dkdv_ws.restype = i32
    lib.dm_attn_bwd_dkdv_noalloc.argtypes = [sp] + [Operand] * 6 + [vp] * 4 + [vp]
    lib.dm_attn_bwd_dkdv_noalloc.restype = i32
    lib.dm_attn_bwd_dkdv_probes.argtypes = [sp] + [Operand] * 6 + [vp] * 6 + [vp]
    lib.dm_attn_bwd_dkdv_probes.restype = i32
    lib.dm_attn_bwd_dq.argtypes = [sp] + [Operand] * 5 + [vp] * 5 + [vp]
    lib.dm_attn_bwd_dq.restype = i32
    lib.dm_attn_bwd_dq_probes.argtypes = [sp] + [Operand] * 5 + [vp] * 6 + [vp]
    lib.dm_attn_bwd_dq_probes.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dm_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != DM_OK:
        raise DmError(status, where)
