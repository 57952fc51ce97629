"""ctypes declarations of libnsa_cmp.so (include/nsa_cmp.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa_cmp.so")

NSA_OK = 0
NSA_ERR_NULLPTR = 1
NSA_ERR_DTYPE = 2
NSA_ERR_SHAPE = 3
NSA_ERR_CONSTRAINT = 4
NSA_ERR_WORKSPACE = 5
NSA_ERR_UNSUPPORTED = 6
NSA_ERR_HIP = 7

NSA_DTYPE_BF16 = 0
NSA_DTYPE_FP16 = 1

# Every symbol include/nsa_cmp.h declares.
EXPORTS = (
    "nsa_compress_out_len",
    "nsa_compress",
    "nsa_compress_attention_get_workspace",
    "nsa_compress_attention_get_workspace_kv",
    "nsa_compress_attention",
    "nsa_compress_attention_noalloc",
    "nsa_compress_attention_fwd",
    "nsa_compress_attention_split_workspace",
    "nsa_compress_attention_fwd_split",
    "nsa_compress_attention_select",
    "nsa_compress_attention_masked",
    "nsa_compress_attention_fwd_masked",
    "nsa_compress_attention_select_masked",
    "nsa_select_attention",
    "nsa_compress_attention_backward",
    "nsa_compress_backward",
    "nsa_plan_get_info",
    "nsa_plan_destroy",
    "nsa_compress_attention_device_plan",
    "nsa_compress_attention_metadata",
    "nsa_status_string",
    "nsa_last_error",
)


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("total_q_tokens", ctypes.c_int64),
        ("total_cmp_tokens", ctypes.c_int64),
        ("total_sel_blocks", ctypes.c_int64),
        ("max_sel_blocks", ctypes.c_int64),
        ("head_num", ctypes.c_int64),
        ("kv_head_num", ctypes.c_int64),
        ("d1", ctypes.c_int64),
        ("d2", ctypes.c_int64),
        ("select_block_count", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("dtype", ctypes.c_int64),
        ("masked_workspace_bytes", ctypes.c_size_t),
        ("backward_workspace_bytes", ctypes.c_size_t),
        ("total_kv_tokens", ctypes.c_int64),
        ("device_metadata", ctypes.c_int64),
        ("status_offset", ctypes.c_int64),
    ]


class Masks(ctypes.Structure):
    """nsa_masks: device byte matrices (NULL = the positional rule)."""
    _fields_ = [
        ("atten_mask", ctypes.c_void_p),
        ("atten_rows", ctypes.c_int64),
        ("atten_cols", ctypes.c_int64),
        ("topk_mask", ctypes.c_void_p),
        ("topk_rows", ctypes.c_int64),
        ("topk_cols", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kv_compression_block_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int
    lib.nsa_compress_out_len.argtypes = [I64, I64, I64]
    lib.nsa_compress_out_len.restype = I64
    lib.nsa_compress.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, I32, P, I64, P]
    lib.nsa_compress.restype = I32
    lib.nsa_compress_attention_get_workspace.argtypes = [
        I64, P, P, P, I64, I64, I64, I64, ctypes.c_float, I64, I64, I64, I64, I32,
        ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_void_p)]
    lib.nsa_compress_attention_get_workspace.restype = I32
    lib.nsa_compress_attention_get_workspace_kv.argtypes = [
        ctypes.c_int64, P, P, P, P] + lib.nsa_compress_attention_get_workspace.argtypes[4:]
    lib.nsa_compress_attention_get_workspace_kv.restype = I32
    lib.nsa_compress_attention.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention.restype = I32
    lib.nsa_compress_attention_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P]
    lib.nsa_compress_attention_noalloc.restype = I32
    lib.nsa_compress_attention_fwd.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_fwd.restype = I32
    lib.nsa_compress_attention_split_workspace.argtypes = [P, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    lib.nsa_compress_attention_split_workspace.restype = I32
    lib.nsa_compress_attention_fwd_split.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_fwd_split.restype = I32
    lib.nsa_compress_attention_select.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_select.restype = I32
    MP = ctypes.POINTER(Masks)
    lib.nsa_compress_attention_masked.argtypes = [P, P, P, P, MP, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_masked.restype = I32
    lib.nsa_compress_attention_fwd_masked.argtypes = [P, P, P, P, MP, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_fwd_masked.restype = I32
    lib.nsa_compress_attention_select_masked.argtypes = [P, P, P, MP, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_select_masked.restype = I32
    lib.nsa_select_attention.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_select_attention.restype = I32
    lib.nsa_compress_attention_backward.argtypes = [P] * 12 + [ctypes.c_size_t, P]
    lib.nsa_compress_attention_backward.restype = I32
    lib.nsa_compress_backward.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, I32, I64, P, P, P]
    lib.nsa_compress_backward.restype = I32
    lib.nsa_plan_get_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.nsa_plan_get_info.restype = I32
    lib.nsa_plan_destroy.argtypes = [P]
    lib.nsa_plan_destroy.restype = None
    lib.nsa_compress_attention_device_plan.argtypes = [P, ctypes.POINTER(ctypes.c_void_p)]
    lib.nsa_compress_attention_device_plan.restype = I32
    lib.nsa_compress_attention_metadata.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.nsa_compress_attention_metadata.restype = I32
    lib.nsa_status_string.argtypes = [I32]
    lib.nsa_status_string.restype = ctypes.c_char_p
    lib.nsa_last_error.argtypes = []
    lib.nsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class NsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{status_name(status)}: {detail}")


def status_name(status: int) -> str:
    return load().nsa_status_string(status).decode()


def check(status: int) -> None:
    """Raise the Python exception the operator page names for a status:
    TypeError for a wrong type, ValueError for a shape or constraint
    violation; NotImplementedError for legal-but-unbuilt cases and
    RuntimeError for runtime failures."""
    if status == NSA_OK:
        return
    detail = load().nsa_last_error().decode()
    msg = f"{status_name(status)}: {detail}"
    if status == NSA_ERR_DTYPE:
        raise TypeError(msg)
    if status in (NSA_ERR_SHAPE, NSA_ERR_CONSTRAINT, NSA_ERR_NULLPTR, NSA_ERR_WORKSPACE):
        raise ValueError(msg)
    if status == NSA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise NsaError(status, detail)
