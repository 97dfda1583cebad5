"""ctypes view of libmcs.so (the C ABI in include/mcs.h)."""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmcs.so")

MCS_SUCCESS = 0
MCS_ERROR_INVALID_VALUE = 1
MCS_ERROR_UNSUPPORTED_SHAPE = 2
MCS_ERROR_MISALIGNED = 3
MCS_ERROR_BUFFER_TOO_SMALL = 4
MCS_ERROR_META_MISMATCH = 5
MCS_ERROR_HIP = 6

MCS_DTYPE_FP32 = 0
MCS_DTYPE_BF16 = 1
MCS_META_VERSION = 3
MCS_HASH_BITS = 8
MCS_VERSION = 3
MCS_SELECT_PHASES = 5
MCS_NOALLOC_SCRATCH_BYTES = 128 << 20
MCS_MAX_SEQ_LEN = 1 << 22

MCS_GROUPING_HASH = 0
MCS_GROUPING_RASTER = 1
MCS_GROUPING_CENTRED_HASH = 2
MCS_GROUPING_MORTON = 3

EXPORTS = ("mcs_version", "mcs_status_string", "mcs_last_hip_error", "mcs_dense_attn", "mcs_meta_layout",
           "mcs_meta_bytes", "mcs_select_workspace_bytes", "mcs_meta_init", "mcs_select", "mcs_select_ex",
           "mcs_sparse_attn", "mcs_select_noalloc", "mcs_meta_layout_ex", "mcs_meta_init_ex",
           "mcs_select_workspace_bytes_ex", "mcs_topk_rows")


class AttnDesc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class Meta(ctypes.Structure):
    _fields_ = [("version", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("max_keep", ctypes.c_int32), ("residual_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("total_idx", ctypes.c_int64),
                ("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64), ("off_perm", ctypes.c_uint64),
                ("off_keep", ctypes.c_uint64), ("off_idx_start", ctypes.c_uint64), ("off_sched", ctypes.c_uint64),
                ("off_count", ctypes.c_uint64), ("off_order", ctypes.c_uint64), ("off_idx", ctypes.c_uint64),
                ("off_residual", ctypes.c_uint64)]


class SelectOptions(ctypes.Structure):
    _fields_ = [("grouping", ctypes.c_int32), ("kv_block", ctypes.c_int32), ("residual", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_y", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("residual_dtype", ctypes.c_int32), ("keep_mass", ctypes.c_float),
                ("phase_events", ctypes.POINTER(ctypes.c_void_p)), ("num_phase_events", ctypes.c_int32)]


class McsError(RuntimeError):
    def __init__(self, status: int, call: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        name = _lib().mcs_status_string(status).decode() if _LIB is not None else str(status)
        extra = f" (hipError {hip_error})" if status == MCS_ERROR_HIP else ""
        super().__init__(f"{call} failed: {name}{extra}")


_LIB = None


def _lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_diffusion_mcs_amd.build` (no CPU fallback exists)")
        _LIB = open_library(LIB_PATH)
    return _LIB


def open_library(path):
    """Loads a libmcs build at `path` and declares its C prototypes."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    DP = ctypes.POINTER(AttnDesc)
    MP = ctypes.POINTER(Meta)
    I32P = ctypes.POINTER(ctypes.c_int32)
    F32P = ctypes.POINTER(ctypes.c_float)
    lib.mcs_version.restype = ctypes.c_int
    lib.mcs_version.argtypes = []
    lib.mcs_status_string.restype = ctypes.c_char_p
    lib.mcs_status_string.argtypes = [ctypes.c_int]
    lib.mcs_last_hip_error.restype = ctypes.c_int
    lib.mcs_last_hip_error.argtypes = []
    lib.mcs_dense_attn.restype = ctypes.c_int
    lib.mcs_dense_attn.argtypes = [DP, P, P, P, P, P]
    lib.mcs_meta_layout.restype = ctypes.c_int
    lib.mcs_meta_layout.argtypes = [DP, ctypes.c_int32, I32P, MP]
    lib.mcs_meta_bytes.restype = ctypes.c_size_t
    lib.mcs_meta_bytes.argtypes = [DP, ctypes.c_int32, I32P]
    lib.mcs_select_workspace_bytes.restype = ctypes.c_size_t
    lib.mcs_select_workspace_bytes.argtypes = [DP, ctypes.c_int32, ctypes.c_int32]
    lib.mcs_meta_init.restype = ctypes.c_int
    lib.mcs_meta_init.argtypes = [DP, ctypes.c_int32, I32P, P, ctypes.c_size_t, MP, P]
    lib.mcs_select.restype = ctypes.c_int
    lib.mcs_select.argtypes = [DP, P, P, P, ctypes.c_int32, I32P, F32P, P, ctypes.c_size_t, P,
                               ctypes.c_size_t, P, MP, P]
    lib.mcs_select_ex.restype = ctypes.c_int
    lib.mcs_select_ex.argtypes = [DP, P, P, P, ctypes.c_int32, I32P, F32P, ctypes.POINTER(SelectOptions), P,
                                  ctypes.c_size_t, P, ctypes.c_size_t, P, MP, P]
    lib.mcs_meta_layout_ex.restype = ctypes.c_int
    lib.mcs_meta_layout_ex.argtypes = [DP, ctypes.c_int32, I32P, ctypes.c_int32, MP]
    lib.mcs_meta_init_ex.restype = ctypes.c_int
    lib.mcs_meta_init_ex.argtypes = [DP, ctypes.c_int32, I32P, ctypes.c_int32, P, ctypes.c_size_t, MP, P]
    lib.mcs_select_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.mcs_select_workspace_bytes_ex.argtypes = [DP, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(SelectOptions)]
    lib.mcs_select_noalloc.restype = ctypes.c_int
    lib.mcs_select_noalloc.argtypes = [DP, P, P, P, ctypes.c_int32, I32P, F32P, ctypes.POINTER(SelectOptions), P,
                                       ctypes.c_size_t, P, MP, P]
    lib.mcs_topk_rows.restype = ctypes.c_int
    lib.mcs_topk_rows.argtypes = [F32P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, P]
    lib.mcs_sparse_attn.restype = ctypes.c_int
    lib.mcs_sparse_attn.argtypes = [DP, P, P, P, MP, P, P]
    return lib


def lib():
    return _lib()


def check(status: int, call: str):
    if status != MCS_SUCCESS:
        raise McsError(status, call, _lib().mcs_last_hip_error() if status == MCS_ERROR_HIP else 0)
