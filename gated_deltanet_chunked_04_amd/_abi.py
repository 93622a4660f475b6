"""ctypes mirror of include/gdn.h and the loader of libgdn.so.

Argument marshalling only: every step of the computation runs in the HIP
library. If the library has not been built this module raises; nothing falls
back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(5)
GDN_DTYPE_BF16, GDN_DTYPE_FP32 = 0, 1
CP_MODES = {"auto": 0, "off": 1, "on": 2, "exact": 3, "warmup": 4, "pages": 5}
GDN_FLAG_KEEP_FORWARD, GDN_FLAG_REUSE_FORWARD, GDN_FLAG_QK_L2NORM, GDN_FLAG_BWD_ADJOINT_PASS = 1, 2, 4, 8
GDN_FLAG_FWD_FUSED, GDN_FLAG_FWD_SPLIT, GDN_FLAG_REUSE_CP = 16, 32, 64
GDN_ABI_VERSION = 10
GDN_NOALLOC_SCRATCH_BYTES = 128 << 20

# Declared entry points of include/gdn.h (checked by the ABI test).
EXPORTS = ("gdn_abi_version", "gdn_status_string", "gdn_plan", "gdn_chunk_fwd_workspace_size",
           "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_bwd_workspace_size", "gdn_chunk_bwd", "gdn_intra_chunk",
           "gdn_cp_modes", "gdn_cp_windows", "gdn_recurrent_fwd", "gdn_profile_enable", "gdn_profile_read")


class GdnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
        ("K", ctypes.c_int64), ("V", ctypes.c_int64),
        ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("cp_mode", ctypes.c_int32), ("warmup_chunks", ctypes.c_int32),
        ("seg_chunks", ctypes.c_int32), ("warmup_eps", ctypes.c_float),
        ("num_cus", ctypes.c_int32), ("flags", ctypes.c_int32), ("warmup_max_chunks", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 5),
        ("cp_states", ctypes.c_void_p),
    ]


class GdnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("cp_on", ctypes.c_int32), ("seg_chunks", ctypes.c_int32),
        ("warmup_chunks", ctypes.c_int32), ("warmup_max_chunks", ctypes.c_int32),
        ("warmup_eps", ctypes.c_float), ("v_tiles", ctypes.c_int32),
        ("max_len", ctypes.c_int64), ("total_chunks", ctypes.c_int64),
        ("total_segments", ctypes.c_int64),
        ("fwd_workspace_bytes", ctypes.c_size_t), ("bwd_workspace_bytes", ctypes.c_size_t),
        ("cp_states_bytes", ctypes.c_size_t),
        ("fused_fwd", ctypes.c_int32), ("bwd_carried", ctypes.c_int32),
        ("reserved_out", ctypes.c_int32 * 2),
    ]


class GdnKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_LIB = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libgdn.so (built by gated_deltanet_chunked_04_amd.build). Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"libgdn.so not found at {path}: build it first "
                           "(python gated_deltanet_chunked_04_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(GdnDesc)
    lib.gdn_abi_version.restype = i32
    lib.gdn_abi_version.argtypes = []
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_plan.restype = i32
    lib.gdn_plan.argtypes = [dp, ctypes.POINTER(GdnPlanInfo)]
    for f in ("gdn_chunk_fwd_workspace_size", "gdn_chunk_bwd_workspace_size"):
        getattr(lib, f).restype = i32
        getattr(lib, f).argtypes = [dp, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd.restype = i32
    lib.gdn_chunk_fwd.argtypes = [dp] + [vp] * 8 + [vp, sz, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i32
    lib.gdn_chunk_fwd_noalloc.argtypes = [dp] + [vp] * 8 + [vp]
    lib.gdn_chunk_bwd.restype = i32
    lib.gdn_chunk_bwd.argtypes = [dp] + [vp] * 14 + [vp, sz, vp]
    lib.gdn_intra_chunk.restype = i32
    lib.gdn_intra_chunk.argtypes = [dp] + [vp] * 7 + [vp, sz, vp]
    lib.gdn_cp_modes.restype = i32
    lib.gdn_cp_modes.argtypes = [dp] + [vp] * 5 + [vp, sz, vp]
    lib.gdn_cp_windows.restype = i32
    lib.gdn_cp_windows.argtypes = [dp] + [vp] * 6 + [vp, sz, vp]
    lib.gdn_recurrent_fwd.restype = i32
    lib.gdn_recurrent_fwd.argtypes = [dp] + [vp] * 8 + [vp]
    lib.gdn_profile_enable.restype = i32
    lib.gdn_profile_enable.argtypes = [i32]
    lib.gdn_profile_read.restype = i32
    lib.gdn_profile_read.argtypes = [ctypes.POINTER(GdnKernelTime), i32]
    if lib.gdn_abi_version() != GDN_ABI_VERSION:
        raise RuntimeError(f"libgdn.so ABI version {lib.gdn_abi_version()} != {GDN_ABI_VERSION}: rebuild it")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().gdn_status_string(int(status)).decode()


def check(status: int, where: str):
    if status != GDN_OK:
        raise GdnError(status, where)
