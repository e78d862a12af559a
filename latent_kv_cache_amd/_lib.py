"""ctypes view of libmlra.so (declared in include/mlra.h).

Loading is lazy; a missing library raises instead of falling back to any
other implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmlra.so")

MLRA_BF16, MLRA_FP32 = 0, 1
MLRA_BRANCH_SUM, MLRA_BRANCH_CONCAT = 0, 1
MLRA_DECODE_WS_HEADER_BYTES = 65792          # zero before a decode workspace's first use
MLRA_DECODE_FLAG_FUSED_MERGE = 1
MLRA_DEVSTATUS_WAIT_EXPIRED, MLRA_DEVSTATUS_MERGE_FAILED = 1, 2
MLRA_STATIC_SCRATCH_BYTES = 64 << 20   # scratch of mlra_decode_attention_static

STATUS_NAMES = {0: "MLRA_OK", 1: "MLRA_ERR_NULL_PTR", 2: "MLRA_ERR_BAD_DIMS",
                3: "MLRA_ERR_UNSUPPORTED", 4: "MLRA_ERR_WORKSPACE", 5: "MLRA_ERR_ALIGNMENT",
                6: "MLRA_ERR_HIP"}

# Functions include/mlra.h declares (checked against the header by the tests).
EXPORTS = ("mlra_decode_make_plan", "mlra_decode_workspace_size", "mlra_decode_attention",
           "mlra_decode_attention_static",
           "mla_decode_attention", "mlra_decode_partials", "mlra_decode_combine",
           "mlra_cache_append", "mlra_out_projection_pack", "mlra_out_projection_workspace_size",
           "mlra_out_projection", "mlra_prefill_make_plan", "mlra_prefill_workspace_size",
           "mlra_prefill_attention", "mlra_decode_workspace_init", "mlra_decode_read_status",
           "mlra_testing_set_wait_limit", "mlra_stream_read", "mlra_status_string", "mlra_version")


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("reduce", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("latent_stride_block", ctypes.c_int64), ("latent_stride_token", ctypes.c_int64),
        ("latent_stride_branch", ctypes.c_int64), ("rope_stride_block", ctypes.c_int64),
        ("rope_stride_token", ctypes.c_int64), ("sum_seq_lens", ctypes.c_int64),
    ]


class DecodePlan(ctypes.Structure):
    _fields_ = [
        ("num_cus", ctypes.c_int32), ("target_groups", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32), ("tiles_per_split", ctypes.c_int32),
        ("splits_per_seq", ctypes.c_int32), ("kernel_variant", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32), ("row_groups", ctypes.c_int32),
        ("fused_merge", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MlraError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        text = lib.mlra_status_string(status).decode() if lib is not None else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load libmlra.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m latent_kv_cache_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        dims_p = ctypes.POINTER(DecodeDims)
        lib.mlra_decode_make_plan.argtypes = [dims_p, i32, i32, ctypes.POINTER(DecodePlan)]
        lib.mlra_decode_make_plan.restype = i32
        lib.mlra_decode_workspace_size.argtypes = [dims_p, i32, ctypes.POINTER(sz)]
        lib.mlra_decode_workspace_size.restype = i32
        lib.mlra_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, f32, f32, vp, vp,
                                              dims_p, vp, sz, vp]
        lib.mlra_decode_attention.restype = i32
        lib.mlra_decode_attention_static.argtypes = [vp, vp, vp, vp, vp, vp, i32, f32, f32, vp,
                                                     vp, dims_p, vp]
        lib.mlra_decode_attention_static.restype = i32
        lib.mla_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, vp, dims_p, vp,
                                             sz, vp]
        lib.mla_decode_attention.restype = i32
        lib.mlra_decode_partials.argtypes = [vp, vp, vp, vp, vp, vp, i32, f32, dims_p, vp, sz, vp]
        lib.mlra_decode_partials.restype = i32
        lib.mlra_decode_combine.argtypes = [vp, i32, f32, vp, vp, dims_p, vp, sz, vp]
        lib.mlra_decode_combine.restype = i32
        lib.mlra_cache_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, f32, f32, dims_p, vp]
        lib.mlra_cache_append.restype = i32
        lib.mlra_out_projection_pack.argtypes = [vp, vp, i32, i32, vp]
        lib.mlra_out_projection_pack.restype = i32
        lib.mlra_out_projection_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        lib.mlra_out_projection_workspace_size.restype = i32
        lib.mlra_out_projection.argtypes = [vp, vp, vp, i32, i32, i32, vp, sz, vp]
        lib.mlra_out_projection.restype = i32
        lib.mlra_prefill_make_plan.argtypes = [dims_p, i32, i32, ctypes.POINTER(DecodePlan)]
        lib.mlra_prefill_make_plan.restype = i32
        lib.mlra_prefill_workspace_size.argtypes = [dims_p, i32, ctypes.POINTER(sz)]
        lib.mlra_prefill_workspace_size.restype = i32
        lib.mlra_prefill_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, f32, f32, vp, vp,
                                               dims_p, vp, sz, vp]
        lib.mlra_prefill_attention.restype = i32
        lib.mlra_decode_workspace_init.argtypes = [vp, sz, vp]
        lib.mlra_decode_workspace_init.restype = i32
        lib.mlra_decode_read_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), i32, vp]
        lib.mlra_decode_read_status.restype = i32
        lib.mlra_stream_read.argtypes = [vp, sz, i32, vp, vp]
        lib.mlra_stream_read.restype = i32
        lib.mlra_testing_set_wait_limit.argtypes = [i32]
        lib.mlra_testing_set_wait_limit.restype = i32
        lib.mlra_status_string.argtypes = [i32]
        lib.mlra_status_string.restype = ctypes.c_char_p
        lib.mlra_version.argtypes = []
        lib.mlra_version.restype = i32
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise MlraError(status, where, load())
