"""ctypes view of libmla.so (include/mla.h). Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1

PAGE_TOKENS = 64
D_QK = 576
D_V = 512
FP8_RECORD_BYTES = 656
META_INTS = 8

EXPORTED_SYMBOLS = (
    "mla_last_error", "mla_version", "mla_decode_args_size", "mla_device_cu_count", "mla_num_parts",
    "mla_get_metadata", "mla_get_metadata_device", "mla_get_metadata_sparse", "mla_workspace_bytes",
    "mla_workspace_bytes_sparse", "mla_decode_kvcache", "mla_decode_kvcache_noalloc",
    "mla_sparse_prefill_args_size", "mla_sparse_prefill_fwd",
)
SCRATCH_BYTES = 128 << 20      # MLA_SCRATCH_BYTES


class MlaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3),
        ("kvcache", ctypes.c_void_p),
        ("kv_stride", ctypes.c_int64 * 3),
        ("kv_format", ctypes.c_int),
        ("num_pages", ctypes.c_int),
        ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int),
        ("cache_seqlens", ctypes.c_void_p),
        ("tile_metadata", ctypes.c_void_p),
        ("num_parts", ctypes.c_int),
        ("num_splits", ctypes.c_void_p),
        ("batch", ctypes.c_int),
        ("s_q", ctypes.c_int),
        ("h_q", ctypes.c_int),
        ("h_kv", ctypes.c_int),
        ("d_qk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("softmax_scale", ctypes.c_float),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("max_splits", ctypes.c_int),
        ("events", ctypes.c_void_p * 3),
        ("indices", ctypes.c_void_p),
        ("idx_stride", ctypes.c_int64 * 2),
        ("topk", ctypes.c_int),
        ("vcache", ctypes.c_void_p),
        ("vc_stride", ctypes.c_int64 * 3),
    ]


class MlaSparsePrefillArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 2),
        ("kv", ctypes.c_void_p),
        ("kv_stride", ctypes.c_int64 * 2),
        ("indices", ctypes.c_void_p),
        ("idx_stride", ctypes.c_int64 * 2),
        ("s_q", ctypes.c_int),
        ("s_kv", ctypes.c_int),
        ("h_q", ctypes.c_int),
        ("h_kv", ctypes.c_int),
        ("topk", ctypes.c_int),
        ("d_qk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("softmax_scale", ctypes.c_float),
        ("tile_metadata", ctypes.c_void_p),
        ("num_parts", ctypes.c_int),
        ("num_splits", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("max_splits", ctypes.c_int),
        ("events", ctypes.c_void_p * 3),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libmla.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_mla_decode_amd.build` "
                          "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_version.argtypes = []
    lib.mla_decode_args_size.restype = ctypes.c_size_t
    lib.mla_decode_args_size.argtypes = []
    lib.mla_device_cu_count.restype = ctypes.c_int
    lib.mla_device_cu_count.argtypes = [ctypes.c_int]
    lib.mla_num_parts.restype = ctypes.c_int
    lib.mla_num_parts.argtypes = [ctypes.c_int] * 5
    lib.mla_get_metadata.restype = ctypes.c_int
    lib.mla_get_metadata.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, i32p, i32p, ctypes.POINTER(ctypes.c_int)]
    lib.mla_get_metadata_device.restype = ctypes.c_int
    lib.mla_get_metadata_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    lib.mla_get_metadata_sparse.restype = ctypes.c_int
    lib.mla_get_metadata_sparse.argtypes = [ctypes.c_int] * 8 + [i32p, i32p, ctypes.POINTER(ctypes.c_int)]
    lib.mla_workspace_bytes_sparse.restype = ctypes.c_size_t
    lib.mla_workspace_bytes_sparse.argtypes = [ctypes.c_int] * 5
    lib.mla_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_workspace_bytes.argtypes = [ctypes.c_int] * 4
    lib.mla_decode_kvcache.restype = ctypes.c_int
    lib.mla_decode_kvcache.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    lib.mla_decode_kvcache_noalloc.restype = ctypes.c_int
    lib.mla_decode_kvcache_noalloc.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    lib.mla_sparse_prefill_args_size.restype = ctypes.c_size_t
    lib.mla_sparse_prefill_args_size.argtypes = []
    lib.mla_sparse_prefill_fwd.restype = ctypes.c_int
    lib.mla_sparse_prefill_fwd.argtypes = [ctypes.POINTER(MlaSparsePrefillArgs), ctypes.c_void_p]
    if lib.mla_sparse_prefill_args_size() != ctypes.sizeof(MlaSparsePrefillArgs):
        raise ImportError(f"mla_sparse_prefill_args layout mismatch: library {lib.mla_sparse_prefill_args_size()} "
                          f"bytes, binding {ctypes.sizeof(MlaSparsePrefillArgs)} bytes")
    if lib.mla_decode_args_size() != ctypes.sizeof(MlaDecodeArgs):
        raise ImportError(f"mla_decode_args layout mismatch: library {lib.mla_decode_args_size()} bytes, "
                          f"binding {ctypes.sizeof(MlaDecodeArgs)} bytes")
    _lib = lib
    return lib


def last_error() -> str:
    return load().mla_last_error().decode("utf-8", "replace")


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def check(status: int) -> None:
    if status == MLA_OK:
        return
    msg = last_error()
    if status == MLA_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    if status == MLA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise MlaError(status, msg)
