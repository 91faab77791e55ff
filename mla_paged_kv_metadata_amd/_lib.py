"""ctypes loader for libmla.so (the C ABI declared in include/mla.h).

The library is built in-tree by mla_paged_kv_metadata_amd.build; loading
fails loudly when it is missing, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB_PATH selects another build of the same library (the sanitizer
# test loads a host-instrumented copy that way).
LIB_PATH = os.environ.get("MLA_LIB_PATH") or os.path.join(_HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE_TOO_SMALL = -3
MLA_ERR_HIP = -4

MLA_KV_BF16 = 0
MLA_KV_FP8_656 = 1

EXPORTED = (
    "mla_metadata_size",
    "mla_metadata_size_for_parts",
    "mla_get_metadata",
    "mla_workspace_size",
    "mla_decode_kvcache",
    "mla_decode_kvcache_noalloc",
    "mla_decode_partial",
    "mla_decode_combine",
    "mla_validate_inputs",
    "mla_validate_host_inputs",
    "mla_append_kv",
    "mla_last_error",
    "mla_version",
)


class MlaDecodeArgs(ctypes.Structure):
    """Mirror of mla_decode_args in include/mla.h (field order matters)."""
    _fields_ = [
        ("batch", ctypes.c_int),
        ("s_q", ctypes.c_int),
        ("h_q", ctypes.c_int),
        ("h_kv", ctypes.c_int),
        ("d_qk", ctypes.c_int),
        ("d_v", ctypes.c_int),
        ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int),
        ("max_blocks_per_seq", ctypes.c_int),
        ("topk", ctypes.c_int),
        ("kv_format", ctypes.c_int),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int),
        ("num_parts", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("kcache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("cache_seqlens", ctypes.c_void_p),
        ("indices", ctypes.c_void_p),
        ("tile_metadata", ctypes.c_void_p),
        ("num_splits", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("qk_fp8", ctypes.c_int),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmla status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mla_paged_kv_metadata_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i, P, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.mla_metadata_size.argtypes = [i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_metadata_size_for_parts.argtypes = [i, i, i, i, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_get_metadata.argtypes = [P, P, i, i, i, i, i, i, P, P, P]
    lib.mla_workspace_size.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.POINTER(sz)]
    lib.mla_decode_kvcache.argtypes = [ctypes.POINTER(MlaDecodeArgs), P]
    lib.mla_decode_kvcache_noalloc.argtypes = [ctypes.POINTER(MlaDecodeArgs), P]
    lib.mla_decode_partial.argtypes = [ctypes.POINTER(MlaDecodeArgs), P]
    lib.mla_decode_combine.argtypes = [ctypes.POINTER(MlaDecodeArgs), P]
    lib.mla_validate_inputs.argtypes = [ctypes.POINTER(MlaDecodeArgs), P]
    lib.mla_validate_host_inputs.argtypes = [ctypes.POINTER(MlaDecodeArgs), P, P, P, P, P]
    lib.mla_append_kv.argtypes = [P, P, i, i, P, i, P]
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_version.argtypes = []
    for name in ("mla_metadata_size", "mla_metadata_size_for_parts", "mla_get_metadata",
                 "mla_workspace_size", "mla_decode_kvcache", "mla_decode_kvcache_noalloc",
                 "mla_decode_partial",
                 "mla_decode_combine", "mla_validate_inputs", "mla_validate_host_inputs",
                 "mla_append_kv", "mla_version"):
        getattr(lib, name).restype = i
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, load().mla_last_error().decode())
