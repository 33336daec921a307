"""ctypes loader of libpagedkv.so (the HIP library built by ``build.py``).

There is no fallback: if the library is missing or fails to load, every call
raises ``RuntimeError``.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libpagedkv.so")

PKV_OK = 0
PKV_F32 = 0
PKV_BF16 = 1
PKV_KERNEL_AUTO = 0
PKV_KERNEL_GENERIC = 1
PKV_KERNEL_FAST = 2
KERNEL_NAMES = {PKV_KERNEL_GENERIC: "generic", PKV_KERNEL_FAST: "fast"}

EXPORTS = (
    "paged_kv_write",
    "paged_attn_plan",
    "paged_attn_workspace_bytes",
    "paged_attn_decode",
    "paged_attn_decode_noalloc",
    "paged_attn_prefix_plan",
    "paged_attn_decode_prefix",
    "paged_attn_multi_plan",
    "paged_attn_decode_multi",
    "paged_block_copy",
    "pkv_status_string",
    "pkv_version",
    "pkv_last_launch_info",
    "pkv_bm_create",
    "pkv_bm_destroy",
    "pkv_bm_num_free",
    "pkv_bm_refcount",
    "pkv_bm_seq_len",
    "pkv_bm_add",
    "pkv_bm_fork",
    "pkv_bm_free",
    "pkv_bm_append",
    "pkv_bm_slots",
    "pkv_bm_block_tables",
)


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("grid_waves", ctypes.c_int32), ("xcd_balance", ctypes.c_int32)]


class DecodePlan(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("partition_tokens", ctypes.c_int32),
        ("max_partitions", ctypes.c_int32),
        ("threads_per_block", ctypes.c_int32),
        ("grid_blocks", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
    ]


class LaunchInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("grid", ctypes.c_int32), ("xcd_balance", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("k_stream", ctypes.c_int32)]


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: status {status} ({text})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is not built; build it with `python -m paged_kv_cache_276_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIBRARY)
    i32, vp, u64 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64
    P = ctypes.POINTER
    L.paged_kv_write.restype = ctypes.c_int
    L.paged_kv_write.argtypes = [vp, vp, vp, i32, vp, vp, P(CacheDesc), vp]
    L.paged_attn_plan.restype = ctypes.c_int
    L.paged_attn_plan.argtypes = [i32, i32, i32, P(CacheDesc), P(DecodeOpts), P(DecodePlan)]
    L.paged_attn_workspace_bytes.restype = ctypes.c_int
    L.paged_attn_workspace_bytes.argtypes = [i32, i32, i32, P(CacheDesc), P(DecodeOpts), P(u64)]
    L.paged_attn_decode.restype = ctypes.c_int
    L.paged_attn_decode.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, ctypes.c_float, vp, vp, u64,
                                    P(CacheDesc), P(DecodeOpts), vp]
    L.paged_attn_decode_noalloc.restype = ctypes.c_int
    L.paged_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, ctypes.c_float, vp,
                                            P(CacheDesc), P(DecodeOpts), vp]
    L.paged_attn_prefix_plan.restype = ctypes.c_int
    L.paged_attn_prefix_plan.argtypes = [i32, i32, i32, i32, i32, P(CacheDesc), P(DecodeOpts), P(DecodePlan)]
    L.paged_attn_decode_prefix.restype = ctypes.c_int
    L.paged_attn_decode_prefix.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, i32, i32, ctypes.c_float,
                                           vp, vp, u64, P(CacheDesc), P(DecodeOpts), vp]
    L.paged_attn_multi_plan.restype = ctypes.c_int
    L.paged_attn_multi_plan.argtypes = [i32, i32, i32, i32, i32, P(CacheDesc), P(DecodeOpts), P(DecodePlan)]
    L.paged_attn_decode_multi.restype = ctypes.c_int
    L.paged_attn_decode_multi.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                                          vp, vp, u64, P(CacheDesc), P(DecodeOpts), vp]
    L.paged_block_copy.restype = ctypes.c_int
    L.paged_block_copy.argtypes = [vp, vp, vp, i32, P(CacheDesc), vp]
    i64 = ctypes.c_int64
    L.pkv_bm_create.restype = ctypes.c_int
    L.pkv_bm_create.argtypes = [i32, i32, P(vp)]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [vp]
    L.pkv_bm_num_free.restype = i32
    L.pkv_bm_num_free.argtypes = [vp]
    L.pkv_bm_refcount.restype = i32
    L.pkv_bm_refcount.argtypes = [vp, i32]
    L.pkv_bm_seq_len.restype = i32
    L.pkv_bm_seq_len.argtypes = [vp, i64]
    L.pkv_bm_add.restype = ctypes.c_int
    L.pkv_bm_add.argtypes = [vp, i64, i32]
    L.pkv_bm_fork.restype = ctypes.c_int
    L.pkv_bm_fork.argtypes = [vp, i64, i64]
    L.pkv_bm_free.restype = ctypes.c_int
    L.pkv_bm_free.argtypes = [vp, i64]
    L.pkv_bm_append.restype = ctypes.c_int
    L.pkv_bm_append.argtypes = [vp, vp, i32, vp, vp, i32, P(i32)]
    L.pkv_bm_slots.restype = ctypes.c_int
    L.pkv_bm_slots.argtypes = [vp, i64, i32, i32, vp]
    L.pkv_bm_block_tables.restype = ctypes.c_int
    L.pkv_bm_block_tables.argtypes = [vp, vp, i32, i32, vp, vp]
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_status_string.argtypes = [ctypes.c_int]
    L.pkv_version.restype = ctypes.c_char_p
    L.pkv_version.argtypes = []
    L.pkv_last_launch_info.restype = ctypes.c_int
    L.pkv_last_launch_info.argtypes = [P(LaunchInfo)]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where, status_string(status))
