"""ctypes view of libpkv.so (declarations mirror include/pkv.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any call.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OUT_OF_PAGES = -2
PKV_ERR_UNSUPPORTED = -3
PKV_ERR_DEVICE = -4
PKV_ERR_BUFFER_TOO_SMALL = -5
PKV_ERR_SHARED_PAGE = -6

PKV_F32 = 0
PKV_BF16 = 1
PKV_I8 = 2

PKV_NOALLOC_SCRATCH_BYTES = 32 << 20

i32p = POINTER(c_int32)
i64p = POINTER(ctypes.c_int64)


class PoolDescC(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("num_pages", c_int32), ("page_size", c_int32),
                ("num_kv_heads", c_int32), ("head_dim", c_int32)]


_SIGNATURES = {
    "pkv_last_error": (c_char_p, []),
    "pkv_alloc_create": (c_int, [c_int32, c_int32, i32p, POINTER(c_void_p)]),
    "pkv_alloc_destroy": (None, [c_void_p]),
    "pkv_seq_new": (c_int, [c_void_p, i32p]),
    "pkv_reserve": (c_int, [c_void_p, c_int32, c_int32]),
    "pkv_truncate": (c_int, [c_void_p, c_int32, c_int32]),
    "pkv_release": (c_int, [c_void_p, c_int32]),
    "pkv_share_prefix": (c_int, [c_void_p, c_int32, c_int32, c_int32]),
    "pkv_fork": (c_int, [c_void_p, c_int32, c_int32]),
    "pkv_reserve_cow": (c_int, [c_void_p, c_int32, c_int32, i32p, i32p]),
    "pkv_copy_pages": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
    "pkv_stream_read": (c_int, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]),
    "pkv_retention_add": (c_int, [c_void_p, c_int32, ctypes.c_double, ctypes.c_double]),
    "pkv_retention_evict": (c_int, [c_void_p, ctypes.c_int64, i32p, c_int32, i32p]),
    "pkv_retention_take": (c_int, [c_void_p, c_int32, i32p]),
    "pkv_retention_pages": (c_int, [c_void_p, i64p]),
    "pkv_seq_len": (c_int, [c_void_p, c_int32, i32p]),
    "pkv_num_free": (c_int, [c_void_p, i32p]),
    "pkv_page_refcount": (c_int, [c_void_p, c_int32, i32p]),
    "pkv_seq_num_blocks": (c_int, [c_void_p, c_int32, i32p]),
    "pkv_block_tables": (c_int, [c_void_p, i32p, c_int32, c_int32, i32p]),
    "pkv_slots": (c_int, [c_void_p, c_int32, c_int32, c_int32, i64p]),
    "pkv_prepare_step": (c_int, [c_void_p, i32p, c_int32, i32p, c_int32, i64p, i32p, i32p]),
    "pkv_plan_prefix": (c_int, [i32p, i64p, c_int32, c_int32, i32p, i32p, i32p]),
    "pkv_store_kv": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_int32, c_void_p]),
    "pkv_i8_block_bytes": (c_size_t, [c_int32, c_int32]),
    "pkv_pool_bytes": (c_size_t, [POINTER(PoolDescC)]),
    "pkv_codec_payload_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "pkv_codec_encode": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                 c_void_p]),
    "pkv_codec_decode": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                 c_void_p]),
    "pkv_workspace_bytes": (c_size_t, [POINTER(PoolDescC), c_int32, c_int32, c_int32, c_int32]),
    "pkv_decode": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                           c_void_p, c_int32, c_void_p, c_int32, c_float, c_void_p, c_void_p,
                           c_size_t, c_void_p]),
    "pkv_decode_noalloc": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                   c_void_p, c_int32, c_void_p, c_int32, c_float, c_void_p, c_void_p]),
    "pkv_prefill_append": (c_int, [POINTER(PoolDescC), c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                   c_int32, c_int32, c_float, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
    "pkv_validate_tables": (c_int, [POINTER(PoolDescC), i32p, c_int32, c_int32, i32p, i32p,
                                    c_int32]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


def lib():
    """The loaded library (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m pagedattention_pkv_store_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    msg = lib().pkv_last_error()
    return msg.decode() if msg else ""
