"""ctypes view of libpagedkv.so (the C ABI declared in include/pagedkv.h).

The library is loaded on first use (`lib()`), so that the package and its
build module import on a tree where it has not been built yet.  Loading
fails loudly: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_OUT_OF_BLOCKS = -2
ERR_UNSUPPORTED = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
ERR_SCRATCH = -6

F32 = 0
BF16 = 1
F16 = 2

# flags of the decode calls
DECODE_CHUNKS = 1

_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)



class ManagerStats(ctypes.Structure):
    """kv_manager_stats_t"""
    _fields_ = [("sequences", ctypes.c_int64), ("blocks_total", ctypes.c_int64),
                ("blocks_free", ctypes.c_int64), ("blocks_used", ctypes.c_int64),
                ("tokens", ctypes.c_int64), ("slots", ctypes.c_int64),
                ("waste_slots", ctypes.c_int64), ("waste_ratio", ctypes.c_double)]


# name -> (restype, argtypes)
SIGNATURES = {
    "kv_pool_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "kv_pool_create": (_c_int, [ctypes.POINTER(_vp), _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _vp, _c_size]),
    "kv_pool_destroy": (_c_int, [_vp]),
    "kv_pool_geometry": (_c_int, [_vp, ctypes.POINTER(_c_int), ctypes.POINTER(_c_int),
                                  ctypes.POINTER(_c_int), ctypes.POINTER(_c_int),
                                  ctypes.POINTER(_c_int), ctypes.POINTER(_c_int),
                                  ctypes.POINTER(_vp)]),
    "kv_pool_alloc_block": (_c_int, [_vp, _i32p]),
    "kv_pool_free_block": (_c_int, [_vp, ctypes.c_int32]),
    "kv_pool_num_free": (_c_int, [_vp]),
    "kv_manager_create": (_c_int, [ctypes.POINTER(_vp), _vp, _c_int]),
    "kv_manager_destroy": (_c_int, [_vp]),
    "kv_manager_add_sequence": (_c_int, [_vp, ctypes.c_int64]),
    "kv_manager_blocks_needed": (ctypes.c_int64, [_vp, _c_int, _vp, _vp]),
    "kv_manager_reserve": (_c_int, [_vp, _c_int, _vp, _vp, _vp]),
    "kv_manager_release": (_c_int, [_vp, ctypes.c_int64]),
    "kv_manager_block_tables": (_c_int, [_vp, _c_int, _vp, _vp, _vp]),
    "kv_manager_stats": (_c_int, [_vp, ctypes.POINTER(ManagerStats)]),
    "kv_append": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp]),
    "kv_append_layers": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp]),
    "kv_append_tokens": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int, _c_int,
                                  _vp]),
    "paged_kv_gather": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int,
                                 _vp]),
    "paged_attention_workspace_bytes": (_c_size, [_vp, _c_int, _c_int]),
    "paged_attention_decode": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int,
                                        ctypes.c_float, _vp, _c_size, ctypes.c_uint, _vp]),
    "paged_attention_decode_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int,
                                               _vp, _c_int, _c_int, ctypes.c_float, _vp, _c_size,
                                               ctypes.c_uint, _vp]),
    "paged_attention_decode_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int,
                                                _c_int, ctypes.c_float, ctypes.c_uint, _vp]),
    "dense_attention_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "dense_attention_decode": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, ctypes.c_float, _vp, _c_size, _vp]),
    "paged_kv_resolve": (_c_int, [_vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _vp]),
    "pagedkv_status_string": (ctypes.c_char_p, [_c_int]),
}


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python -m paged_kv_cache_resolve_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on the first call; raises ImportError if it
    has not been built)."""
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


class LazyLib:
    """Attribute access loads the library on first use, then forwards."""

    def __getattr__(self, name):
        return getattr(lib(), name)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str, library=None):
        self.status = status
        msg = (library or lib()).pagedkv_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")


class OutOfBlocksError(PagedKVError, MemoryError):
    pass
