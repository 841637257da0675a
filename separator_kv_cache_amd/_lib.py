"""ctypes view of libsepattn.so (the C ABI declared in include/sepattn.h)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_uint32, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsepattn.so")

OK, EINVAL, ENOTSUP, EHIP, ESPACE = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
MAX_SEP_IDS = 64
BWD_NOALLOC_MAX_ROWS = 1 << 22


class SepattnMask(ctypes.Structure):
    _fields_ = [("B", c_int), ("L", c_int), ("a", c_int), ("n", c_int),
                ("is_sep", c_void_p), ("sep_idx", c_void_p), ("sep_before", c_void_p),
                ("sep_cnt", c_void_p), ("plain_idx", c_void_p), ("plain_cnt", c_void_p),
                ("kept", c_void_p)]


class SepattnShape(ctypes.Structure):
    _fields_ = [("B", c_int), ("Hq", c_int), ("Hkv", c_int), ("L", c_int), ("d", c_int),
                ("q_stride", c_int64 * 3), ("k_stride", c_int64 * 3),
                ("v_stride", c_int64 * 3), ("o_stride", c_int64 * 3)]


class SepCacheStruct(ctypes.Structure):
    _fields_ = [("B", c_int), ("Hkv", c_int), ("d", c_int), ("a", c_int), ("s", c_int), ("n", c_int),
                ("k", c_void_p), ("v", c_void_p), ("slot_pos", c_void_p), ("slot_sep", c_void_p),
                ("state", c_void_p), ("theta", c_float), ("c", c_int)]


_SIGS = {
    "sepattn_last_error": (ctypes.c_char_p, []),
    "sepattn_version": (c_int, []),
    "sepattn_mask_bytes": (c_size_t, [c_int, c_int]),
    "sepattn_mask_carve": (c_int, [POINTER(SepattnMask), c_int, c_int, c_int, c_int, c_void_p, c_size_t]),
    "sepattn_build_mask": (c_int, [c_void_p, POINTER(c_int32), c_int, POINTER(SepattnMask), c_void_p]),
    "sepattn_mask_bits": (c_int, [POINTER(SepattnMask), c_void_p, c_void_p]),
    "sepattn_fwd_tile_rows": (c_int, [c_int]),
    "sepattn_tile_desc": (c_int, [POINTER(SepattnMask), c_int, c_void_p, c_void_p]),
    "sepattn_fwd": (c_int, [POINTER(SepattnShape), c_int, POINTER(SepattnMask), c_void_p, c_void_p,
                            c_void_p, c_float, c_void_p, c_void_p, c_void_p]),
    "sepattn_bwd_workspace_size": (c_size_t, [POINTER(SepattnShape)]),
    "sepattn_bwd": (c_int, [POINTER(SepattnShape), c_int, POINTER(SepattnMask), c_void_p, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_size_t, c_void_p]),
    "sepattn_bwd_noalloc": (c_int, [POINTER(SepattnShape), c_int, POINTER(SepattnMask), c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
    "sepcache_slots": (c_int, [c_int, c_int, c_int, c_int]),
    "sepcache_k_rows": (c_int, [c_int]),
    "sepcache_reset": (c_int, [POINTER(SepCacheStruct), c_void_p]),
    "sepcache_append": (c_int, [POINTER(SepCacheStruct), c_void_p, c_void_p, c_void_p, c_void_p]),
    "sepcache_evict": (c_int, [POINTER(SepCacheStruct), c_void_p]),
    "sepcache_push": (c_int, [POINTER(SepCacheStruct), c_void_p, c_void_p, c_void_p, c_void_p]),
    "sepcache_decode_workspace_size": (c_size_t, [POINTER(SepCacheStruct), c_int]),
    "sepcache_decode": (c_int, [POINTER(SepCacheStruct), c_int, c_void_p, c_float, c_int, c_void_p,
                                c_void_p, c_size_t, c_void_p]),
    "sepcache_export_order": (c_int, [POINTER(SepCacheStruct), c_void_p, c_void_p, c_void_p]),
    "sepattn_build_mask_fixed": (c_int, [c_int, POINTER(SepattnMask), c_void_p]),
    "sepcache_prefill": (c_int, [POINTER(SepCacheStruct), c_void_p, c_void_p, POINTER(c_int64), POINTER(c_int64),
                                 POINTER(SepattnMask), c_void_p]),
    "sepcache_step": (c_int, [POINTER(SepCacheStruct), c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_float,
                              c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
}

EXPORTED = tuple(_SIGS)

_lib = None


class SepattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sepattn error {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Loads the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m separator_kv_cache_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(rc: int) -> None:
    if rc != OK:
        raise SepattnError(rc, load().sepattn_last_error().decode())
