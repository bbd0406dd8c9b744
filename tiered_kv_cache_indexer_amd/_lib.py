"""ctypes binding of libtkv.so (argument marshalling only).

Every step of the path runs in the HIP kernels behind the C ABI declared in
``include/tkv.h``; this module only converts Python/PyTorch arguments into
pointers and sizes.  There is no fallback: a missing library or a missing GPU
raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtkv.so")

KV_BF16, KV_FP8, KV_NVFP4 = 0, 1, 2
ERR_PAGE_RANGE, ERR_CAPACITY, ERR_NOT_RESIDENT, ERR_BAD_MISS, ERR_RUN_LEN = 1, 2, 4, 8, 16

E = {0: "TKV_OK", -1: "TKV_E_INVALID_ARG", -2: "TKV_E_UNSUPPORTED_FORMAT", -3: "TKV_E_CAPACITY",
     -4: "TKV_E_OOM", -5: "TKV_E_HIP", -6: "TKV_E_STATE"}


class TkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{E.get(code, code)}: {msg}")
        self.code = code


class Config(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("kv_format", C.c_int32),
                ("num_logical_pages", C.c_int64), ("num_slots", C.c_int32),
                ("max_batch", C.c_int32), ("max_rows", C.c_int32), ("max_topk", C.c_int32),
                ("max_pages_per_req", C.c_int32), ("max_width", C.c_int32)]


class Sizes(C.Structure):
    _fields_ = [("pool_bytes", C.c_size_t), ("slab_bytes", C.c_size_t), ("state_bytes", C.c_size_t),
                ("workspace_bytes", C.c_size_t), ("mirror_bytes", C.c_size_t),
                ("row_bytes", C.c_size_t), ("layer_bytes", C.c_size_t)]


class DeviceBuffers(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("slab", C.c_void_p), ("state", C.c_void_p),
                ("workspace", C.c_void_p)]


class Counters(C.Structure):
    _fields_ = [("ensure_calls", C.c_int64), ("hits", C.c_int64), ("misses", C.c_int64),
                ("fresh_allocs", C.c_int64), ("evictions", C.c_int64), ("drops", C.c_int64),
                ("bytes_fetched", C.c_int64), ("bytes_mirrored", C.c_int64), ("clock", C.c_int64),
                ("error_word", C.c_int32), ("reserved", C.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


P = C.c_void_p
I32, I64 = C.c_int32, C.c_int64

SIGNATURES = {
    "tkv_required_bytes": (C.c_int, [C.POINTER(Config), C.POINTER(Sizes)]),
    "tkv_create": (C.c_int, [C.POINTER(Config), C.POINTER(C.c_void_p)]),
    "tkv_attach_device": (C.c_int, [P, C.POINTER(DeviceBuffers), P]),
    "tkv_set_select_width": (C.c_int, [P, I32, I32, I32]),
    "tkv_select_width": (I32, [P]),
    "tkv_reset_residency": (C.c_int, [P, P]),
    "tkv_select_pages": (C.c_int, [P, I32, P, I32, P, P, P, I32, P, I32, P, I32, P, P, P]),
    "tkv_lru_ensure": (C.c_int, [P, P, I32, P, P, P, P, P]),
    "tkv_fetch_pages": (C.c_int, [P, P, P, I32, P]),
    "tkv_sparse_paged_attn": (C.c_int, [P, I32, P, I32, P, P, P, I32, P, P, I32, I32, P, P]),
    "tkv_sparse_paged_attn_host_tail": (C.c_int, [P, I32, P, I32, P, P, P, I32, P, P, I32, I32, P, P]),
    "tkv_decode_layer": (C.c_int, [P, I32, P, I32, P, I32, P, P, P, I32, P, P, P, P, P, P, P]),
    "tkv_decode_layer_prefetch": (C.c_int, [P, I32, P, I32, P, I32, P, P, P, I32, P, P, P, P, P, P, P, I32, P, P]),
    "tkv_fetch_pages_layer": (C.c_int, [P, P, P, I32, I32, P]),
    "tkv_fetch_pages_rest": (C.c_int, [P, I32, I32, P]),
    "tkv_decode_layer_split": (C.c_int, [P, I32, P, I32, P, I32, P, P, P, I32, P, P, P, P, P, P, P, P]),
    "tkv_ensure_write_pages": (C.c_int, [P, I32, P, P, P, I32, P, I32, P, P]),
    "tkv_store_kv_mirror": (C.c_int, [P, I32, P, P, I32, P, P, P, P, I32, P, I32, P]),
    "tkv_store_kv_mirror_split": (C.c_int, [P, I32, P, P, I32, P, P, P, P, I32, P, I32, P, P]),
    "tkv_mirror_flush": (C.c_int, [P, P]),
    "tkv_read_counters": (C.c_int, [P, C.POINTER(Counters), P]),
    "tkv_debug_read_state": (C.c_int, [P, P, P, P, C.POINTER(C.c_int64), P]),
    "tkv_debug_e4m3_encode": (C.c_int, [P, P, I64, P]),
    "tkv_debug_e4m3_decode": (C.c_int, [P, P, I64, P]),
    "tkv_debug_set_attn_kernel": (C.c_int, [P, I32]),
    "tkv_debug_set_attn_range": (C.c_int, [P, I32]),
    "tkv_prefix_record_bytes": (I64, [P]),
    "tkv_prefix_save": (C.c_int, [P, P, I32, P, P]),
    "tkv_prefix_restore": (C.c_int, [P, P, I32, P, P]),
    "tkv_prefix_restore_noalloc": (C.c_int, [P, P, I32, P, P]),
    "tkv_mirror_host_ptr": (C.c_void_p, [P]),
    "tkv_destroy": (None, [P]),
    "tkv_last_error": (C.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libtkv.so and declare every entry point.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tiered_kv_cache_indexer_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc: int):
    if rc != 0:
        raise TkvError(rc, load().tkv_last_error().decode())
