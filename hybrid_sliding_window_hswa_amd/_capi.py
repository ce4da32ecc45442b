"""ctypes declarations of libhswa.so (the C ABI in include/hswa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhswa.so")

HSWA_OK = 0
HSWA_E_INVAL = -1
HSWA_E_NOSPC = -2
HSWA_E_HIP = -3
HSWA_E_UNSUPPORTED = -4

HSWA_OUT_F32 = 0
HSWA_OUT_F16 = 1
HSWA_KV_BF16 = 0
HSWA_KV_FP8 = 1
HSWA_LAYER_FULL = 0
HSWA_LAYER_SWA = 1
HSWA_DECODE_SCRATCH_BYTES = 128 << 20

I32P = C.POINTER(C.c_int32)

# every symbol include/hswa.h declares
EXPORTED = (
    "hswa_last_error", "hswa_status_string", "hswa_version",
    "hswa_pool_create", "hswa_pool_destroy", "hswa_pool_get_view",
    "hswa_pool_alloc", "hswa_pool_evict", "hswa_pool_evict_alloc", "hswa_pool_import",
    "hswa_pool_release",
    "hswa_pool_truncate", "hswa_pool_match_len", "hswa_pool_read_tables", "hswa_pool_fork",
    "hswa_prefill_chunk", "hswa_decode", "hswa_decode_workspace_bytes", "hswa_append_kv",
    "hswa_decode_noalloc",
    "hswa_pool_window_counts", "hswa_kv_offload", "hswa_kv_restore", "hswa_kv_copy",
)


class PoolDesc(C.Structure):
    _fields_ = [
        ("page_size", C.c_int32),
        ("window", C.c_int32),
        ("ring_slots", C.c_int32),
        ("max_seqs", C.c_int32),
        ("max_pages_per_seq", C.c_int32),
        ("num_full_pages", C.c_int32),
        ("full_free_order", I32P),
        ("ring_pages", I32P),
        ("dev_seq_len", C.c_void_p),
        ("dev_fpt", C.c_void_p),
        ("dev_rpt", C.c_void_p),
        ("dev_map", C.c_void_p),
    ]


class PoolView(C.Structure):
    _fields_ = [
        ("seq_len", C.c_void_p),
        ("fpt", C.c_void_p),
        ("rpt", C.c_void_p),
        ("map", C.c_void_p),
        ("max_seqs", C.c_int32),
        ("max_pages_per_seq", C.c_int32),
        ("ring_slots", C.c_int32),
        ("window", C.c_int32),
    ]


class AttnArgs(C.Structure):
    _fields_ = [
        ("kind", C.c_int32),
        ("window", C.c_int32),
        ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("scale", C.c_float),
        ("num_seqs", C.c_int32),
        ("seq_ids", C.c_void_p),
        ("cu_q", C.c_void_p),
        ("total_q", C.c_int32),
        ("max_q_len", C.c_int32),
        ("max_seq_len", C.c_int32),
        ("q", C.c_void_p),
        ("k_new", C.c_void_p),
        ("v_new", C.c_void_p),
        ("pool", PoolView),
        ("k_cache", C.c_void_p),
        ("v_cache", C.c_void_p),
        ("out", C.c_void_p),
        ("vlen_out", C.c_void_p),
        ("kv_dtype", C.c_int32),
        ("k_scale", C.c_void_p),
        ("v_scale", C.c_void_p),
        ("out_dtype", C.c_int32),
        ("q_pos", C.c_void_p),
    ]


class XferArgs(C.Structure):
    _fields_ = [
        ("kind", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("num_seqs", C.c_int32),
        ("seq_ids", C.c_void_p),
        ("cu_tok", C.c_void_p),
        ("first_pos", C.c_void_p),
        ("total_tok", C.c_int32),
        ("max_tok", C.c_int32),
        ("pool", PoolView),
        ("k_cache", C.c_void_p),
        ("v_cache", C.c_void_p),
        ("buf_k", C.c_void_p),
        ("buf_v", C.c_void_p),
        ("kv_dtype", C.c_int32),
        ("k_scale", C.c_void_p),
        ("v_scale", C.c_void_p),
        ("buf_k_scale", C.c_void_p),
        ("buf_v_scale", C.c_void_p),
    ]


class KvCopyArgs(C.Structure):
    _fields_ = [
        ("kind", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("num_seqs", C.c_int32),
        ("src_ids", C.c_void_p),
        ("dst_ids", C.c_void_p),
        ("first_pos", C.c_void_p),
        ("end_pos", C.c_void_p),
        ("max_tok", C.c_int32),
        ("pool", PoolView),
        ("k_cache", C.c_void_p),
        ("v_cache", C.c_void_p),
        ("kv_dtype", C.c_int32),
        ("k_scale", C.c_void_p),
        ("v_scale", C.c_void_p),
    ]


_lib = None


def load():
    """The loaded library (raises ImportError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m hybrid_sliding_window_hswa_amd.build` (there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    lib.hswa_last_error.restype = C.c_char_p
    lib.hswa_last_error.argtypes = []
    lib.hswa_status_string.restype = C.c_char_p
    lib.hswa_status_string.argtypes = [C.c_int]
    lib.hswa_version.restype = C.c_int
    lib.hswa_version.argtypes = []
    lib.hswa_pool_create.restype = C.c_int
    lib.hswa_pool_create.argtypes = [C.POINTER(PoolDesc), C.POINTER(C.c_void_p)]
    lib.hswa_pool_destroy.restype = None
    lib.hswa_pool_destroy.argtypes = [C.c_void_p]
    lib.hswa_pool_get_view.restype = C.c_int
    lib.hswa_pool_get_view.argtypes = [C.c_void_p, C.POINTER(PoolView)]
    for name in ("hswa_pool_alloc", "hswa_pool_import"):
        f = getattr(lib, name)
        f.restype = C.c_int
        f.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, I32P, I32P, C.c_void_p]
    lib.hswa_pool_evict.restype = C.c_int
    lib.hswa_pool_evict.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, C.c_int64, I32P,
                                    C.c_void_p]
    lib.hswa_pool_evict_alloc.restype = C.c_int
    lib.hswa_pool_evict_alloc.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, C.c_int64, I32P,
                                          C.c_int32, I32P, I32P, I32P, I32P, C.c_void_p]
    lib.hswa_pool_release.restype = C.c_int
    lib.hswa_pool_release.argtypes = [C.c_void_p, C.c_int32, I32P, C.c_void_p]
    lib.hswa_pool_match_len.restype = C.c_int
    lib.hswa_pool_match_len.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, C.c_int32, I32P]
    lib.hswa_pool_truncate.restype = C.c_int
    lib.hswa_pool_truncate.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, C.c_void_p]
    lib.hswa_pool_fork.restype = C.c_int
    lib.hswa_pool_fork.argtypes = [C.c_void_p, C.c_int32, I32P, I32P, I32P, I32P, I32P,
                                   C.c_void_p]
    lib.hswa_pool_read_tables.restype = C.c_int
    lib.hswa_pool_read_tables.argtypes = [C.c_void_p, I32P, I32P, I32P, I32P, I32P]
    for name in ("hswa_prefill_chunk", "hswa_append_kv"):
        f = getattr(lib, name)
        f.restype = C.c_int
        f.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
    lib.hswa_decode.restype = C.c_int
    lib.hswa_decode.argtypes = [C.POINTER(AttnArgs), C.c_void_p, C.c_size_t, C.c_void_p]
    lib.hswa_decode_noalloc.restype = C.c_int
    lib.hswa_decode_noalloc.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
    lib.hswa_pool_window_counts.restype = C.c_int
    lib.hswa_pool_window_counts.argtypes = [C.c_void_p, C.c_int32, C.c_int32, I32P, I32P]
    for name in ("hswa_kv_offload", "hswa_kv_restore"):
        f = getattr(lib, name)
        f.restype = C.c_int
        f.argtypes = [C.POINTER(XferArgs), C.c_void_p]
    lib.hswa_kv_copy.restype = C.c_int
    lib.hswa_kv_copy.argtypes = [C.POINTER(KvCopyArgs), C.c_void_p]
    lib.hswa_decode_workspace_bytes.restype = C.c_size_t
    lib.hswa_decode_workspace_bytes.argtypes = [C.POINTER(AttnArgs)]
    _lib = lib
    return lib
