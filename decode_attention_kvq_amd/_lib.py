"""ctypes view of libkvq.so (the C ABI declared in include/kvq.h and include/kvq_calib.h)."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

(KVQ_OK, KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH,
 KVQ_ERR_SCRATCH) = range(7)
KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20      # include/kvq.h
KVQ_F32, KVQ_BF16 = 0, 1
KVQ_KEYS_GROUP_MINMAX, KVQ_KEYS_PER_TOKEN = 0, 1

EXPORTED = ("kvq_cache_buffer_bytes", "kvq_quantize_append", "kvq_rotate_query", "kvq_append_and_rotate",
            "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_attention_noalloc",
            "kvq_decode_step_workspace_bytes", "kvq_decode_step",
            "kvq_status_string", "kvq_probe_stream_read",
            "kvq_calib_workspace_bytes", "kvq_calib_eigenbasis_workspace_bytes", "kvq_calib_contribution",
            "kvq_calib_covariance", "kvq_calib_eigenbasis")


class KvqConfig(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("key_mode", ctypes.c_int32), ("bits", ctypes.c_int32)]


class KvqCache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_stats", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_norms", ctypes.c_void_p),
                ("modality", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("k_tail", ctypes.c_void_p),
                ("append_tickets", ctypes.c_void_p), ("seq_len_host", ctypes.POINTER(ctypes.c_int32))]


class KvqParams(ctypes.Structure):
    _fields_ = [("signs", ctypes.c_void_p), ("rot", ctypes.c_void_p),
                ("codebook", ctypes.c_float * 16)]


class KvqCalibShape(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("n_queries", ctypes.c_int32)]


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libkvq.so; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_kvq_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.kvq_cache_buffer_bytes.argtypes = [P(KvqConfig), P(ctypes.c_size_t * 6)]
    lib.kvq_cache_buffer_bytes.restype = ctypes.c_int
    lib.kvq_quantize_append.argtypes = [P(KvqConfig), P(KvqCache), P(KvqParams), ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_quantize_append.restype = ctypes.c_int
    lib.kvq_rotate_query.argtypes = [P(KvqConfig), P(KvqParams), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_rotate_query.restype = ctypes.c_int
    lib.kvq_append_and_rotate.argtypes = [P(KvqConfig), P(KvqCache), P(KvqParams), ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_append_and_rotate.restype = ctypes.c_int
    lib.kvq_decode_workspace_bytes.argtypes = [P(KvqConfig), ctypes.c_int32]
    lib.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_decode_attention.argtypes = [P(KvqConfig), P(KvqCache), P(KvqParams), ctypes.c_void_p,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_decode_attention.restype = ctypes.c_int
    lib.kvq_decode_attention_noalloc.argtypes = [P(KvqConfig), P(KvqCache), P(KvqParams), ctypes.c_void_p,
                                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.kvq_decode_attention_noalloc.restype = ctypes.c_int
    lib.kvq_decode_step_workspace_bytes.argtypes = [P(KvqConfig), ctypes.c_int32]
    lib.kvq_decode_step_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_decode_step.argtypes = [P(KvqConfig), P(KvqCache), P(KvqParams), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_decode_step.restype = ctypes.c_int
    V = ctypes.c_void_p
    lib.kvq_calib_workspace_bytes.argtypes = [P(KvqCalibShape)]
    lib.kvq_calib_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_calib_eigenbasis_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.kvq_calib_eigenbasis_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_calib_contribution.argtypes = [P(KvqCalibShape), V, ctypes.c_int32, V, ctypes.c_int32, ctypes.c_double,
                                           V, V, ctypes.c_size_t, V]
    lib.kvq_calib_contribution.restype = ctypes.c_int
    lib.kvq_calib_covariance.argtypes = [P(KvqCalibShape), V, ctypes.c_int32, V, V, V, V, V, ctypes.c_size_t, V]
    lib.kvq_calib_covariance.restype = ctypes.c_int
    lib.kvq_calib_eigenbasis.argtypes = [ctypes.c_int32, ctypes.c_int32, V, V, V, V, ctypes.c_size_t, V]
    lib.kvq_calib_eigenbasis.restype = ctypes.c_int
    lib.kvq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p]
    lib.kvq_probe_stream_read.restype = ctypes.c_int
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().kvq_status_string(status).decode()
    except RuntimeError:
        return "library not loaded"


def check(fn: str, status: int) -> None:
    if status != KVQ_OK:
        raise KvqError(fn, status)
