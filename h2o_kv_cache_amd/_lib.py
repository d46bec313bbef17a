"""ctypes loader of libh2o.so (built in-tree by h2o_kv_cache_amd.build)."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libh2o.so")

H2O_OK = 0
H2O_ERR_INVALID_ARG = 1
H2O_ERR_UNSUPPORTED = 2
H2O_ERR_WORKSPACE = 3
H2O_ERR_HIP = 4

EXPORTED = ("h2o_workspace_size", "h2o_attn_chunk", "h2o_score_accumulate",
            "h2o_evict_select", "kv_scatter", "h2o_attn_chunk_q8", "kv_scatter_q8",
            "h2o_quantize_rows_q8", "h2o_snapkv_select", "h2o_snapkv_compact",
            "h2o_attn_bwd_workspace_size",
            "h2o_attn_chunk_bwd", "h2o_timing_start", "h2o_timing_stop",
            "h2o_attn_chunk_static", "h2o_step", "h2o_status_string")

# bytes of the library's static scratch (H2O_STATIC_SCRATCH_BYTES in h2o.h)
STATIC_SCRATCH_BYTES = 64 << 20


class H2OShape(ctypes.Structure):
    """Mirror of h2o_shape_t (include/h2o.h)."""
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cache_len", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("n_valid", ctypes.c_int32), ("scale", ctypes.c_float)]


_lib = None
_lock = threading.Lock()


def _declare(lib):
    P = ctypes.c_void_p
    S = ctypes.POINTER(H2OShape)
    lib.h2o_workspace_size.argtypes = [S]
    lib.h2o_workspace_size.restype = ctypes.c_size_t
    lib.h2o_attn_chunk.argtypes = [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.h2o_attn_chunk.restype = ctypes.c_int
    lib.h2o_score_accumulate.argtypes = [S, P, P, P, P]
    lib.h2o_score_accumulate.restype = ctypes.c_int
    lib.h2o_evict_select.argtypes = [S, P, P, P]
    lib.h2o_evict_select.restype = ctypes.c_int
    lib.kv_scatter.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_int64, P]
    lib.kv_scatter.restype = ctypes.c_int
    lib.h2o_attn_chunk_q8.argtypes = [S] + [P] * 11 + [ctypes.c_size_t, P]
    lib.h2o_attn_chunk_q8.restype = ctypes.c_int
    lib.kv_scatter_q8.argtypes = [S] + [P] * 10 + [ctypes.c_int64, P]
    lib.kv_scatter_q8.restype = ctypes.c_int
    lib.h2o_quantize_rows_q8.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P]
    lib.h2o_quantize_rows_q8.restype = ctypes.c_int
    lib.h2o_snapkv_select.argtypes = [S, P, ctypes.c_int32, P, P]
    lib.h2o_snapkv_select.restype = ctypes.c_int
    lib.h2o_snapkv_compact.argtypes = ([S] + [P] * 7 + [ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int64] + [P] * 5)
    lib.h2o_snapkv_compact.restype = ctypes.c_int
    lib.h2o_attn_bwd_workspace_size.argtypes = [S]
    lib.h2o_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.h2o_attn_chunk_bwd.argtypes = [S] + [P] * 14 + [ctypes.c_size_t, P]
    lib.h2o_attn_chunk_bwd.restype = ctypes.c_int
    lib.h2o_timing_start.argtypes = [ctypes.c_int32]
    lib.h2o_timing_start.restype = ctypes.c_int
    lib.h2o_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    lib.h2o_timing_stop.restype = ctypes.c_int
    lib.h2o_step.argtypes = [S] + [P] * 12 + [ctypes.c_int64, P, ctypes.c_size_t, P]
    lib.h2o_step.restype = ctypes.c_int
    lib.h2o_attn_chunk_static.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.h2o_attn_chunk_static.restype = ctypes.c_int
    lib.h2o_status_string.argtypes = [ctypes.c_int]
    lib.h2o_status_string.restype = ctypes.c_char_p
    return lib


def load(build_if_missing: bool = True):
    """Load libh2o.so; compile it first (hipcc, gfx950) if it is not built.

    There is no other implementation behind this binding: if the library
    cannot be built or loaded this raises.
    """
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise RuntimeError(f"{LIB_PATH} is not built "
                                   "(python -m h2o_kv_cache_amd.build)")
            from . import build as _build
            _build.build()
        _lib = _declare(ctypes.CDLL(LIB_PATH))
        return _lib
