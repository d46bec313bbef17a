"""Python binding of libh2o.so: one chunked H2O sparse-attention step on
MI355X (gfx950).

The functions below carry the C ABI's names (include/h2o.h) and only marshal
arguments: they check dtypes, shapes, devices and contiguity of the torch
tensors, then pass raw device pointers and the current HIP stream to the
library.  Every step of the computation runs in the library's kernels.

Layouts (B batch, Hq / Hkv query / KV heads, D head_dim, C cache slots,
S chunk tokens):
    q            [B, Hq, S, D]   bfloat16
    k/v_cache    [B, Hkv, C, D]  bfloat16
    k/v_new      [B, Hkv, S, D]  bfloat16
    out          [B, Hq, S, D]   float32
    lse          [B, Hq, S]      float32
    wsum         [B, Hkv, C + S] float32
    scores       [B, Hkv, C]     float32
    new_scores   [B, Hkv, S]     float32
    pos          [B, Hkv, C]     int64
    evict_idx    [B, Hkv, S]     int32
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import H2OShape, STATIC_SCRATCH_BYTES

__all__ = ["Shape", "H2OError", "h2o_workspace_size", "h2o_attn_chunk",
           "h2o_score_accumulate", "h2o_evict_select", "kv_scatter",
           "h2o_attn_chunk_q8", "kv_scatter_q8", "h2o_quantize_rows_q8",
           "h2o_snapkv_select", "h2o_snapkv_compact", "h2o_attn_bwd_workspace_size", "h2o_attn_chunk_bwd",
           "h2o_timing_start", "h2o_timing_stop", "h2o_status_string", "H2OCache",
           "h2o_attn_chunk_static", "STATIC_SCRATCH_BYTES", "h2o_step",
           "load_library", "ATTN_KERNELS"]

# the four kernels of h2o_attn_chunk, in launch order (h2o_timing_stop order)
ATTN_KERNELS = ("attn_fwd", "attn_combine", "attn_colsum", "wsum_reduce")


class H2OError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {h2o_status_string(status)} (status {status})")


@dataclass(frozen=True)
class Shape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_len: int
    chunk_len: int
    n_valid: int = 0
    scale: float = 0.0

    def c(self) -> H2OShape:
        return H2OShape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                        self.cache_len, self.chunk_len, self.n_valid, self.scale)

    def with_n(self, n_valid: int) -> "Shape":
        return Shape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                     self.cache_len, self.chunk_len, n_valid, self.scale)


def load_library():
    return _lib.load()


def h2o_status_string(status: int) -> str:
    return _lib.load().h2o_status_string(int(status)).decode()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: torch.Tensor, name: str, shape, dtypes) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)


def _check(status: int, where: str):
    if status != 0:
        raise H2OError(status, where)


def h2o_workspace_size(shape: Shape) -> int:
    sh = shape.c()
    return int(_lib.load().h2o_workspace_size(ctypes.byref(sh)))


def h2o_attn_chunk(shape: Shape, q, k_cache, v_cache, k_new, v_new, out, lse, wsum,
                   ws, stream=None):
    s = shape
    B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim,
                           s.cache_len, s.chunk_len)
    args = [
        _ptr(q, "q", (B, Hq, S, D), _BF16),
        _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(out, "out", (B, Hq, S, D), _F32),
        ctypes.c_void_p(None) if lse is None else _ptr(lse, "lse", (B, Hq, S), _F32),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
    ]
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    sh = s.c()
    _check(_lib.load().h2o_attn_chunk(ctypes.byref(sh), *args, ctypes.c_void_p(ws.data_ptr()),
                                      ctypes.c_size_t(nbytes), _stream(stream)),
           "h2o_attn_chunk")


def h2o_step(shape: Shape, q, k_cache, v_cache, k_new, v_new, out, lse, wsum, scores,
             new_scores, evict_idx, pos, p0: int, ws, stream=None):
    """The four calls of a step in one (attention, accumulation, choice,
    scatter); one-token chunks on the few-row path run the work after the
    streaming pass as one kernel."""
    s = shape
    B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim,
                           s.cache_len, s.chunk_len)
    args = [
        _ptr(q, "q", (B, Hq, S, D), _BF16),
        _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(out, "out", (B, Hq, S, D), _F32),
        ctypes.c_void_p(None) if lse is None else _ptr(lse, "lse", (B, Hq, S), _F32),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
        _ptr(scores, "scores", (B, Hkv, C), _F32),
        _ptr(new_scores, "new_scores", (B, Hkv, S), _F32),
        _ptr(evict_idx, "evict_idx", (B, Hkv, S), (torch.int32,)),
        ctypes.c_void_p(None) if pos is None else _ptr(pos, "pos", (B, Hkv, C), (torch.int64,)),
    ]
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    sh = s.c()
    _check(_lib.load().h2o_step(ctypes.byref(sh), *args, ctypes.c_int64(int(p0)),
                                ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes),
                                _stream(stream)), "h2o_step")


def h2o_attn_chunk_static(shape: Shape, q, k_cache, v_cache, k_new, v_new, out, lse, wsum,
                          stream=None):
    """h2o_attn_chunk with the library's static device scratch instead of a
    caller workspace (for callers that cannot allocate); shapes whose
    workspace exceeds STATIC_SCRATCH_BYTES are rejected."""
    s = shape
    B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim,
                           s.cache_len, s.chunk_len)
    args = [
        _ptr(q, "q", (B, Hq, S, D), _BF16),
        _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(out, "out", (B, Hq, S, D), _F32),
        ctypes.c_void_p(None) if lse is None else _ptr(lse, "lse", (B, Hq, S), _F32),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
    ]
    sh = s.c()
    _check(_lib.load().h2o_attn_chunk_static(ctypes.byref(sh), *args, _stream(stream)),
           "h2o_attn_chunk_static")


def h2o_score_accumulate(shape: Shape, scores, new_scores, wsum, stream=None):
    s = shape
    B, Hkv, C, S = s.batch, s.n_kv_heads, s.cache_len, s.chunk_len
    sh = s.c()
    _check(_lib.load().h2o_score_accumulate(
        ctypes.byref(sh), _ptr(scores, "scores", (B, Hkv, C), _F32),
        _ptr(new_scores, "new_scores", (B, Hkv, S), _F32),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32), _stream(stream)),
        "h2o_score_accumulate")


def h2o_evict_select(shape: Shape, scores, evict_idx, stream=None):
    s = shape
    B, Hkv, C, S = s.batch, s.n_kv_heads, s.cache_len, s.chunk_len
    sh = s.c()
    _check(_lib.load().h2o_evict_select(
        ctypes.byref(sh), _ptr(scores, "scores", (B, Hkv, C), _F32),
        _ptr(evict_idx, "evict_idx", (B, Hkv, S), (torch.int32,)), _stream(stream)),
        "h2o_evict_select")


def kv_scatter(shape: Shape, k_cache, v_cache, scores, pos, k_new, v_new, new_scores,
               evict_idx, p0: int, stream=None):
    s = shape
    B, Hkv, D, C, S = s.batch, s.n_kv_heads, s.head_dim, s.cache_len, s.chunk_len
    sh = s.c()
    _check(_lib.load().kv_scatter(
        ctypes.byref(sh), _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        _ptr(scores, "scores", (B, Hkv, C), _F32),
        ctypes.c_void_p(None) if pos is None else _ptr(pos, "pos", (B, Hkv, C), (torch.int64,)),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(new_scores, "new_scores", (B, Hkv, S), _F32),
        _ptr(evict_idx, "evict_idx", (B, Hkv, S), (torch.int32,)),
        ctypes.c_int64(int(p0)), _stream(stream)),
        "kv_scatter")


_I8 = (torch.int8,)


def h2o_attn_chunk_q8(shape: Shape, q, k_cache, k_scale, v_cache, v_scale, k_new, v_new, out,
                      lse, wsum, ws, stream=None):
    s = shape
    B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.cache_len,
                           s.chunk_len)
    sh = s.c()
    nbytes = ws.numel() * ws.element_size()
    _check(_lib.load().h2o_attn_chunk_q8(
        ctypes.byref(sh), _ptr(q, "q", (B, Hq, S, D), _BF16),
        _ptr(k_cache, "k_cache", (B, Hkv, C, D), _I8),
        _ptr(k_scale, "k_scale", (B, Hkv, C), _F32),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _I8),
        _ptr(v_scale, "v_scale", (B, Hkv, C), _F32),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(out, "out", (B, Hq, S, D), _F32),
        ctypes.c_void_p(None) if lse is None else _ptr(lse, "lse", (B, Hq, S), _F32),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes), _stream(stream)),
        "h2o_attn_chunk_q8")


def kv_scatter_q8(shape: Shape, k_cache, k_scale, v_cache, v_scale, scores, pos, k_new, v_new,
                  new_scores, evict_idx, p0: int, stream=None):
    s = shape
    B, Hkv, D, C, S = s.batch, s.n_kv_heads, s.head_dim, s.cache_len, s.chunk_len
    sh = s.c()
    _check(_lib.load().kv_scatter_q8(
        ctypes.byref(sh), _ptr(k_cache, "k_cache", (B, Hkv, C, D), _I8),
        _ptr(k_scale, "k_scale", (B, Hkv, C), _F32),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _I8),
        _ptr(v_scale, "v_scale", (B, Hkv, C), _F32),
        _ptr(scores, "scores", (B, Hkv, C), _F32),
        ctypes.c_void_p(None) if pos is None else _ptr(pos, "pos", (B, Hkv, C), (torch.int64,)),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(new_scores, "new_scores", (B, Hkv, S), _F32),
        _ptr(evict_idx, "evict_idx", (B, Hkv, S), (torch.int32,)),
        ctypes.c_int64(int(p0)), _stream(stream)),
        "kv_scatter_q8")


def h2o_quantize_rows_q8(x, codes, scales, stream=None):
    """x [..., D] bf16 -> codes [..., D] int8, scales [...] fp32 (contiguous)."""
    D = x.shape[-1]
    rows = x.numel() // D
    _check(_lib.load().h2o_quantize_rows_q8(
        _ptr(x, "x", tuple(x.shape), _BF16), ctypes.c_int64(rows), ctypes.c_int32(D),
        _ptr(codes, "codes", tuple(x.shape), _I8),
        _ptr(scales, "scales", tuple(x.shape[:-1]), _F32), _stream(stream)),
        "h2o_quantize_rows_q8")


def h2o_snapkv_select(shape: Shape, wsum, budget: int, keep_idx, stream=None):
    s = shape
    B, Hkv, C, S = s.batch, s.n_kv_heads, s.cache_len, s.chunk_len
    sh = s.c()
    keep = (ctypes.c_void_p(None) if keep_idx is None
            else _ptr(keep_idx, "keep_idx", (B, Hkv, int(budget)), (torch.int32,)))
    _check(_lib.load().h2o_snapkv_select(
        ctypes.byref(sh), _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
        ctypes.c_int32(int(budget)), keep, _stream(stream)),
        "h2o_snapkv_select")


def h2o_snapkv_compact(shape: Shape, k_cache, v_cache, pos, k_new, v_new, wsum, keep_idx,
                       budget: int, out_len: int, p0: int, k_out, v_out, pos_out=None,
                       scores_out=None, stream=None):
    s = shape
    B, Hkv, D, C, S = s.batch, s.n_kv_heads, s.head_dim, s.cache_len, s.chunk_len
    L = int(out_len)
    sh = s.c()
    none = ctypes.c_void_p(None)
    _check(_lib.load().h2o_snapkv_compact(
        ctypes.byref(sh), _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        none if pos is None else _ptr(pos, "pos", (B, Hkv, C), (torch.int64,)),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(wsum, "wsum", (B, Hkv, C + S), _F32),
        none if keep_idx is None else _ptr(keep_idx, "keep_idx", (B, Hkv, int(budget)),
                                           (torch.int32,)),
        ctypes.c_int32(int(budget)), ctypes.c_int32(L), ctypes.c_int64(int(p0)),
        _ptr(k_out, "k_out", (B, Hkv, L, D), _BF16),
        _ptr(v_out, "v_out", (B, Hkv, L, D), _BF16),
        none if pos_out is None else _ptr(pos_out, "pos_out", (B, Hkv, L), (torch.int64,)),
        none if scores_out is None else _ptr(scores_out, "scores_out", (B, Hkv, L), _F32),
        _stream(stream)),
        "h2o_snapkv_compact")


def h2o_attn_bwd_workspace_size(shape: Shape) -> int:
    sh = shape.c()
    return int(_lib.load().h2o_attn_bwd_workspace_size(ctypes.byref(sh)))


def h2o_attn_chunk_bwd(shape: Shape, q, k_cache, v_cache, k_new, v_new, out, lse, dout,
                       dq, dk_cache, dv_cache, dk_new, dv_new, ws, stream=None):
    """Gradients of h2o_attn_chunk's output (slot layout fixed).  dout is
    bf16; the gradients are fp32 and every element is written."""
    s = shape
    B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim,
                           s.cache_len, s.chunk_len)
    args = [
        _ptr(q, "q", (B, Hq, S, D), _BF16),
        _ptr(k_cache, "k_cache", (B, Hkv, C, D), _BF16),
        _ptr(v_cache, "v_cache", (B, Hkv, C, D), _BF16),
        _ptr(k_new, "k_new", (B, Hkv, S, D), _BF16),
        _ptr(v_new, "v_new", (B, Hkv, S, D), _BF16),
        _ptr(out, "out", (B, Hq, S, D), _F32),
        _ptr(lse, "lse", (B, Hq, S), _F32),
        _ptr(dout, "dout", (B, Hq, S, D), _BF16),
        _ptr(dq, "dq", (B, Hq, S, D), _F32),
        _ptr(dk_cache, "dk_cache", (B, Hkv, C, D), _F32),
        _ptr(dv_cache, "dv_cache", (B, Hkv, C, D), _F32),
        _ptr(dk_new, "dk_new", (B, Hkv, S, D), _F32),
        _ptr(dv_new, "dv_new", (B, Hkv, S, D), _F32),
    ]
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    sh = s.c()
    _check(_lib.load().h2o_attn_chunk_bwd(ctypes.byref(sh), *args,
                                          ctypes.c_void_p(ws.data_ptr()),
                                          ctypes.c_size_t(nbytes), _stream(stream)),
           "h2o_attn_chunk_bwd")


def h2o_timing_start(max_calls: int):
    _check(_lib.load().h2o_timing_start(int(max_calls)), "h2o_timing_start")


def h2o_timing_stop():
    """Returns ({kernel: summed ms}, timed calls)."""
    ms = (ctypes.c_double * 4)()
    calls = ctypes.c_int32(0)
    _check(_lib.load().h2o_timing_stop(ms, ctypes.byref(calls)), "h2o_timing_stop")
    return {k: ms[i] for i, k in enumerate(ATTN_KERNELS)}, int(calls.value)


class H2OCache:
    """Device buffers of one layer's H2O cache plus the per-step outputs.

    ``step`` enqueues the four library calls in order on the current stream and
    advances ``n_valid`` on the host; it never synchronises.
    """

    def __init__(self, shape: Shape, device="cuda", n_valid: int = 0):
        s = shape
        B, Hq, Hkv, D, C, S = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim,
                               s.cache_len, s.chunk_len)
        self.shape = s.with_n(n_valid)
        dev = torch.device(device)
        self.k_cache = torch.zeros((B, Hkv, C, D), dtype=torch.bfloat16, device=dev)
        self.v_cache = torch.zeros((B, Hkv, C, D), dtype=torch.bfloat16, device=dev)
        self.scores = torch.zeros((B, Hkv, C), dtype=torch.float32, device=dev)
        self.pos = torch.full((B, Hkv, C), -1, dtype=torch.int64, device=dev)
        self.out = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        self.wsum = torch.empty((B, Hkv, C + S), dtype=torch.float32, device=dev)
        self.new_scores = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
        self.evict_idx = torch.empty((B, Hkv, S), dtype=torch.int32, device=dev)
        self.ws = torch.empty(max(h2o_workspace_size(self.shape), 256),
                              dtype=torch.uint8, device=dev)

    @property
    def n_valid(self) -> int:
        return self.shape.n_valid

    def set_n_valid(self, n: int):
        self.shape = self.shape.with_n(n)

    def step(self, q, k_new, v_new, p0: int, stream=None):
        s = self.shape
        h2o_attn_chunk(s, q, self.k_cache, self.v_cache, k_new, v_new, self.out, self.lse,
                       self.wsum, self.ws, stream)
        h2o_score_accumulate(s, self.scores, self.new_scores, self.wsum, stream)
        h2o_evict_select(s, self.scores, self.evict_idx, stream)
        kv_scatter(s, self.k_cache, self.v_cache, self.scores, self.pos, k_new, v_new,
                   self.new_scores, self.evict_idx, p0, stream)
        self.shape = s.with_n(min(s.cache_len, s.n_valid + s.chunk_len))
