"""Seeded synthetic workloads for the H2O chunk step.

This module produces inputs only: it holds none of the method's arithmetic.
Both the CPU oracle (through the tests) and the HIP path receive the arrays it
returns, so the two sides always see bit-identical inputs.

Shapes follow the long-context setups of "Learning how to Forget: Fine-tuning
for Long-Context Sparse Attention" (arXiv 2608.19920): chunk sizes 2048 / 1024
(page 2, Table 1 caption), 64k / 128k contexts (Table 1), chunk 128 (Table 5)
and the Qwen3-4B-Instruct-2507 checkpoint (Table 2 / Table 4 captions), whose
attention shape (32 query heads, 8 KV heads, head_dim 128, 36 layers) is used
here.  The Helmet data itself is not reproduced: every tensor is drawn from a
counter-keyed Philox stream.

Random streams are keyed by ``(base_seed, cfg_id, layer, step, tensor_id[, b])``
through ``numpy.random.SeedSequence`` so that any chunk of any layer can be
regenerated on its own, in any order.

All floating-point tensors are rounded to bfloat16 with round-to-nearest-even
on the host.  ``to_bf16`` returns both the raw 16-bit patterns (what is
uploaded to the device) and the float32 values those patterns denote (what the
oracle consumes).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

BASE_SEED = 0

# tensor ids of the counter-keyed streams
T_Q, T_K, T_V, T_HEAVY, T_KC, T_VC, T_HEAVY_C, T_SCORE, T_POS = range(9)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus value distribution."""
    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_len: int
    chunk_len: int
    seq_len: int          # tokens processed in a full run (decode: steps)
    layers: int
    value_std: float      # std of Q, K, V entries before rounding
    heavy_frac: float     # fraction of K rows scaled by heavy_scale
    heavy_scale: float
    prefilled: bool       # cache starts full (decode-shaped runs)
    keep_budget: int = 0  # SnapKV-style one-shot runs: cache slots kept

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def steps(self) -> int:
        if self.prefilled:
            return self.seq_len
        return self.seq_len // self.chunk_len

    @property
    def fill_steps(self) -> int:
        return 0 if self.prefilled else self.cache_len // self.chunk_len

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 2 q heads / 1 kv head, D=64, C=256, S=64, T=2048
    "tiny": Workload("tiny", 0, 1, 2, 1, 64, 256, 64, 2048, 1,
                     1.0, 0.0, 1.0, False),
    # 8 q / 2 kv heads, D=128, C=2048, S=256, T=16384; N(0,1)/sqrt(128)
    "small_gqa": Workload("small_gqa", 1, 1, 8, 2, 128, 2048, 256, 16384, 1,
                          1.0 / math.sqrt(128.0), 0.0, 1.0, False),
    # Qwen3-4B-shaped layer at 64k: C=8192, S=2048, 5% heavy K rows x4
    "qwen3_4b_64k": Workload("qwen3_4b_64k", 2, 1, 32, 8, 128, 8192, 2048,
                             65536, 1, 1.0, 0.05, 4.0, False),
    # Qwen3-4B-shaped layers at 128k: C=16384, S=1024, 36 layers
    "qwen3_4b_128k": Workload("qwen3_4b_128k", 3, 1, 32, 8, 128, 16384, 1024,
                              131072, 36, 1.0, 0.05, 4.0, False),
    # small chunks at 64k: C=8192, S=128 (the pages' 128-token setting), 36 layers
    "qwen3_4b_64k_s128": Workload("qwen3_4b_64k_s128", 5, 1, 32, 8, 128, 8192, 128,
                                  65536, 36, 1.0, 0.05, 4.0, False),
    # the same layers with 256- and 512-token chunks (between the 128-token
    # setting and the 1k/2k chunks)
    "qwen3_4b_64k_s256": Workload("qwen3_4b_64k_s256", 8, 1, 32, 8, 128, 8192, 256,
                                  65536, 36, 1.0, 0.05, 4.0, False),
    "qwen3_4b_64k_s512": Workload("qwen3_4b_64k_s512", 9, 1, 32, 8, 128, 8192, 512,
                                  65536, 36, 1.0, 0.05, 4.0, False),
    # one GPU's share of the 128k layers under 8-way KV-head sharding: one KV
    # head with its 4 query heads, same cache, chunk and value distribution
    "qwen3_4b_128k_head": Workload("qwen3_4b_128k_head", 7, 1, 4, 1, 128, 16384, 1024,
                                   131072, 36, 1.0, 0.05, 4.0, False),
    # SnapKV-style one-shot choice at the end of a 131072-token prompt: the
    # cache holds the first 130048 prompt tokens (positions 0..130047), the
    # last 1024 form the observation window (the chunk); 15360 slots are
    # kept, so the compacted cache holds 16384 tokens like the 128k runs
    "qwen3_4b_128k_snapkv": Workload("qwen3_4b_128k_snapkv", 6, 1, 32, 8, 128, 130048, 1024,
                                     131072, 36, 1.0, 0.05, 4.0, True, 15360),
    # decode: 16 sequences, cache pre-filled, one token per step, 4096 steps
    "decode": Workload("decode", 4, 16, 32, 8, 128, 16384, 1, 4096, 1,
                       1.0, 0.05, 4.0, True),
}


def _rng(wl: Workload, layer: int, step: int, tensor: int, b: int = 0):
    ss = np.random.SeedSequence([BASE_SEED, wl.cfg_id, layer, step, tensor, b])
    return np.random.Generator(np.random.Philox(ss))


def to_bf16(x: np.ndarray):
    """Round float32 to bfloat16 (round to nearest, ties to even).

    Returns ``(bits, values)``: ``bits`` is uint16, ``values`` is the float32
    array those bits denote.  Inputs are finite here; NaN is not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    bits = r.astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(wl, layer, step, tensor, shape):
    """Per-batch-row streams so that B is a stack of independent sequences."""
    out = np.empty(shape, np.float32)
    for b in range(shape[0]):
        g = _rng(wl, layer, step, tensor, b)
        out[b] = g.standard_normal(shape[1:], dtype=np.float32)
    return out


def _heavy_mask(wl, layer, step, tensor, shape):
    """Bernoulli(heavy_frac) per (b, kv head, position) -> bool [B, Hkv, N]."""
    out = np.zeros(shape, bool)
    if wl.heavy_frac <= 0.0:
        return out
    for b in range(shape[0]):
        g = _rng(wl, layer, step, tensor, b)
        out[b] = g.random(shape[1:]) < wl.heavy_frac
    return out


@dataclass
class Chunk:
    """One chunk of new tokens for one layer.  ``*_bits`` are bf16 patterns."""
    q_bits: np.ndarray     # [B, Hq, S, D] uint16
    k_bits: np.ndarray     # [B, Hkv, S, D]
    v_bits: np.ndarray     # [B, Hkv, S, D]
    q: np.ndarray          # float32 values of the same
    k: np.ndarray
    v: np.ndarray
    p0: int                # absolute position of the chunk's first token


def gen_chunk(wl: Workload, layer: int, step: int) -> Chunk:
    B, Hq, Hkv, S, D = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.chunk_len, wl.head_dim
    q = _normal(wl, layer, step, T_Q, (B, Hq, S, D)) * np.float32(wl.value_std)
    k = _normal(wl, layer, step, T_K, (B, Hkv, S, D)) * np.float32(wl.value_std)
    v = _normal(wl, layer, step, T_V, (B, Hkv, S, D)) * np.float32(wl.value_std)
    heavy = _heavy_mask(wl, layer, step, T_HEAVY, (B, Hkv, S))
    k[heavy] *= np.float32(wl.heavy_scale)
    qb, qv = to_bf16(q)
    kb, kv = to_bf16(k)
    vb, vv = to_bf16(v)
    p0 = (wl.cache_len + step) if wl.prefilled else step * S
    return Chunk(qb, kb, vb, qv, kv, vv, p0)


@dataclass
class CacheState:
    """Full per-layer cache state: everything needed to resume a step."""
    k_bits: np.ndarray     # [B, Hkv, C, D] uint16
    v_bits: np.ndarray
    scores: np.ndarray     # [B, Hkv, C] float32
    pos: np.ndarray        # [B, Hkv, C] int64, -1 = empty
    n_valid: int

    @property
    def k(self):
        return bf16_bits_to_f32(self.k_bits)

    @property
    def v(self):
        return bf16_bits_to_f32(self.v_bits)

    def copy(self) -> "CacheState":
        return CacheState(self.k_bits.copy(), self.v_bits.copy(),
                          self.scores.copy(), self.pos.copy(), self.n_valid)


def empty_state(wl: Workload) -> CacheState:
    B, Hkv, C, D = wl.batch, wl.n_kv_heads, wl.cache_len, wl.head_dim
    return CacheState(np.zeros((B, Hkv, C, D), np.uint16),
                      np.zeros((B, Hkv, C, D), np.uint16),
                      np.zeros((B, Hkv, C), np.float32),
                      np.full((B, Hkv, C), -1, np.int64), 0)


def prefilled_state(wl: Workload, layer: int = 0) -> CacheState:
    """Cache pre-filled from seed: K/V drawn like chunk rows, scores 0,
    positions 0..C-1 in slot order, every slot valid."""
    B, Hkv, C, D = wl.batch, wl.n_kv_heads, wl.cache_len, wl.head_dim
    k = _normal(wl, layer, 0, T_KC, (B, Hkv, C, D)) * np.float32(wl.value_std)
    v = _normal(wl, layer, 0, T_VC, (B, Hkv, C, D)) * np.float32(wl.value_std)
    heavy = _heavy_mask(wl, layer, 0, T_HEAVY_C, (B, Hkv, C))
    k[heavy] *= np.float32(wl.heavy_scale)
    kb, _ = to_bf16(k)
    vb, _ = to_bf16(v)
    pos = np.broadcast_to(np.arange(C, dtype=np.int64), (B, Hkv, C)).copy()
    return CacheState(kb, vb, np.zeros((B, Hkv, C), np.float32), pos, C)


def steady_state(wl: Workload, layer: int = 0, step: int | None = None) -> CacheState:
    """A synthetic full cache as it could stand after ``step`` chunks.

    K/V rows are drawn like chunk rows, scores are positive (uniform on
    [0, 8)), and positions are a random choice of C distinct earlier
    positions.  Used to start a full-size step without replaying the whole
    history; any such state is a valid input to a step.
    """
    B, Hkv, C, D, S = wl.batch, wl.n_kv_heads, wl.cache_len, wl.head_dim, wl.chunk_len
    if step is None:
        step = wl.fill_steps + 2
    p0 = (C + step) if wl.prefilled else step * S
    st = prefilled_state(wl, layer)
    scores = np.empty((B, Hkv, C), np.float32)
    pos = np.empty((B, Hkv, C), np.int64)
    for b in range(B):
        g = _rng(wl, layer, step, T_SCORE, b)
        scores[b] = g.random((Hkv, C), dtype=np.float32) * np.float32(8.0)
        gp = _rng(wl, layer, step, T_POS, b)
        for h in range(Hkv):
            pos[b, h] = np.sort(gp.choice(p0, size=C, replace=False))
    st.scores = scores
    st.pos = pos
    return st


def partial_state(wl: Workload, n_valid: int, layer: int = 0) -> CacheState:
    """A cache filled up to ``n_valid`` slots during the fill phase: slot j holds
    position j, valid slots have positive scores, the rest are empty (-1)."""
    st = steady_state(wl, layer, wl.fill_steps + 2)
    st.n_valid = int(n_valid)
    st.pos[...] = -1
    st.pos[..., :n_valid] = np.arange(n_valid, dtype=np.int64)
    st.scores[..., n_valid:] = 0.0
    return st


def chunk_start(wl: Workload, step: int) -> int:
    return (wl.cache_len + step) if wl.prefilled else step * wl.chunk_len
