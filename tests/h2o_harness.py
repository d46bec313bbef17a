"""Shared helpers of the GPU parity tests: upload an oracle state, run one step
through the C ABI (via the ctypes binding), run the oracle on the same inputs,
and compare at the stated tolerances.

Tolerances (bf16 inputs, fp32 accumulation):
  out, wsum, new_scores   max-abs 2e-2
  lse                     max-abs 1e-3 (fp32 log-sum-exp of <= 2^20 terms)
  scores                  relative 1e-3
  evict_idx, slot layout  bit-exact, except that slots whose oracle score lies
                          within 1e-6 (relative) of the eviction cut may be
                          swapped.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import synth
import h2o_kv_cache_amd as h2o

TOL_OUT = 2e-2
TOL_WSUM = 2e-2
TOL_LSE = 1e-3
REL_SCORE = 1e-3
TIE_REL = 1e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    arr = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(arr).to("cuda").view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class HostState:
    k_bits: np.ndarray
    v_bits: np.ndarray
    scores: np.ndarray   # float32
    pos: np.ndarray      # int64
    n_valid: int


def state_from_synth(st: synth.CacheState) -> HostState:
    return HostState(st.k_bits.copy(), st.v_bits.copy(), st.scores.astype(np.float32),
                     st.pos.copy(), st.n_valid)


def shape_of(B, Hq, Hkv, D, C, S, n, scale=0.0) -> h2o.Shape:
    return h2o.Shape(B, Hq, Hkv, D, C, S, n, scale)


def gpu_step(shape: h2o.Shape, st: HostState, q_bits, k_bits, v_bits, p0, runs=1):
    """One step through the four C-ABI calls; returns host copies."""
    B, Hq, Hkv, D, C, S = (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.cache_len, shape.chunk_len)
    shape = shape.with_n(st.n_valid)
    results = []
    for _ in range(runs):
        kc, vc = dev_bf16(st.k_bits), dev_bf16(st.v_bits)
        scores = torch.from_numpy(st.scores.astype(np.float32)).cuda()
        pos = torch.from_numpy(st.pos.astype(np.int64)).cuda()
        q, kn, vn = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits)
        out = torch.full((B, Hq, S, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq, S), float("nan"), device="cuda")
        wsum = torch.full((B, Hkv, C + S), float("nan"), device="cuda")
        new_scores = torch.full((B, Hkv, S), float("nan"), device="cuda")
        evict = torch.full((B, Hkv, S), -7, dtype=torch.int32, device="cuda")
        ws = torch.full((max(h2o.h2o_workspace_size(shape), 256),), 0xFF, dtype=torch.uint8,
                        device="cuda")   # NaN-patterned scratch
        h2o.h2o_attn_chunk(shape, q, kc, vc, kn, vn, out, lse, wsum, ws)
        h2o.h2o_score_accumulate(shape, scores, new_scores, wsum)
        acc = scores.clone()
        h2o.h2o_evict_select(shape, scores, evict)
        h2o.kv_scatter(shape, kc, vc, scores, pos, kn, vn, new_scores, evict, p0)
        torch.cuda.synchronize()
        results.append(dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(),
                            wsum=wsum.cpu().numpy(), new_scores=new_scores.cpu().numpy(),
                            scores_acc=acc.cpu().numpy(), evict_idx=evict.cpu().numpy(),
                            k_bits=host_bits(kc), v_bits=host_bits(vc),
                            scores=scores.cpu().numpy(), pos=pos.cpu().numpy()))
    return results if runs > 1 else results[0]


def gpu_step_fused(shape: h2o.Shape, st: HostState, q_bits, k_bits, v_bits, p0):
    """One step through the single-call entry point h2o_step; host copies in
    the layout of gpu_step (scores_acc is not observable here and is left
    out)."""
    B, Hq, Hkv, D, C, S = (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.cache_len, shape.chunk_len)
    shape = shape.with_n(st.n_valid)
    kc, vc = dev_bf16(st.k_bits), dev_bf16(st.v_bits)
    scores = torch.from_numpy(st.scores.astype(np.float32)).cuda()
    pos = torch.from_numpy(st.pos.astype(np.int64)).cuda()
    q, kn, vn = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits)
    out = torch.full((B, Hq, S, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    wsum = torch.full((B, Hkv, C + S), float("nan"), device="cuda")
    new_scores = torch.full((B, Hkv, S), float("nan"), device="cuda")
    evict = torch.full((B, Hkv, S), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(h2o.h2o_workspace_size(shape), 256),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    h2o.h2o_step(shape, q, kc, vc, kn, vn, out, lse, wsum, scores, new_scores, evict, pos, p0, ws)
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), wsum=wsum.cpu().numpy(),
                new_scores=new_scores.cpu().numpy(), evict_idx=evict.cpu().numpy(),
                k_bits=host_bits(kc), v_bits=host_bits(vc), scores=scores.cpu().numpy(),
                pos=pos.cpu().numpy())


def oracle_step(st: HostState, q_bits, k_bits, v_bits, p0, scale=None, heads=None):
    """The oracle on the same inputs (float64).  ``heads`` restricts the
    comparison to a subset of KV heads (per-head work is independent)."""
    kc = synth.bf16_bits_to_f32(st.k_bits)
    vc = synth.bf16_bits_to_f32(st.v_bits)
    q = synth.bf16_bits_to_f32(q_bits)
    kn = synth.bf16_bits_to_f32(k_bits)
    vn = synth.bf16_bits_to_f32(v_bits)
    sc = st.scores.astype(np.float64)
    pos = st.pos
    if heads is not None:
        Hkv = kc.shape[1]
        G = q.shape[1] // Hkv
        qh = [h * G + g for h in heads for g in range(G)]
        kc, vc, kn, vn = kc[:, heads], vc[:, heads], kn[:, heads], vn[:, heads]
        sc, pos, q = sc[:, heads], pos[:, heads], q[:, qh]
    return oracle.h2o_step(kc, vc, sc, pos, st.n_valid, q, kn, vn, p0, scale)


def select_heads(g: dict, Hkv: int, G: int, heads):
    if heads is None:
        return g
    qh = [h * G + x for h in heads for x in range(G)]
    out = {}
    for k, v in g.items():
        if k in ("out", "lse"):
            out[k] = v[:, qh]
        else:
            out[k] = v[:, heads]
    return out


def _evict_ok(ge, re_, acc, n, C, S):
    """True if the GPU choice equals the oracle's, or differs only in slots
    whose oracle score is within TIE_REL of the eviction cut."""
    if np.array_equal(ge, re_):
        return True, True
    if len(set(ge.tolist())) != S or list(ge) != sorted(ge) or ge.min() < 0 or ge.max() >= C:
        return False, False
    free = C - n
    if free >= S or not set(range(n, C)).issubset(set(ge.tolist())):
        return False, False
    need = S - free
    vals = acc[:n]
    cut = np.sort(vals, kind="stable")[need - 1]
    for j in set(ge.tolist()) ^ set(re_.tolist()):
        if abs(vals[j] - cut) > TIE_REL * max(abs(cut), abs(vals[j]), 1e-30):
            return False, False
    return True, False


def compare(g: dict, r: dict, st: HostState, k_bits, v_bits, p0, label=""):
    """Assert parity of one step; returns a dict of error statistics."""
    stats = {}
    n = st.n_valid
    C = g["scores"].shape[-1]
    S = g["evict_idx"].shape[-1]
    e_out = float(np.max(np.abs(g["out"] - r["out"])))
    e_w = float(np.max(np.abs(g["wsum"] - r["wsum"])))
    e_lse = float(np.max(np.abs(g["lse"] - r["lse"])))
    e_new = float(np.max(np.abs(g["new_scores"] - r["new_scores"])))
    stats.update(out=e_out, wsum=e_w, lse=e_lse, new=e_new)
    assert np.all(np.isfinite(g["out"])), label
    assert e_out <= TOL_OUT, (label, "out", e_out)
    assert e_w <= TOL_WSUM, (label, "wsum", e_w)
    assert e_lse <= TOL_LSE, (label, "lse", e_lse)
    assert e_new <= TOL_WSUM, (label, "new_scores", e_new)
    # empty slots have exactly zero summed weight
    assert np.all(g["wsum"][..., n:C] == 0.0), label
    # accumulated scores, relative
    acc_r = r["scores_acc"]
    rel = np.abs(g["scores_acc"][..., :n] - acc_r[..., :n]) / np.maximum(np.abs(acc_r[..., :n]), 1e-6)
    stats["score_rel"] = float(rel.max()) if rel.size else 0.0
    assert stats["score_rel"] <= REL_SCORE, (label, "scores", stats["score_rel"])
    B, Hkv = g["evict_idx"].shape[:2]
    swaps = 0
    for b in range(B):
        for h in range(Hkv):
            ge = g["evict_idx"][b, h].astype(np.int64)
            re_ = r["evict_idx"][b, h]
            ok, same = _evict_ok(ge, re_, acc_r[b, h], n, C, S)
            assert ok, (label, "evict", b, h, ge[:16], re_[:16])
            kb_new = k_bits[b, h]
            vb_new = v_bits[b, h]
            if same:
                kr = synth.to_bf16(r["k_cache"][b, h].astype(np.float32))[0]
                vr = synth.to_bf16(r["v_cache"][b, h].astype(np.float32))[0]
                assert np.array_equal(g["k_bits"][b, h], kr), (label, "k layout", b, h)
                assert np.array_equal(g["v_bits"][b, h], vr), (label, "v layout", b, h)
                assert np.array_equal(g["pos"][b, h], r["pos"][b, h]), (label, "pos", b, h)
                srel = np.abs(g["scores"][b, h] - r["scores"][b, h]) / np.maximum(
                    np.abs(r["scores"][b, h]), 1e-6)
                valid = r["pos"][b, h] >= 0
                assert np.all(srel[valid] <= REL_SCORE), (label, "scores after", b, h)
            else:
                swaps += 1
            # the GPU layout agrees with the GPU's own choice
            for t, j in enumerate(ge):
                assert np.array_equal(g["k_bits"][b, h, j], kb_new[t]), (label, b, h, t)
                assert np.array_equal(g["v_bits"][b, h, j], vb_new[t]), (label, b, h, t)
                assert g["pos"][b, h, j] == p0 + t
    stats["tie_swaps"] = swaps
    return stats
