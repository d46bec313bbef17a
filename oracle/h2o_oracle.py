"""CPU oracle of one chunked H2O sparse-attention step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP library.

Sources (cited by page title and section; the pages are web copies of the
paper "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention",
arXiv 2608.19920):

* [LtF-zh] the Chinese translation page of the paper:
  §1 (sparse attention keeps K/V in a fixed number of slots; when the cache is
  full a policy evicts slots), §1 contributions (the H2O kernel returns the
  summed attention weights), §2 (SnapKV uses H2O-like summed attention
  weights; grouped attention heads; FlashInfer's 1 << N_q << N_k regime).
* [LtF-ko] the Korean summary page of the same paper: the glossary entry for
  H2O (slots are scored by how often and how strongly they were attended to,
  and the low scorers are evicted), Table 1 / Table 5 captions (sequences are
  processed in chunks of S = 2048, 1024 or 128 tokens).

The pages define the policy only in these words; the section that details H2O
is not part of them.  Where they are silent this oracle takes the plainest
reading, listed here and implemented below:

  R1  score of a slot = raw sum of the softmax weights it received since it
      was inserted (no normalisation, no decay);
  R2  scores are kept per (batch, KV head): the weights of the G query heads
      that share a KV head are summed together;
  R3  query head a reads KV head a // G (contiguous groups);
  R4  logits are tau * <q, k> with tau = 1/sqrt(D) unless a scale is given;
  R5  every valid cache slot is visible to every chunk query; inside the chunk
      query i sees chunk keys t <= i;
  R6  a freshly inserted token starts with the weight its own chunk gave it
      (the chunk columns of the summed weights);
  R7  scores are accumulated first, then the S slots to overwrite are chosen
      among the C cache slots; the chunk itself is always inserted;
  R8  empty slots (index >= n_valid) are taken first, in slot order; then
      valid slots in increasing (score, slot) order, NaN scores last;
  R9  the chosen slots are listed in increasing slot order and chunk token t
      goes to the t-th of them;
  R10 positions are absolute token indices; -1 marks an empty slot.

  R18 8-bit cache (Q-Hitter-like): cached K and V rows are stored as int8
      codes with one float32 scale per (token, KV head) row, amax / 127,
      codes = round-half-even(x / scale); attention reads the dequantised
      rows, the chunk's own K/V are used unquantised in their step and
      quantised when written; scores and the choice are unchanged.
  R17 SnapKV-style one-shot choice: made once, from the summed weights of
      one observation chunk (the window) over the cache slots; the lowest
      (weight, slot) slots beyond the budget are dropped in R8's order, the
      kept slots are compacted in slot order and the window is appended.

The backward of the attention with the slot layout fixed
(``attention_chunk_backward``) follows [LtF-zh] abstract and §1: the paper's
fine-tuning computes gradients through the sparse attention with the cache
policy in place.

Arithmetic is float64 by default.  ``dtype=np.float32`` runs the same code in
float32 (the timed CPU baseline).  Inputs are the bf16-rounded values the
device sees, passed in as float arrays.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# a1 + a2: attention of the chunk over (valid cache slots) + (causal chunk)
# ---------------------------------------------------------------------------
def attention_chunk(q, k_cache, v_cache, k_new, v_new, n_valid, scale=None,
                    dtype=np.float64):
    """Causal GQA attention of a query chunk against cache slots and chunk.

    Shapes: q [B, Hq, S, D]; k_cache, v_cache [B, Hkv, C, D];
    k_new, v_new [B, Hkv, S, D]; 0 <= n_valid <= C.

    Returns ``(out, lse, wsum)``:
      out  [B, Hq, S, D]   softmax(logits) @ values over the visible keys (R5);
      lse  [B, Hq, S]      natural-log log-sum-exp of each row's logits;
      wsum [B, Hkv, C + S] summed attention weights per key (R1, R2): column
           j < n_valid is cache slot j, n_valid <= j < C is 0 (empty slot),
           column C + t is chunk token t.

    Follows [LtF-zh] §1 contributions (attention that also returns the summed
    attention weights) and §2 (SnapKV's summed attention weights; grouped
    query heads).
    """
    B, Hq, S, D = q.shape
    Hkv, C = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    n = int(n_valid)
    tau = (1.0 / math.sqrt(D)) if (scale is None or scale <= 0) else float(scale)
    out = np.zeros((B, Hq, S, D), dtype)
    lse = np.zeros((B, Hq, S), dtype)
    wsum = np.zeros((B, Hkv, C + S), dtype)
    # visible[i, j]: all n cache slots, then chunk key t visible iff t <= i
    visible = np.concatenate([np.ones((S, n), bool),
                              np.tril(np.ones((S, S), bool))], axis=1)
    for b in range(B):
        for a in range(Hq):
            h = a // G                                            # R3
            keys = np.concatenate([k_cache[b, h, :n], k_new[b, h]]).astype(dtype)
            vals = np.concatenate([v_cache[b, h, :n], v_new[b, h]]).astype(dtype)
            s = dtype(tau) * (q[b, a].astype(dtype) @ keys.T)     # [S, n+S]
            s = np.where(visible, s, dtype(-np.inf))
            m = s.max(axis=1, keepdims=True)
            L = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            p = np.exp(s - L)                                     # masked -> 0
            out[b, a] = p @ vals
            lse[b, a] = L[:, 0]
            col = p.sum(axis=0)                                   # over queries
            wsum[b, h, :n] += col[:n]                             # R2
            wsum[b, h, C:] += col[n:]
    return out, lse, wsum


def attention_chunk_backward(q, k_cache, v_cache, k_new, v_new, n_valid, dout, scale=None,
                             dtype=np.float64):
    """Gradients of ``out`` of :func:`attention_chunk` with respect to all of
    its inputs, for a given upstream gradient ``dout`` [B, Hq, S, D].

    The slot layout (which keys are visible) is fixed: the eviction decisions
    that produced it are discrete and not differentiated.  This is the step a
    fine-tuning loop calls to push gradients through the sparse attention with
    the cache policy in place ([LtF-zh] abstract and §1: gradients for the
    whole model are computed under any KV cache policy, with no approximation
    beyond the sparse attention itself).

    Written out from the chain rule of out = softmax(tau Q K^T) V over the
    visible keys (R3-R5):  dp = dout V^T;  D_i = sum_j p_ij dp_ij;
    ds = p * (dp - D);  dq = tau ds K;  dk = tau ds^T Q;  dv = p^T dout,
    with the G query heads of a KV head summed into its key / value gradients.

    Returns ``(dq, dk_cache, dv_cache, dk_new, dv_new)``; the cache gradients
    are zero for empty slots (index >= n_valid).
    """
    B, Hq, S, D = q.shape
    Hkv, C = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    n = int(n_valid)
    tau = (1.0 / math.sqrt(D)) if (scale is None or scale <= 0) else float(scale)
    dq = np.zeros((B, Hq, S, D), dtype)
    dk_cache = np.zeros((B, Hkv, C, D), dtype)
    dv_cache = np.zeros((B, Hkv, C, D), dtype)
    dk_new = np.zeros((B, Hkv, S, D), dtype)
    dv_new = np.zeros((B, Hkv, S, D), dtype)
    visible = np.concatenate([np.ones((S, n), bool),
                              np.tril(np.ones((S, S), bool))], axis=1)
    for b in range(B):
        for a in range(Hq):
            h = a // G
            keys = np.concatenate([k_cache[b, h, :n], k_new[b, h]]).astype(dtype)
            vals = np.concatenate([v_cache[b, h, :n], v_new[b, h]]).astype(dtype)
            qa = q[b, a].astype(dtype)
            go = dout[b, a].astype(dtype)
            s = dtype(tau) * (qa @ keys.T)
            s = np.where(visible, s, dtype(-np.inf))
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)                      # masked -> 0
            dp = go @ vals.T
            drow = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - drow)
            dq[b, a] = dtype(tau) * (ds @ keys)
            dk = dtype(tau) * (ds.T @ qa)
            dv = p.T @ go
            dk_cache[b, h, :n] += dk[:n]
            dv_cache[b, h, :n] += dv[:n]
            dk_new[b, h] += dk[n:]
            dv_new[b, h] += dv[n:]
    return dq, dk_cache, dv_cache, dk_new, dv_new


# ---------------------------------------------------------------------------
# a3: score accumulation
# ---------------------------------------------------------------------------
def score_accumulate(scores, wsum, n_valid):
    """Add this step's summed weights to the scores of the valid slots (R1)
    and return the starting scores of the chunk tokens (R6).

    scores [B, Hkv, C] (not modified); wsum [B, Hkv, C + S].
    Returns ``(scores_after, new_scores [B, Hkv, S])``.
    [LtF-ko] glossary (H2O scores slots by accumulated attention);
    [LtF-zh] §2 (summed attention weights as the score).
    """
    C = scores.shape[-1]
    n = int(n_valid)
    acc = scores.astype(wsum.dtype, copy=True)
    acc[..., :n] += wsum[..., :n]
    return acc, wsum[..., C:].copy()


# ---------------------------------------------------------------------------
# a4: eviction choice
# ---------------------------------------------------------------------------
def evict_select(scores, n_valid, S):
    """The S slots each (batch, KV head) overwrites this step (R7-R9).

    Empty slots come first in slot order; the rest are the lowest-scoring valid
    slots, ties broken towards the lower slot index and NaN scores taken last.
    The result [B, Hkv, S] (int64) is sorted by slot index.
    [LtF-zh] §1 (evict slots only when the cache is full);
    [LtF-ko] glossary (low-scoring entries are the ones evicted).
    """
    B, Hkv, C = scores.shape
    n = int(n_valid)
    out = np.empty((B, Hkv, S), np.int64)
    free = np.arange(n, C, dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            if free.size >= S:
                chosen = free[:S]
            else:
                need = S - free.size
                # stable sort: equal scores keep slot order; NaN sorts last
                order = np.argsort(scores[b, h, :n], kind="stable")
                chosen = np.concatenate([free, order[:need].astype(np.int64)])
            out[b, h] = np.sort(chosen)
    return out


# ---------------------------------------------------------------------------
# a5: scatter of the chunk into the chosen slots
# ---------------------------------------------------------------------------
def kv_scatter(k_cache, v_cache, scores, pos, k_new, v_new, new_scores,
               evict_idx, p0):
    """Write chunk token t into slot evict_idx[..., t] (R9, R10), in place.

    k_cache, v_cache [B, Hkv, C, D]; scores, pos [B, Hkv, C];
    k_new, v_new [B, Hkv, S, D]; new_scores [B, Hkv, S].
    [LtF-zh] §1 (the chunk's K/V take the evicted slots).
    """
    B, Hkv, S = evict_idx.shape
    for b in range(B):
        for h in range(Hkv):
            for t in range(S):
                j = int(evict_idx[b, h, t])
                k_cache[b, h, j] = k_new[b, h, t]
                v_cache[b, h, j] = v_new[b, h, t]
                scores[b, h, j] = new_scores[b, h, t]
                pos[b, h, j] = p0 + t


# ---------------------------------------------------------------------------
# Quantised (8-bit) KV cache: Q-Hitter-like H2O over int8 cache rows
# ---------------------------------------------------------------------------
def quantize_rows_int8(x):
    """Symmetric 8-bit quantisation of K or V rows, one scale per row (R18).

    [LtF-zh] §2: cache buffers can be quantised to 8 bits (or fewer), and
    Q-Hitter combines H2O with such quantisation.  Reading: every stored
    (token, KV head) row gets scale = amax / 127 (amax = the row's largest
    |x|) and codes = round-half-even(x / scale), both computed in float32, the
    precision the device takes the same decision in; a row of zeros gets
    scale 0 and codes 0.  Rows must be finite.
    x [..., D] (float32 values, here bf16-representable); returns
    (codes int8 [..., D], scale float32 [...]).
    """
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / safe[..., None])                      # float32 division
    q = np.clip(q, -127, 127)
    q = np.where(scale[..., None] > 0, q, 0)
    return q.astype(np.int8), scale


def dequantize_rows_int8(codes, scale, dtype=np.float64):
    """codes * scale, exactly (float64)."""
    return codes.astype(dtype) * np.asarray(scale, dtype)[..., None]


def attention_chunk_q8(q, kq, k_scale, vq, v_scale, k_new, v_new, n_valid, scale=None,
                       dtype=np.float64):
    """a1 + a2 with the cache slots stored as int8 rows (R18): the cache keys
    and values are the dequantised rows; the chunk's own keys and values are
    used as given (they are quantised only when written into the cache).
    Returns (out, lse, wsum) as :func:`attention_chunk`."""
    return attention_chunk(q, dequantize_rows_int8(kq, k_scale, dtype),
                           dequantize_rows_int8(vq, v_scale, dtype), k_new, v_new,
                           n_valid, scale, dtype)


def kv_scatter_q8(kq, k_scale, vq, v_scale, scores, pos, k_new, v_new, new_scores,
                  evict_idx, p0):
    """a5 into an int8 cache (R18), in place: chunk token t is quantised and
    written to slot evict_idx[..., t] (codes and scale), with its score and
    position as :func:`kv_scatter`."""
    ck, sk = quantize_rows_int8(k_new)
    cv, sv = quantize_rows_int8(v_new)
    B, Hkv, S = evict_idx.shape
    for b in range(B):
        for h in range(Hkv):
            for t in range(S):
                j = int(evict_idx[b, h, t])
                kq[b, h, j] = ck[b, h, t]
                vq[b, h, j] = cv[b, h, t]
                k_scale[b, h, j] = sk[b, h, t]
                v_scale[b, h, j] = sv[b, h, t]
                scores[b, h, j] = new_scores[b, h, t]
                pos[b, h, j] = p0 + t


# ---------------------------------------------------------------------------
# SnapKV-style one-shot choice from the same summed weights
# ---------------------------------------------------------------------------
def snapkv_keep(wsum, n_valid, budget):
    """The `budget` cache slots each (batch, KV head) keeps when the choice is
    made once, from one observation chunk's summed weights.

    [LtF-zh] §2: SnapKV ranks cache entries by H2O-like summed attention
    weights but decides only at one point of the generation.  Reading (R17):
    the weights are the summed weights ``attention_chunk`` returns for the
    window chunk, columns j < n_valid; the n_valid - budget slots with the
    lowest (weight, slot) pairs are dropped -- the order of R8: equal weights
    drop the lower slot first, -0.0 equals +0.0, NaN ranks last -- and the
    rest are kept, listed in increasing slot order.
    wsum [B, Hkv, C + S]; returns [B, Hkv, budget] int64.
    """
    B, Hkv, _ = wsum.shape
    n = int(n_valid)
    budget = int(budget)
    drop = n - budget
    out = np.empty((B, Hkv, budget), np.int64)
    for b in range(B):
        for h in range(Hkv):
            # stable sort: equal weights keep slot order; NaN sorts last
            order = np.argsort(wsum[b, h, :n], kind="stable")
            out[b, h] = np.sort(order[drop:])
    return out


def snapkv_compact(k_cache, v_cache, pos, k_new, v_new, wsum, keep_idx, out_len, p0):
    """The cache after a SnapKV choice, in a new cache of out_len slots (R17):
    slot i < budget holds kept slot keep_idx[i] (its K, V, position and
    summed weight), slot budget + t holds window token t (position p0 + t,
    score = its own column, as R6), later slots are empty (position -1,
    zeros).  Returns (k_out, v_out, pos_out, scores_out).
    [LtF-zh] §1 (fixed slots) and §2 (SnapKV keeps the entries it chose).
    """
    B, Hkv, C, D = k_cache.shape
    S = k_new.shape[2]
    budget = keep_idx.shape[2]
    k_out = np.zeros((B, Hkv, out_len, D), k_cache.dtype)
    v_out = np.zeros((B, Hkv, out_len, D), v_cache.dtype)
    pos_out = np.full((B, Hkv, out_len), -1, np.int64)
    scores_out = np.zeros((B, Hkv, out_len), wsum.dtype)
    for b in range(B):
        for h in range(Hkv):
            for i in range(budget):
                j = int(keep_idx[b, h, i])
                k_out[b, h, i] = k_cache[b, h, j]
                v_out[b, h, i] = v_cache[b, h, j]
                pos_out[b, h, i] = pos[b, h, j]
                scores_out[b, h, i] = wsum[b, h, j]
            for t in range(S):
                k_out[b, h, budget + t] = k_new[b, h, t]
                v_out[b, h, budget + t] = v_new[b, h, t]
                pos_out[b, h, budget + t] = p0 + t
                scores_out[b, h, budget + t] = wsum[b, h, C + t]
    return k_out, v_out, pos_out, scores_out


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------
def h2o_step(k_cache, v_cache, scores, pos, n_valid, q, k_new, v_new, p0,
             scale=None, dtype=np.float64):
    """One chunk step: attend, accumulate, choose, scatter.

    The cache arrays are not modified; updated copies are returned.
    Returns a dict with out, lse, wsum, scores_acc (after accumulation, before
    the scatter), new_scores, evict_idx and the next state (k_cache, v_cache,
    scores, pos, n_valid).
    """
    C = k_cache.shape[2]
    S = q.shape[2]
    out, lse, wsum = attention_chunk(q, k_cache, v_cache, k_new, v_new,
                                     n_valid, scale, dtype)
    acc, new_scores = score_accumulate(scores, wsum, n_valid)
    evict = evict_select(acc, n_valid, S)
    kc = k_cache.copy()
    vc = v_cache.copy()
    sc = acc.copy()
    ps = pos.copy()
    kv_scatter(kc, vc, sc, ps, k_new, v_new, new_scores, evict, p0)
    return dict(out=out, lse=lse, wsum=wsum, scores_acc=acc,
                new_scores=new_scores, evict_idx=evict, k_cache=kc,
                v_cache=vc, scores=sc, pos=ps,
                n_valid=min(C, int(n_valid) + S))


def h2o_step_q8(kq, k_scale, vq, v_scale, scores, pos, n_valid, q, k_new, v_new, p0,
                scale=None, dtype=np.float64):
    """One chunk step over an int8 cache (R18): attend to the dequantised
    cache, accumulate, choose (unchanged), scatter the quantised chunk.
    The cache arrays are not modified; updated copies are returned in a dict
    like :func:`h2o_step` (keys kq, k_scale, vq, v_scale instead of
    k_cache, v_cache)."""
    C = kq.shape[2]
    S = q.shape[2]
    out, lse, wsum = attention_chunk_q8(q, kq, k_scale, vq, v_scale, k_new, v_new, n_valid,
                                        scale, dtype)
    acc, new_scores = score_accumulate(scores, wsum, n_valid)
    evict = evict_select(acc, n_valid, S)
    kq2, ks2, vq2, vs2 = kq.copy(), k_scale.copy(), vq.copy(), v_scale.copy()
    sc = acc.copy()
    ps = pos.copy()
    kv_scatter_q8(kq2, ks2, vq2, vs2, sc, ps, k_new, v_new, new_scores, evict, p0)
    return dict(out=out, lse=lse, wsum=wsum, scores_acc=acc, new_scores=new_scores,
                evict_idx=evict, kq=kq2, k_scale=ks2, vq=vq2, v_scale=vs2, scores=sc,
                pos=ps, n_valid=min(C, int(n_valid) + S))
