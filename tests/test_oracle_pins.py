"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a library routine on a special case, a
brute-force re-simulation written independently of it, an exact closed form
or an invariant of the definitions.  Together they are meant to catch a
dropped term, a wrong sign, index or mask, or a transposed operand anywhere in
``oracle/h2o_oracle.py``.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _run_steps(q_all, k_all, v_all, C, S, scale=None):
    """Drive the oracle over a whole sequence; returns per-step results."""
    B, Hq, T, D = q_all.shape
    Hkv = k_all.shape[1]
    kc = np.zeros((B, Hkv, C, D))
    vc = np.zeros((B, Hkv, C, D))
    sc = np.zeros((B, Hkv, C))
    pos = np.full((B, Hkv, C), -1, np.int64)
    n = 0
    res = []
    for step in range(T // S):
        sl = slice(step * S, (step + 1) * S)
        r = oracle.h2o_step(kc, vc, sc, pos, n, q_all[:, :, sl], k_all[:, :, sl],
                            v_all[:, :, sl], step * S, scale)
        r["n_before"] = n
        r["scores_before"] = sc
        r["pos_before"] = pos
        res.append(r)
        kc, vc, sc, pos, n = r["k_cache"], r["v_cache"], r["scores"], r["pos"], r["n_valid"]
    return res


# ---------------------------------------------------------------------------
# 1. cache >= sequence: exactly causal GQA attention (library routine)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,D,S,T", [(2, 4, 2, 16, 16, 128), (1, 6, 2, 8, 5, 40),
                                            (1, 2, 1, 64, 64, 256)])
def test_no_eviction_equals_causal_sdpa(B, Hq, Hkv, D, S, T):
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    res = _run_steps(q, k, v, C=T, S=S)
    out = np.concatenate([r["out"] for r in res], axis=2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # nothing was ever evicted: slots hold positions in order
    assert np.array_equal(res[-1]["pos"], np.broadcast_to(np.arange(T), (B, Hkv, T)))


def test_no_eviction_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, D, S, T = 1, 4, 2, 16, 8, 64
    q, k, v = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    res = _run_steps(q, k, v, C=T, S=S)
    lse = np.concatenate([r["lse"] for r in res], axis=2)
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    logits = (qt @ kt.transpose(-1, -2)) / math.sqrt(D)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    ref = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 2. brute force: full history + explicit keep-mask over positions
# ---------------------------------------------------------------------------
def _bruteforce(q_all, k_all, v_all, C, S):
    """Independent re-simulation indexed by absolute position.

    It keeps the whole history and, per (b, kv head), the set of kept
    positions, the score of every kept position and the slot each occupies.
    Attention at each step runs over the full history with a keep-mask.
    """
    B, Hq, T, D = q_all.shape
    Hkv = k_all.shape[1]
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(D)
    kept = [[dict() for _ in range(Hkv)] for _ in range(B)]     # pos -> slot
    score = [[dict() for _ in range(Hkv)] for _ in range(B)]    # pos -> score
    steps = []
    for step in range(T // S):
        p0 = step * S
        outs = np.zeros((B, Hq, S, D))
        wpos = [[dict() for _ in range(Hkv)] for _ in range(B)]  # pos -> weight
        for b in range(B):
            for a in range(Hq):
                h = a // G
                for i in range(S):
                    qi = q_all[b, a, p0 + i]
                    vis = [p for p in range(p0 + i + 1)
                           if p >= p0 or p in kept[b][h]]
                    logit = np.array([tau * float(qi @ k_all[b, h, p]) for p in vis])
                    w = np.exp(logit - logit.max())
                    w /= w.sum()
                    outs[b, a, i] = sum(wk * v_all[b, h, p] for wk, p in zip(w, vis))
                    for wk, p in zip(w, vis):
                        wpos[b][h][p] = wpos[b][h].get(p, 0.0) + wk
        evicted = [[None] * Hkv for _ in range(B)]
        for b in range(B):
            for h in range(Hkv):
                for p in kept[b][h]:
                    score[b][h][p] += wpos[b][h][p]
                used = set(kept[b][h].values())
                free = [j for j in range(C) if j not in used]
                if len(free) >= S:
                    slots = free[:S]
                    gone = []
                else:
                    need = S - len(free)
                    ranked = sorted(kept[b][h], key=lambda p: (score[b][h][p], kept[b][h][p]))
                    gone = ranked[:need]
                    slots = sorted(free + [kept[b][h][p] for p in gone])
                for p in gone:
                    del kept[b][h][p]
                    del score[b][h][p]
                for t, j in enumerate(slots):
                    kept[b][h][p0 + t] = j
                    score[b][h][p0 + t] = wpos[b][h][p0 + t]
                evicted[b][h] = slots
        steps.append(dict(out=outs, wpos=wpos, evict=evicted,
                          kept=[[dict(kept[b][h]) for h in range(Hkv)] for b in range(B)],
                          score=[[dict(score[b][h]) for h in range(Hkv)] for b in range(B)]))
    return steps


@pytest.mark.parametrize("B,Hq,Hkv,D,C,S,T", [(1, 4, 2, 8, 24, 8, 96), (2, 2, 1, 4, 16, 4, 64),
                                              (1, 3, 3, 4, 12, 5, 60)])
def test_slot_oracle_equals_bruteforce(B, Hq, Hkv, D, C, S, T):
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D, std=1.5), _rand(rng, B, Hkv, T, D)
    res = _run_steps(q, k, v, C, S)
    bf = _bruteforce(q, k, v, C, S)
    for r, x in zip(res, bf):
        np.testing.assert_allclose(r["out"], x["out"], rtol=0, atol=1e-12)
        n = r["n_before"]
        for b in range(B):
            for h in range(Hkv):
                pos_before = r["pos_before"][b, h]
                for j in range(C):
                    expect = x["wpos"][b][h][int(pos_before[j])] if j < n else 0.0
                    assert abs(r["wsum"][b, h, j] - expect) < 1e-12
                p0 = r["pos"][b, h].max() - S + 1
                for t in range(S):
                    assert abs(r["wsum"][b, h, C + t] - x["wpos"][b][h][p0 + t]) < 1e-12
                assert list(r["evict_idx"][b, h]) == x["evict"][b][h]
                # layout: slot -> position and slot -> score agree with brute force
                kept = x["kept"][b][h]
                assert sorted(kept.values()) == [j for j in range(C) if r["pos"][b, h, j] >= 0]
                for p, j in kept.items():
                    assert r["pos"][b, h, j] == p
                    assert abs(r["scores"][b, h, j] - x["score"][b][h][p]) < 1e-12
                    assert np.array_equal(r["k_cache"][b, h, j], k[b, h, p])
                    assert np.array_equal(r["v_cache"][b, h, j], v[b, h, p])


# ---------------------------------------------------------------------------
# 3. closed form under uniform attention (exact rationals, tests/golden)
# ---------------------------------------------------------------------------
def test_uniform_attention_closed_form():
    with open(os.path.join(HERE, "golden", "uniform_attention.json")) as f:
        cases = json.load(f)["cases"]
    rng = np.random.default_rng(4)
    for cs in cases:
        n, S, G, C = cs["n_valid"], cs["chunk_len"], cs["group"], cs["cache_len"]
        B, Hkv, D = 1, 2, 8
        Hq = G * Hkv
        q = _rand(rng, B, Hq, S, D)
        kc = np.zeros((B, Hkv, C, D))
        kn = np.zeros((B, Hkv, S, D))
        vc = _rand(rng, B, Hkv, C, D)
        vn = _rand(rng, B, Hkv, S, D)
        out, lse, wsum = oracle.attention_chunk(q, kc, vc, kn, vn, n)
        cache_w = float(Fraction(*cs["cache_slot_wsum"]))
        np.testing.assert_allclose(wsum[:, :, :n], np.full(wsum[:, :, :n].shape, cache_w),
                                   rtol=1e-14, atol=0)
        assert np.all(wsum[:, :, n:C] == 0.0)
        for t in range(S):
            np.testing.assert_allclose(wsum[:, :, C + t],
                                       np.full(wsum[:, :, C + t].shape, float(Fraction(*cs["chunk_wsum"][t]))),
                                       rtol=1e-14, atol=0)
        np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.array(cs["lse_exp"], float)), lse.shape),
                                   rtol=0, atol=1e-14)
        for a in range(Hq):
            h = a // G
            for i in range(S):
                mean = np.concatenate([vc[0, h, :n], vn[0, h, :i + 1]]).mean(axis=0)
                np.testing.assert_allclose(out[0, a, i], mean, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# 4. invariants of one step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [0, 8, 16, 24, 32])
def test_summed_weights_total_and_mass_conservation(n):
    rng = np.random.default_rng(5 + n)
    B, Hq, Hkv, D, C, S = 2, 6, 2, 8, 32, 8
    G = Hq // Hkv
    q = _rand(rng, B, Hq, S, D)
    kc, vc = _rand(rng, B, Hkv, C, D, std=2.0), _rand(rng, B, Hkv, C, D)
    kn, vn = _rand(rng, B, Hkv, S, D, std=2.0), _rand(rng, B, Hkv, S, D)
    sc = rng.random((B, Hkv, C)) * 3.0
    pos = np.full((B, Hkv, C), -1, np.int64)
    pos[:, :, :n] = np.arange(n)
    r = oracle.h2o_step(kc, vc, sc, pos, n, q, kn, vn, p0=100)
    # every query row's weights sum to 1: total = S * G per kv head
    np.testing.assert_allclose(r["wsum"].sum(axis=-1), np.full((B, Hkv), float(S * G)), rtol=1e-13)
    assert np.all(r["wsum"] >= 0.0)
    # mass: sum(after) = sum(before over valid) + S*G - sum(evicted, accumulated)
    n_after = r["n_valid"]
    for b in range(B):
        for h in range(Hkv):
            ev = r["evict_idx"][b, h]
            ev_valid = ev[ev < n]
            before = sc[b, h, :n].sum()
            after = r["scores"][b, h, :n_after].sum()
            lost = r["scores_acc"][b, h, ev_valid].sum()
            assert abs(after - (before + S * G - lost)) < 1e-11
    # accumulate touched only valid slots
    assert np.array_equal(r["scores_acc"][:, :, n:], sc[:, :, n:])


def test_accumulate_adds_only_valid_slots():
    sc = np.arange(12, dtype=float).reshape(1, 2, 6)
    w = np.ones((1, 2, 6 + 3)) * 0.5
    w[..., 6:] = [[[7.0, 8.0, 9.0]]]
    acc, new = oracle.score_accumulate(sc, w, 4)
    assert np.array_equal(acc[..., :4], sc[..., :4] + 0.5)
    assert np.array_equal(acc[..., 4:], sc[..., 4:])
    assert np.array_equal(new, np.broadcast_to([7.0, 8.0, 9.0], (1, 2, 3)))


# ---------------------------------------------------------------------------
# 5. selection against brute force
# ---------------------------------------------------------------------------
def _select_bruteforce(scores_row, n, S):
    C = scores_row.shape[0]
    free = list(range(n, C))
    if len(free) >= S:
        return free[:S]

    def key(j):
        s = float(scores_row[j])
        return (1, 0.0, j) if math.isnan(s) else (0, s, j)
    ranked = sorted(range(n), key=key)
    return sorted(free + ranked[:S - len(free)])


def test_select_matches_full_sort():
    rng = np.random.default_rng(6)
    for trial in range(200):
        C = int(rng.integers(1, 40))
        S = int(rng.integers(1, C + 1))
        n = int(rng.integers(0, C + 1))
        kind = trial % 4
        if kind == 0:
            s = rng.random((2, 3, C))
        elif kind == 1:                                   # many exact ties
            s = rng.integers(0, 3, (2, 3, C)).astype(float)
        elif kind == 2:                                   # specials
            s = rng.choice([0.0, -0.0, 1.0, np.inf, -np.inf, np.nan, 2.5, -1.0], (2, 3, C))
        else:
            s = rng.standard_normal((2, 3, C)).astype(np.float32)
        e = oracle.evict_select(s, n, S)
        for b in range(2):
            for h in range(3):
                assert list(e[b, h]) == _select_bruteforce(s[b, h], n, S), (C, S, n, s[b, h])


def test_select_single_slot_is_argmin():
    rng = np.random.default_rng(7)
    for _ in range(50):
        s = rng.integers(0, 5, (3, 4, 33)).astype(float)    # ties: first index wins
        e = oracle.evict_select(s, 33, 1)
        assert np.array_equal(e[..., 0], np.argmin(s, axis=-1))


# ---------------------------------------------------------------------------
# 6. exact-tie trajectory (closed form), decode shaped
# ---------------------------------------------------------------------------
def test_exact_tie_trajectory_evicts_slot_zero():
    """S = 1, scores start at 0, K = 0 so attention is uniform over C + 1 keys
    with weight w = G / (C + 1) per column.  Step 1: all C slots tie at w, slot
    0 goes (lowest index), the new token starts at w.  Step 2: all slots tie at
    2w, slot 0 goes again.  From step 3 on slot 0 is the strict minimum."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, C = 1, 4, 1, 8, 16
    G = Hq // Hkv
    w = G / (C + 1)
    kc = np.zeros((B, Hkv, C, D))
    vc = _rand(rng, B, Hkv, C, D)
    sc = np.zeros((B, Hkv, C))
    pos = np.broadcast_to(np.arange(C), (B, Hkv, C)).astype(np.int64).copy()
    n = C
    for step in range(6):
        q = _rand(rng, B, Hq, 1, D)
        r = oracle.h2o_step(kc, vc, sc, pos, n, q, np.zeros((B, Hkv, 1, D)),
                            _rand(rng, B, Hkv, 1, D), p0=C + step)
        assert r["evict_idx"][0, 0, 0] == 0
        assert r["new_scores"][0, 0, 0] == pytest.approx(w, rel=1e-15)
        if step < 2:   # exact tie among all slots
            assert np.all(r["scores_acc"][0, 0] == r["scores_acc"][0, 0, 0])
        else:
            assert r["scores_acc"][0, 0, 0] < r["scores_acc"][0, 0, 1:].min()
        kc, vc, sc, pos = r["k_cache"], r["v_cache"], r["scores"], r["pos"]
        assert pos[0, 0, 0] == C + step


# ---------------------------------------------------------------------------
# 7. layout invariants of the scatter
# ---------------------------------------------------------------------------
def test_scatter_layout_invariants():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, C, S, T = 2, 4, 2, 8, 40, 8, 200
    q, k, v = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    res = _run_steps(q, k, v, C, S)
    for step, r in enumerate(res):
        p0 = step * S
        for b in range(B):
            for h in range(Hkv):
                pos = r["pos"][b, h]
                valid = pos[pos >= 0]
                assert len(set(valid.tolist())) == valid.size           # unique
                kept_before = set(r["pos_before"][b, h][r["pos_before"][b, h] >= 0].tolist())
                ev = r["evict_idx"][b, h]
                gone = {int(r["pos_before"][b, h][j]) for j in ev if r["pos_before"][b, h][j] >= 0}
                assert set(valid.tolist()) == (kept_before - gone) | set(range(p0, p0 + S))
                for t, j in enumerate(ev):
                    assert np.array_equal(r["k_cache"][b, h, j], k[b, h, p0 + t])
                    assert np.array_equal(r["v_cache"][b, h, j], v[b, h, p0 + t])
                    assert r["scores"][b, h, j] == r["wsum"][b, h, C + t]
                assert list(ev) == sorted(ev)
        assert r["n_valid"] == min(C, (step + 1) * S)


def test_partial_overflow_takes_free_slots_then_lowest():
    """n = C - 3 with S = 5: the 3 empty slots plus the 2 lowest-scoring valid
    slots are overwritten, in slot order."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, D, C, S = 1, 2, 1, 4, 12, 5
    n = C - 3
    sc = np.array([[[5.0, 0.1, 7.0, 0.2, 9.0, 9.0, 9.0, 9.0, 0.05, 0, 0, 0]]])
    kc, vc = _rand(rng, B, Hkv, C, D), _rand(rng, B, Hkv, C, D)
    pos = np.full((B, Hkv, C), -1, np.int64)
    pos[..., :n] = np.arange(n)
    q, kn, vn = _rand(rng, B, Hq, S, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    r = oracle.h2o_step(kc, vc, sc, pos, n, q, kn, vn, p0=50)
    acc = r["scores_acc"][0, 0, :n]
    low2 = sorted(np.argsort(acc, kind="stable")[:2].tolist())
    assert list(r["evict_idx"][0, 0]) == sorted(low2 + [9, 10, 11])
    assert r["n_valid"] == C
