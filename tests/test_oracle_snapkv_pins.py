"""Pins of the oracle's SnapKV-style one-shot choice and compaction against
things other than their own code: brute force over subsets, a hand-ordered
case with special values, the eviction choice at a full cache, the uniform-
attention closed form, and attention over the compacted cache against
attention over the original keys with an explicit keep-mask.  CPU only."""
import itertools
import math

import numpy as np
import pytest

import oracle


def test_keep_is_the_max_weight_subset_brute_force():
    # distinct weights: the kept set is the unique subset of `budget` slots
    # with the largest total weight
    rng = np.random.default_rng(11)
    for n in (1, 4, 7, 9):
        w = rng.permutation(np.linspace(0.1, 3.0, n))
        wsum = np.zeros((1, 1, n + 3))
        wsum[0, 0, :n] = w
        for budget in range(n + 1):
            best = max(itertools.combinations(range(n), budget),
                       key=lambda c: sum(w[j] for j in c))
            got = oracle.snapkv_keep(wsum, n, budget)[0, 0]
            assert got.tolist() == sorted(best), (n, budget)


def test_keep_hand_ordered_special_values():
    # ascending (weight, slot): (-0.0, 2) (0.0, 3) (1, 1) (1, 5) (inf, 4) (nan, 0)
    w = np.array([np.nan, 1.0, -0.0, 0.0, np.inf, 1.0, 7.0, 7.0])   # slots 6, 7 empty
    wsum = w.reshape(1, 1, -1)
    assert oracle.snapkv_keep(wsum, 6, 3)[0, 0].tolist() == [0, 4, 5]
    assert oracle.snapkv_keep(wsum, 6, 4)[0, 0].tolist() == [0, 1, 4, 5]
    assert oracle.snapkv_keep(wsum, 6, 1)[0, 0].tolist() == [0]
    assert oracle.snapkv_keep(wsum, 6, 0).shape == (1, 1, 0)
    assert oracle.snapkv_keep(wsum, 6, 6)[0, 0].tolist() == list(range(6))


def test_keep_all_but_argmin_and_equal_weights():
    rng = np.random.default_rng(12)
    wsum = rng.random((2, 3, 40)).astype(np.float32)
    wsum[1, 2, 5] = wsum[1, 2, 9] = -1.0           # tie at the minimum: slot 5 drops
    keep = oracle.snapkv_keep(wsum, 30, 29)
    for b in range(2):
        for h in range(3):
            drop = int(np.argmin(wsum[b, h, :30]))   # first occurrence
            assert keep[b, h].tolist() == [j for j in range(30) if j != drop]
    flat = np.full((1, 1, 20), 0.25)
    assert oracle.snapkv_keep(flat, 16, 5)[0, 0].tolist() == [11, 12, 13, 14, 15]


def test_keep_is_the_complement_of_eviction_at_a_full_cache():
    rng = np.random.default_rng(13)
    B, Hkv, n, S = 2, 2, 50, 8
    wsum = np.round(rng.random((B, Hkv, n + S)) * 8) / 8      # many ties
    for budget in (0, 1, 17, 49, 50):
        keep = oracle.snapkv_keep(wsum, n, budget)
        if budget == n:
            assert (keep == np.arange(n)).all()
            continue
        ev = oracle.evict_select(wsum[:, :, :n].copy(), n, n - budget)
        for b in range(B):
            for h in range(Hkv):
                assert keep[b, h].tolist() == sorted(set(range(n)) - set(ev[b, h].tolist()))


def test_uniform_attention_keeps_the_most_recent_slots():
    # K == 0: attention is uniform, every cache slot gets the same summed
    # weight G * (H(n+S) - H(n)), so the ties drop the oldest slots
    B, Hq, Hkv, D, C, S, n = 1, 4, 2, 8, 40, 6, 30
    rng = np.random.default_rng(14)
    q = rng.standard_normal((B, Hq, S, D))
    z = np.zeros((B, Hkv, C, D))
    v = rng.standard_normal((B, Hkv, C, D))
    kn = np.zeros((B, Hkv, S, D))
    vn = rng.standard_normal((B, Hkv, S, D))
    _, _, wsum = oracle.attention_chunk(q, z, v, kn, vn, n)
    G = Hq // Hkv
    H = lambda x: sum(1.0 / k for k in range(1, x + 1))
    np.testing.assert_allclose(wsum[:, :, :n], G * (H(n + S) - H(n)), rtol=1e-12)
    # exact ties in float64 are not guaranteed; quantise like a reduction tree
    # that gives every slot the same bits
    w = np.broadcast_to(wsum[:, :, :1], wsum[:, :, :n].shape).copy()
    full = np.concatenate([w, np.zeros((B, Hkv, C - n)), wsum[:, :, C:]], axis=2)
    keep = oracle.snapkv_keep(full, n, 12)
    assert (keep == np.arange(n - 12, n)).all()


def _masked_attention(q, keys, vals, visible, tau):
    s = tau * (q @ keys.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vals


@pytest.mark.parametrize("budget", [0, 9, 25])
def test_compacted_cache_attends_like_the_kept_keys(budget):
    # one more chunk attending over the compacted cache must equal attention
    # over the original cache + window with an explicit keep-mask
    B, Hq, Hkv, D, C, S, n, S2 = 1, 4, 2, 16, 32, 5, 25, 3
    rng = np.random.default_rng(15 + budget)
    f = lambda *s: rng.standard_normal(s)
    kc, vc, kn, vn = f(B, Hkv, C, D), f(B, Hkv, C, D), f(B, Hkv, S, D), f(B, Hkv, S, D)
    pos = np.full((B, Hkv, C), -1, np.int64)
    pos[:, :, :n] = np.arange(n)
    q = f(B, Hq, S, D)
    _, _, wsum = oracle.attention_chunk(q, kc, vc, kn, vn, n)
    keep = oracle.snapkv_keep(wsum, n, budget)
    out_len = budget + S + 4
    ko, vo, po, so = oracle.snapkv_compact(kc, vc, pos, kn, vn, wsum, keep, out_len, p0=n)
    # positions: kept slots in increasing order, then the window, then empty
    for h in range(Hkv):
        kept_pos = po[0, h, :budget]
        assert (np.diff(kept_pos) > 0).all() and set(kept_pos) <= set(range(n))
        assert po[0, h, budget:budget + S].tolist() == list(range(n, n + S))
        assert (po[0, h, budget + S:] == -1).all()
    # summed weights travel with their rows
    np.testing.assert_array_equal(so[0, :, budget:budget + S], wsum[0, :, C:])
    q2, k2, v2 = f(B, Hq, S2, D), f(B, Hkv, S2, D), f(B, Hkv, S2, D)
    got, _, _ = oracle.attention_chunk(q2, ko, vo, k2, v2, budget + S)
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(D)
    for a in range(Hq):
        h = a // G
        kept = set(int(j) for j in keep[0, h])
        keys = np.concatenate([kc[0, h, :n], kn[0, h], k2[0, h]])
        vals = np.concatenate([vc[0, h, :n], vn[0, h], v2[0, h]])
        vis = np.zeros((S2, n + S + S2), bool)
        vis[:, [j for j in range(n) if j in kept]] = True
        vis[:, n:n + S] = True
        vis[:, n + S:] = np.tril(np.ones((S2, S2), bool))
        want = _masked_attention(q2[0, a], keys, vals, vis, tau)
        np.testing.assert_allclose(got[0, a], want, rtol=1e-12, atol=1e-12)


def test_compacted_rows_scores_and_positions_brute_force():
    # the compacted cache written out by hand from a keep mask: the kept slots
    # in slot order with their K, V, position and summed weight, then the
    # window rows with their own columns; distinct weights per slot and head,
    # so an index slip between slot and output row shows
    rng = np.random.default_rng(16)
    B, Hkv, C, D, S, n, budget, out_len = 2, 3, 20, 4, 3, 17, 6, 12
    kc, vc = rng.standard_normal((B, Hkv, C, D)), rng.standard_normal((B, Hkv, C, D))
    kn, vn = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    pos = rng.permutation(1000)[:B * Hkv * C].reshape(B, Hkv, C).astype(np.int64)
    wsum = rng.permutation(B * Hkv * (C + S)).reshape(B, Hkv, C + S) * 0.5 + 0.125
    keep = oracle.snapkv_keep(wsum, n, budget)
    ko, vo, po, so = oracle.snapkv_compact(kc, vc, pos, kn, vn, wsum, keep, out_len, p0=500)
    for b in range(B):
        for h in range(Hkv):
            # mask: the budget largest weights among the n valid slots
            mask = np.zeros(C, bool)
            mask[np.argsort(-wsum[b, h, :n])[:budget]] = True
            rows = [j for j in range(C) if mask[j]]
            assert len(rows) == budget
            for i, j in enumerate(rows):
                np.testing.assert_array_equal(ko[b, h, i], kc[b, h, j])
                np.testing.assert_array_equal(vo[b, h, i], vc[b, h, j])
                assert po[b, h, i] == pos[b, h, j]
                assert so[b, h, i] == wsum[b, h, j]
            for t in range(S):
                i = budget + t
                np.testing.assert_array_equal(ko[b, h, i], kn[b, h, t])
                np.testing.assert_array_equal(vo[b, h, i], vn[b, h, t])
                assert po[b, h, i] == 500 + t
                assert so[b, h, i] == wsum[b, h, C + t]
            tail = slice(budget + S, out_len)
            assert (ko[b, h, tail] == 0).all() and (vo[b, h, tail] == 0).all()
            assert (po[b, h, tail] == -1).all() and (so[b, h, tail] == 0).all()
