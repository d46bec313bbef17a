"""GPU parity of the SnapKV-style one-shot choice and compaction, and of the
slot choice on caches longer than the register-resident select handles,
through the C ABI against the oracle.

Bars: the keep list and the eviction list are bit-exact against the oracle on
identical weights (integer work); end to end (attention -> choice ->
compaction) the kept set may differ from the oracle's only in slots whose
oracle weight lies within 1e-6 (relative) of the cut, every compacted row is
bit-identical to the input row the GPU chose, and the scores carried along
match at the summed-weight tolerance (max-abs 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import h2o_kv_cache_amd as h2o
from h2o_harness import TIE_REL, TOL_WSUM, dev_bf16, host_bits, log, shape_of

pytestmark = pytest.mark.gpu


def _weights(rng, B, Hkv, W, special=False):
    """Positive weights with many exact ties; optionally -0.0, +0.0, +inf,
    NaN and negative values planted in every row."""
    w = rng.random((B, Hkv, W), dtype=np.float32) * np.float32(8.0)
    w[..., ::3] = np.round(w[..., ::3] * 4) / 4
    if special:
        for b in range(B):
            for h in range(Hkv):
                idx = rng.choice(W, size=min(W, 12), replace=False)
                vals = [-0.0, 0.0, np.inf, np.nan, -1.5, -np.inf, 0.0, -0.0, np.nan,
                        np.inf, 3.0, 3.0]
                w[b, h, idx] = vals[:len(idx)]
    return w


def _gpu_keep(shape, wsum_np, budget):
    B, Hkv = shape.batch, shape.n_kv_heads
    wsum = torch.from_numpy(wsum_np).cuda()
    keep = (torch.full((B, Hkv, budget), -7, dtype=torch.int32, device="cuda")
            if budget > 0 else None)
    h2o.h2o_snapkv_select(shape, wsum, budget, keep)
    torch.cuda.synchronize()
    return keep.cpu().numpy() if keep is not None else np.zeros((B, Hkv, 0), np.int32)


@pytest.mark.parametrize("B,Hkv,C,S,n,budget,special", [
    (1, 2, 300, 20, 300, 100, False),
    (2, 3, 1000, 64, 777, 0, True),
    (1, 1, 1000, 64, 777, 777, True),
    (1, 2, 5000, 100, 4999, 1, True),
    (1, 2, 5000, 100, 4999, 4998, True),
    (1, 2, 4097, 33, 4097, 2048, True),
    (1, 4, 70000, 512, 70000, 6000, True),
    (1, 8, 130048, 1024, 130048, 15360, False),
])
def test_keep_select_bit_exact(B, Hkv, C, S, n, budget, special):
    log(f"snapkv select B={B} Hkv={Hkv} C={C} S={S} n={n} budget={budget}")
    rng = np.random.default_rng(C + n + budget)
    w = _weights(rng, B, Hkv, C + S, special)
    w[..., n:C] = np.nan                      # empty slots: never read
    shape = shape_of(B, 4 * Hkv, Hkv, 128, C, S, n)
    got = _gpu_keep(shape, w, budget)
    want = oracle.snapkv_keep(w, n, budget)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("C,S,n", [(100000, 512, 100000), (100000, 512, 99800),
                                   (100000, 512, 50000), (70001, 1, 70001)])
def test_evict_select_long_cache_bit_exact(C, S, n):
    # rows longer than 65536 slots take the streaming select
    log(f"evict select long cache C={C} S={S} n={n}")
    rng = np.random.default_rng(C + S + n)
    B, Hkv = 1, 2
    sc = _weights(rng, B, Hkv, C, special=True)
    sc[..., n:] = np.nan                      # empty slots are taken first regardless
    shape = shape_of(B, 8, Hkv, 128, C, S, n)
    ev = torch.full((B, Hkv, S), -7, dtype=torch.int32, device="cuda")
    h2o.h2o_evict_select(shape, torch.from_numpy(sc).cuda(), ev)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ev.cpu().numpy(), oracle.evict_select(sc, n, S))


def _keep_ok(gk, ok, w, n, budget):
    """GPU keep list equals the oracle's, or differs only in slots whose
    oracle weight lies within TIE_REL of the cut."""
    if np.array_equal(gk, ok):
        return True
    if (len(set(gk.tolist())) != budget or list(gk) != sorted(gk) or gk.min() < 0
            or gk.max() >= n):
        return False
    drop = n - budget
    cut = np.sort(w[:n], kind="stable")[drop]   # smallest kept weight
    for j in set(gk.tolist()) ^ set(ok.tolist()):
        if abs(w[j] - cut) > TIE_REL * max(abs(cut), abs(w[j]), 1e-30):
            return False
    return True


def _run_end_to_end(B, Hq, Hkv, D, C, S, n, budget, kc_bits, vc_bits, pos, q_bits, kn_bits,
                    vn_bits, heads=None):
    out_len = budget + S + 8
    p0 = int(pos.max()) + 1 if n > 0 else 0
    shape = shape_of(B, Hq, Hkv, D, C, S, n)
    kc, vc = dev_bf16(kc_bits), dev_bf16(vc_bits)
    q, kn, vn = dev_bf16(q_bits), dev_bf16(kn_bits), dev_bf16(vn_bits)
    pos_d = torch.from_numpy(pos).cuda()
    out = torch.empty((B, Hq, S, D), device="cuda")
    wsum = torch.empty((B, Hkv, C + S), device="cuda")
    ws = torch.empty(max(h2o.h2o_workspace_size(shape), 256), dtype=torch.uint8, device="cuda")
    h2o.h2o_attn_chunk(shape, q, kc, vc, kn, vn, out, None, wsum, ws)
    keep = (torch.full((B, Hkv, budget), -7, dtype=torch.int32, device="cuda")
            if budget > 0 else None)
    h2o.h2o_snapkv_select(shape, wsum, budget, keep)
    ko = torch.full((B, Hkv, out_len, D), 0x3F80, dtype=torch.int16, device="cuda")
    vo = torch.full((B, Hkv, out_len, D), 0x3F80, dtype=torch.int16, device="cuda")
    po = torch.full((B, Hkv, out_len), -9, dtype=torch.int64, device="cuda")
    so = torch.full((B, Hkv, out_len), -9.0, device="cuda")
    h2o.h2o_snapkv_compact(shape, kc, vc, pos_d, kn, vn, wsum, keep, budget, out_len, p0,
                           ko, vo, po, so)
    torch.cuda.synchronize()
    g = dict(wsum=wsum.cpu().numpy(),
             keep=keep.cpu().numpy() if keep is not None else np.zeros((B, Hkv, 0), np.int32),
             ko=host_bits(ko), vo=host_bits(vo), po=po.cpu().numpy(), so=so.cpu().numpy())

    # oracle (float64) on the same bf16 inputs, optionally on a subset of KV heads
    heads = list(range(Hkv)) if heads is None else heads
    G = Hq // Hkv
    qh = [h * G + x for h in heads for x in range(G)]
    f = synth.bf16_bits_to_f32
    _, _, w_o = oracle.attention_chunk(f(q_bits)[:, qh], f(kc_bits)[:, heads],
                                       f(vc_bits)[:, heads], f(kn_bits)[:, heads],
                                       f(vn_bits)[:, heads], n)
    keep_o = oracle.snapkv_keep(w_o, n, budget)
    swapped = 0
    for bi in range(B):
        for hi, h in enumerate(heads):
            wg, wo = g["wsum"][bi, h], w_o[bi, hi]
            err = max(np.abs(wg[:n] - wo[:n]).max(initial=0.0),
                      np.abs(wg[C:] - wo[C:]).max())
            assert err <= TOL_WSUM, (bi, h, err)
            gk, ok = g["keep"][bi, h], keep_o[bi, hi]
            assert _keep_ok(gk, ok, wo, n, budget), (bi, h)
            swapped += len(set(gk.tolist()) ^ set(ok.tolist())) // 2
            # compacted rows: the GPU's chosen input rows, then the window
            rows_k = np.concatenate([kc_bits[bi, h][gk], kn_bits[bi, h]])
            rows_v = np.concatenate([vc_bits[bi, h][gk], vn_bits[bi, h]])
            np.testing.assert_array_equal(g["ko"][bi, h, :budget + S], rows_k)
            np.testing.assert_array_equal(g["vo"][bi, h, :budget + S], rows_v)
            want_pos = np.concatenate([pos[bi, h][gk], p0 + np.arange(S)])
            np.testing.assert_array_equal(g["po"][bi, h, :budget + S], want_pos)
            # scores: the weights of the chosen rows (oracle's, at the wsum bar)
            want_sc = np.concatenate([wo[gk], wo[C:]])
            assert np.abs(g["so"][bi, h, :budget + S] - want_sc).max(initial=0.0) <= TOL_WSUM
            # rows past budget + S are not written
            assert (g["ko"][bi, h, budget + S:] == 0x3F80).all()
            assert (g["po"][bi, h, budget + S:] == -9).all()
    log(f"  end to end ok; slots swapped inside the tie band: {swapped}")


@pytest.mark.parametrize("B,Hq,Hkv,D,C,S,n,budget", [
    (1, 4, 2, 64, 600, 64, 500, 200),
    (2, 6, 2, 128, 1000, 100, 999, 333),
    (1, 4, 1, 128, 256, 32, 256, 0),
    (1, 8, 2, 128, 2048, 256, 2048, 2048),
])
def test_snapkv_end_to_end_small(B, Hq, Hkv, D, C, S, n, budget):
    log(f"snapkv end to end B={B} Hq={Hq} Hkv={Hkv} D={D} C={C} S={S} n={n} budget={budget}")
    rng = np.random.default_rng(C * 7 + budget)

    def bits(*shape, scale=1.0):
        return synth.to_bf16(rng.standard_normal(shape).astype(np.float32) * scale)[0]
    kc, vc = bits(B, Hkv, C, D), bits(B, Hkv, C, D)
    heavy = rng.random((B, Hkv, C)) < 0.05
    kc[heavy] = synth.to_bf16(synth.bf16_bits_to_f32(kc[heavy]) * 4)[0]
    kc[:, :, n:] = 0x7FC0                      # NaN garbage in empty slots
    vc[:, :, n:] = 0x7FC0
    pos = np.full((B, Hkv, C), -1, np.int64)
    pos[:, :, :n] = np.arange(n)
    _run_end_to_end(B, Hq, Hkv, D, C, S, n, budget, kc, vc, pos, bits(B, Hq, S, D),
                    bits(B, Hkv, S, D), bits(B, Hkv, S, D))


def test_snapkv_qwen3_128k_prompt_one_head():
    """The full-size workload (131072-token prompt: 130048 cache slots plus a
    1024-token window, budget 15360), GPU on all 8 KV heads, oracle on one."""
    wl = synth.WORKLOADS["qwen3_4b_128k_snapkv"]
    log("snapkv 128k prompt: generating the prompt cache")
    st = synth.prefilled_state(wl, layer=0)
    ch = synth.gen_chunk(wl, layer=0, step=0)
    assert ch.p0 == wl.cache_len
    _run_end_to_end(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                    wl.chunk_len, wl.cache_len, wl.keep_budget, st.k_bits, st.v_bits, st.pos,
                    ch.q_bits, ch.k_bits, ch.v_bits, heads=[3])
