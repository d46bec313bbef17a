"""GPU parity of the HIP path against the CPU oracle, step by step, with the
oracle's cache state fed in before every step (no compounding of float
differences).  Every call goes through the C ABI of libh2o.so."""
import numpy as np
import pytest
import torch

import synth
from synth import WORKLOADS

from h2o_harness import (HostState, compare, gpu_step, log, oracle_step, select_heads,
                         shape_of, state_from_synth)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import h2o_kv_cache_amd as h2o
    h2o.load_library()


def _state_from_oracle(r) -> HostState:
    return HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                     synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                     r["scores"].astype(np.float32), r["pos"].copy(), r["n_valid"])


def _trajectory(wl, steps, layer=0, every=1):
    """Run ``steps`` chunk steps from an empty cache; the oracle's state is fed
    to the GPU before each compared step."""
    st = state_from_synth(synth.empty_state(wl) if not wl.prefilled
                          else synth.prefilled_state(wl, layer))
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st.n_valid)
    worst = {}
    for step in range(steps):
        ch = synth.gen_chunk(wl, layer, step)
        r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        if step % every == 0:
            log(f"[parity] {wl.name} layer {layer} step {step} n={st.n_valid}")
            g = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
            s = compare(g, r, st, ch.k_bits, ch.v_bits, ch.p0, f"{wl.name}:{step}")
            for k, v in s.items():
                worst[k] = max(worst.get(k, 0), v)
        st = _state_from_oracle(r)
    log(f"[parity] {wl.name} worst {worst}")
    return worst


def test_tiny_full_run():
    _trajectory(WORKLOADS["tiny"], WORKLOADS["tiny"].steps)


def test_small_gqa_full_run():
    _trajectory(WORKLOADS["small_gqa"], WORKLOADS["small_gqa"].steps)


def _steady(wl, heads, step=None, layer=0, n_valid=None):
    if n_valid is None:
        st = state_from_synth(synth.steady_state(wl, layer, step))
    else:                     # a partly filled cache
        st = state_from_synth(synth.partial_state(wl, n_valid, layer))
    step = step if step is not None else wl.fill_steps + 2
    ch = synth.gen_chunk(wl, layer, step)
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st.n_valid)
    log(f"[parity] {wl.name} steady step {step} n={st.n_valid} heads={heads}")
    g = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
    r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0, heads=heads)
    G = wl.group
    gs = select_heads(g, wl.n_kv_heads, G, heads)
    sub = HostState(st.k_bits[:, heads], st.v_bits[:, heads], st.scores[:, heads],
                    st.pos[:, heads], st.n_valid)
    s = compare(gs, r, sub, ch.k_bits[:, heads], ch.v_bits[:, heads], ch.p0,
                f"{wl.name}:steady")
    log(f"[parity] {wl.name} stats {s}")
    return s


def test_qwen3_64k_steady_step():
    _steady(WORKLOADS["qwen3_4b_64k"], heads=[0, 5])


def test_qwen3_128k_steady_step():
    _steady(WORKLOADS["qwen3_4b_128k"], heads=[2, 7], layer=3)


def test_qwen3_128k_one_head_share_steady_step():
    # one KV head: 16 row-tile workgroups, so pass 1 runs 16 key splits
    _steady(WORKLOADS["qwen3_4b_128k_head"], heads=[0], layer=1)


def test_qwen3_128k_fill_step():
    wl = WORKLOADS["qwen3_4b_128k"]
    _steady(wl, heads=[1], step=9, n_valid=9 * wl.chunk_len)


def test_qwen3_64k_small_chunk_steady_steps():
    wl = WORKLOADS["qwen3_4b_64k_s128"]
    for step in (wl.fill_steps + 2, wl.fill_steps + 301):
        _steady(wl, heads=[3, 6], step=step, layer=5)


def test_qwen3_64k_small_chunk_fill_step():
    wl = WORKLOADS["qwen3_4b_64k_s128"]
    _steady(wl, heads=[0], step=17, n_valid=17 * wl.chunk_len)


@pytest.mark.parametrize("name", ["qwen3_4b_64k_s256", "qwen3_4b_64k_s512"])
def test_qwen3_64k_mid_chunk_steady_step(name):
    wl = WORKLOADS[name]
    _steady(wl, heads=[1, 4], step=wl.fill_steps + 5, layer=2)


def test_qwen3_64k_s512_fill_step():
    wl = WORKLOADS["qwen3_4b_64k_s512"]
    _steady(wl, heads=[6], step=7, n_valid=7 * wl.chunk_len)


def test_decode_steps():
    wl = WORKLOADS["decode"]
    st = state_from_synth(synth.prefilled_state(wl))
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st.n_valid)
    for step in range(4):
        ch = synth.gen_chunk(wl, 0, step)
        log(f"[parity] decode step {step}")
        g = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        s = compare(g, r, st, ch.k_bits, ch.v_bits, ch.p0, f"decode:{step}")
        log(f"[parity] decode stats {s}")
        st = _state_from_oracle(r)


# --------------------------------------------------------------------------
# edge cases at small sizes: ragged tiles, head_dim 64, G = 1 / 3, S = C,
# S = 1, partial overflow, batch > 1, garbage in empty slots
# --------------------------------------------------------------------------
EDGE = [
    # name, B, Hq, Hkv, D, C, S, steps, std, heavy
    ("d64_g1_ragged", 1, 2, 2, 64, 100, 7, 20, 1.0, 0.0),
    ("g3_ragged", 2, 6, 2, 128, 200, 50, 8, 1.0, 0.05),
    ("s_eq_c", 1, 4, 1, 128, 64, 64, 4, 1.0, 0.0),
    ("s1_from_empty", 3, 8, 2, 128, 50, 1, 60, 1.0, 0.05),
    ("one_row_tile_tail", 1, 4, 1, 64, 300, 33, 12, 2.0, 0.1),
    ("big_group", 1, 16, 1, 128, 512, 40, 16, 1.0, 0.05),
    # few query rows per KV head (G * S <= 32): the logits path
    ("few_rows_causal", 2, 12, 3, 128, 300, 8, 40, 1.0, 0.05),
    ("few_rows_ragged", 1, 6, 2, 64, 97, 5, 25, 1.0, 0.05),
    # the 16-row kernel at its limit (R = 16) and the 32-row one just above it
    ("rows_16_decode", 2, 16, 1, 128, 230, 1, 40, 1.0, 0.05),
    ("rows_17_g1", 1, 1, 1, 64, 150, 17, 12, 1.0, 0.05),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,C,S,steps,std,heavy", EDGE)
def test_edge_trajectories(name, B, Hq, Hkv, D, C, S, steps, std, heavy):
    wl = synth.Workload(name, 100 + EDGE.index(next(e for e in EDGE if e[0] == name)), B, Hq,
                        Hkv, D, C, S, S * steps, 1, std, heavy, 4.0, False)
    _trajectory(wl, steps)


def test_partial_overflow_and_garbage_slots():
    """n + S > C with free slots left, and NaN bit patterns in empty slots."""
    wl = synth.Workload("overflow", 120, 1, 4, 2, 128, 160, 48, 48 * 4, 1, 1.0, 0.05, 4.0, False)
    st = state_from_synth(synth.empty_state(wl))
    for step in range(3):          # fill 144 of 160 slots through the oracle
        ch = synth.gen_chunk(wl, 0, step)
        st = _state_from_oracle(oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0))
    assert st.n_valid == 144
    st.k_bits[..., 144:, :] = 0x7FC1      # NaN
    st.v_bits[..., 144:, :] = 0xFF80      # -inf
    st.scores[..., 144:] = np.nan
    ch = synth.gen_chunk(wl, 0, 3)
    shape = shape_of(1, 4, 2, 128, 160, 48, st.n_valid)
    g = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
    r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
    compare(g, r, st, ch.k_bits, ch.v_bits, ch.p0, "overflow")
    assert set(range(144, 160)).issubset(set(g["evict_idx"][0, 0].tolist()))


# name, B, Hq, Hkv, D, C, S, heavy cache slot, heavy chunk column
WIDE = [
    ("wide_row_tiles", 1, 4, 1, 128, 1024, 128, 700, 90),
    ("wide_few_rows", 2, 8, 2, 128, 512, 1, 300, 0),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,C,S,slot,col", WIDE)
def test_wide_logit_spread(name, B, Hq, Hkv, D, C, S, slot, col):
    """All-positive queries against one cache slot (and one chunk key) of
    constant 8.0: their logits exceed every row's first-tile maximum by about
    130 in base 2, so weights against that reference would overflow fp32 and
    pass 1 has to redo the rows against their exact maxima."""
    wl = synth.Workload(name, 130 + [w[0] for w in WIDE].index(name), B, Hq, Hkv, D, C, S,
                        4 * S, 1, 1.0, 0.0, 1.0, False)
    step = C // S + 1
    st = state_from_synth(synth.steady_state(wl, 0, step))
    ch = synth.gen_chunk(wl, 0, step)
    q = synth.to_bf16(np.abs(synth.bf16_bits_to_f32(ch.q_bits)) + np.float32(0.25))[0]
    big = synth.to_bf16(np.full(D, 8.0, np.float32))[0]
    st.k_bits[:, :, slot, :] = big
    kn = ch.k_bits.copy()
    kn[:, :, col, :] = big
    shape = shape_of(B, Hq, Hkv, D, C, S, st.n_valid)
    log(f"[parity] {name} heavy slot {slot} chunk column {col}")
    g = gpu_step(shape, st, q, kn, ch.v_bits, ch.p0)
    r = oracle_step(st, q, kn, ch.v_bits, ch.p0)
    s = compare(g, r, st, kn, ch.v_bits, ch.p0, name)
    log(f"[parity] {name} stats {s}")
    # the heavy keys take nearly all of the weight of the rows that see them
    assert r["wsum"][0, 0, slot] > 0.25 * (Hq // Hkv) * S


def test_exact_tie_trajectory():
    """K = 0, S = 1, scores 0: every slot ties exactly at steps 1 and 2 and
    slot 0 is the minimum afterwards -- slot 0 is evicted every step."""
    B, Hq, Hkv, D, C = 2, 4, 2, 128, 96
    rng = np.random.default_rng(11)
    st = HostState(np.zeros((B, Hkv, C, D), np.uint16),
                   synth.to_bf16(rng.standard_normal((B, Hkv, C, D)).astype(np.float32))[0],
                   np.zeros((B, Hkv, C), np.float32),
                   np.broadcast_to(np.arange(C), (B, Hkv, C)).astype(np.int64).copy(), C)
    shape = shape_of(B, Hq, Hkv, D, C, 1, C)
    for step in range(5):
        q = synth.to_bf16(rng.standard_normal((B, Hq, 1, D)).astype(np.float32))[0]
        kn = np.zeros((B, Hkv, 1, D), np.uint16)
        vn = synth.to_bf16(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))[0]
        g = gpu_step(shape, st, q, kn, vn, C + step)
        assert np.all(g["evict_idx"] == 0), g["evict_idx"]
        r = oracle_step(st, q, kn, vn, C + step)
        compare(g, r, st, kn, vn, C + step, f"tie:{step}")
        st = _state_from_oracle(r)


def test_select_special_scores():
    """Selection on hand-made scores: ties, -0.0 vs +0.0, +-inf, NaN."""
    import h2o_kv_cache_amd as h2o
    import oracle
    rng = np.random.default_rng(12)
    # sizes cover each keys-per-thread run of the kernel (4, 16, 64)
    fixed = [(16384, 1024, 16384), (16384, 1, 16384), (40000, 2048, 40000), (65536, 3000, 65000)]
    for trial in range(30 + len(fixed)):
        if trial < len(fixed):
            C, S, n = fixed[trial]
        else:
            C = int(rng.integers(2, 3000))
            S = int(rng.integers(1, min(C, 700) + 1))
            n = int(rng.integers(max(0, C - S - 3), C + 1))
        B, Hkv = 2, 3
        pool = np.array([0.0, -0.0, 1.0, np.inf, -np.inf, np.nan, 2.5, -1.0, 1e-30, 3.0],
                        np.float32)
        if trial % 2:
            sc = rng.choice(pool, (B, Hkv, C)).astype(np.float32)
        else:
            sc = rng.integers(0, 7, (B, Hkv, C)).astype(np.float32)
        shape = shape_of(B, 2 * Hkv, Hkv, 128, C, S, n)
        scores = torch.from_numpy(sc).cuda()
        ev = torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda")
        h2o.h2o_evict_select(shape, scores, ev)
        torch.cuda.synchronize()
        ref = oracle.evict_select(sc.astype(np.float64), n, S)
        assert np.array_equal(ev.cpu().numpy(), ref), (trial, C, S, n)


def test_repeat_is_bit_identical():
    wl = WORKLOADS["small_gqa"]
    st = state_from_synth(synth.steady_state(wl))
    ch = synth.gen_chunk(wl, 0, 12)
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st.n_valid)
    a, b = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0, runs=2)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
