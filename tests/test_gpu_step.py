"""The single-call step h2o_step against the four calls and the oracle.

For one-token chunks on the few-row path (at most 32 query heads per KV head)
h2o_step runs the split merge, the summed weights, the score update, the
choice and the scatter as one kernel; every other shape runs the four calls'
kernels in order.  Either way its results must equal the four separate calls
bit for bit, and the oracle's at the parity tolerances."""
import numpy as np
import pytest
import torch

import synth
from synth import WORKLOADS

from h2o_harness import (HostState, compare, gpu_step, gpu_step_fused, log, oracle_step,
                         shape_of, state_from_synth)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import h2o_kv_cache_amd as h2o
    h2o.load_library()


def _same(a, b, label):
    for k in a:
        if k == "scores_acc":
            continue
        assert np.array_equal(a[k], b[k], equal_nan=True), (label, k)


# name, B, Hq, Hkv, D, C, S, steps, heavy, prefilled
CASES = [
    ("decode_g4", 3, 32, 8, 128, 4096, 1, 6, 0.05, True),
    ("decode_fill", 2, 8, 2, 128, 300, 1, 6, 0.05, False),
    ("decode_g32", 1, 32, 1, 128, 2000, 1, 5, 0.05, True),
    ("decode_d64_g3", 2, 6, 2, 64, 777, 1, 5, 0.05, True),
    ("chunk_s48", 1, 8, 2, 128, 512, 48, 4, 0.05, False),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,C,S,steps,heavy,prefilled", CASES)
def test_step_equals_four_calls_and_oracle(name, B, Hq, Hkv, D, C, S, steps, heavy, prefilled):
    wl = synth.Workload(name, 200 + [c[0] for c in CASES].index(name), B, Hq, Hkv, D, C, S,
                        S * steps, 1, 1.0, heavy, 4.0, prefilled)
    st = state_from_synth(synth.prefilled_state(wl) if prefilled else synth.empty_state(wl))
    if not prefilled:   # start close to full so that the run reaches eviction steps
        for step in range(max(0, C // S - 2)):
            ch = synth.gen_chunk(wl, 0, step)
            r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
            st = HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                           synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                           r["scores"].astype(np.float32), r["pos"].copy(), r["n_valid"])
        first = max(0, C // S - 2)
    else:
        first = 0
    shape = shape_of(B, Hq, Hkv, D, C, S, st.n_valid)
    for step in range(first, first + steps):
        ch = synth.gen_chunk(wl, 0, step)
        log(f"[step] {name} step {step} n={st.n_valid}")
        g4 = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        g1 = gpu_step_fused(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        _same(g1, g4, f"{name}:{step}")
        r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        s = compare(g4, r, st, ch.k_bits, ch.v_bits, ch.p0, f"{name}:{step}")
        log(f"[step] {name} step {step} {s}")
        st = HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                       synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                       r["scores"].astype(np.float32), r["pos"].copy(), r["n_valid"])


def test_step_decode_full_size():
    # the decode workload's own shape: 16 sequences x 8 KV heads x 16384 slots
    wl = WORKLOADS["decode"]
    st = state_from_synth(synth.prefilled_state(wl))
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st.n_valid)
    for step in range(2):
        ch = synth.gen_chunk(wl, 0, step)
        log(f"[step] decode full size step {step}")
        g4 = gpu_step(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        g1 = gpu_step_fused(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        _same(g1, g4, f"decode:{step}")
        r = oracle_step(st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0)
        compare(g1 | {"scores_acc": g4["scores_acc"]}, r, st, ch.k_bits, ch.v_bits, ch.p0,
                f"decode:{step}")
        st = HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                       synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                       r["scores"].astype(np.float32), r["pos"].copy(), r["n_valid"])


def test_step_exact_ties_and_special_scores():
    """K = 0 and scores 0: all slots tie and the lowest slot goes; then
    special score values (NaN ranks above +inf, -0.0 == +0.0)."""
    B, Hq, Hkv, D, C = 2, 4, 2, 128, 96
    rng = np.random.default_rng(31)
    st = HostState(np.zeros((B, Hkv, C, D), np.uint16),
                   synth.to_bf16(rng.standard_normal((B, Hkv, C, D)).astype(np.float32))[0],
                   np.zeros((B, Hkv, C), np.float32),
                   np.broadcast_to(np.arange(C), (B, Hkv, C)).astype(np.int64).copy(), C)
    shape = shape_of(B, Hq, Hkv, D, C, 1, C)
    for step in range(3):
        q = synth.to_bf16(rng.standard_normal((B, Hq, 1, D)).astype(np.float32))[0]
        kn = np.zeros((B, Hkv, 1, D), np.uint16)
        vn = synth.to_bf16(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))[0]
        g1 = gpu_step_fused(shape, st, q, kn, vn, C + step)
        assert np.all(g1["evict_idx"] == 0), g1["evict_idx"]
        g4 = gpu_step(shape, st, q, kn, vn, C + step)
        _same(g1, g4, f"tie:{step}")
        r = oracle_step(st, q, kn, vn, C + step)
        st = HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                       synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                       r["scores"].astype(np.float32), r["pos"].copy(), r["n_valid"])
    # special values: the minimum is -inf at slot 40 (-0.0 / +0.0 elsewhere,
    # NaN never chosen)
    sc = np.zeros((B, Hkv, C), np.float32)
    sc[:, :, ::3] = -0.0
    sc[:, :, 5] = np.nan
    sc[:, :, 7] = np.inf
    sc[:, :, 40] = -np.inf
    st.scores = sc
    q = synth.to_bf16(rng.standard_normal((B, Hq, 1, D)).astype(np.float32))[0]
    kn = synth.to_bf16(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))[0]
    vn = synth.to_bf16(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))[0]
    g1 = gpu_step_fused(shape, st, q, kn, vn, 500)
    g4 = gpu_step(shape, st, q, kn, vn, 500)
    _same(g1, g4, "special")
    assert np.all(g1["evict_idx"] == 40)
