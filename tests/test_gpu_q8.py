"""GPU parity of the 8-bit KV cache (int8 codes + one fp32 scale per row)
through the C ABI against the oracle.

Bars: quantisation is bit-exact (codes and scales: the same correctly
rounded fp32 divisions on both sides); attention over the int8 cache meets
the bf16 path's tolerances (out and summed weights max-abs 2e-2, log-sum-exp
1e-3) against the float64 oracle on the dequantised rows; a whole step
(attention, accumulate, choice, quantising scatter) keeps the eviction set
bit-exact outside the 1e-6 tie band and writes bit-exact codes and scales.
Cache inputs are quantised on the host by the oracle's quantiser."""
import numpy as np
import pytest
import torch

import oracle
import synth
import h2o_kv_cache_amd as h2o
from h2o_harness import (REL_SCORE, TOL_LSE, TOL_OUT, TOL_WSUM, _evict_ok, dev_bf16, log,
                         shape_of)

pytestmark = pytest.mark.gpu

f32 = synth.bf16_bits_to_f32


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_rows_bit_exact(D):
    log(f"q8 quantize rows D={D}")
    rng = np.random.default_rng(D)
    rows = 3001
    x = rng.standard_normal((rows, D)).astype(np.float32) * rng.uniform(1e-3, 50, (rows, 1))
    x = x.astype(np.float32)
    x[5] = 0.0                                    # zero row
    x[6] = 0.0
    x[6, 3] = -2.0 ** -20                          # one tiny value
    x[7] = np.arange(D) % 5 - 2.0                 # many exact ties after scaling
    x[8, :] = 127.0 * 2.0 ** 7
    x[8, 1:6] = np.array([0.5, 1.5, 2.5, -0.5, -1.5]) * 2.0 ** 7   # exact halves
    bits, vals = synth.to_bf16(x)
    codes = torch.full((rows, D), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((rows,), -1.0, device="cuda")
    h2o.h2o_quantize_rows_q8(dev_bf16(bits), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = oracle.quantize_rows_int8(vals)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)


def _q8_inputs(rng, B, Hq, Hkv, D, C, S, n, heavy=True, garbage=True):
    def bits(*shape):
        return synth.to_bf16(rng.standard_normal(shape).astype(np.float32))[0]
    kc, vc = bits(B, Hkv, C, D), bits(B, Hkv, C, D)
    if heavy:
        hv = rng.random((B, Hkv, C)) < 0.05
        kc[hv] = synth.to_bf16(f32(kc[hv]) * 4)[0]
    kq, ks = oracle.quantize_rows_int8(f32(kc))
    vq, vs = oracle.quantize_rows_int8(f32(vc))
    if garbage:   # empty slots: arbitrary codes, NaN scales; never read
        kq[:, :, n:] = 77
        vq[:, :, n:] = -99
        ks[:, :, n:] = np.nan
        vs[:, :, n:] = np.nan
    return kq, ks, vq, vs, bits(B, Hq, S, D), bits(B, Hkv, S, D), bits(B, Hkv, S, D)


def _gpu_attn_q8(shape, kq, ks, vq, vs, qb, knb, vnb):
    B, Hq, Hkv, D, C, S = (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.cache_len, shape.chunk_len)
    out = torch.full((B, Hq, S, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    wsum = torch.full((B, Hkv, C + S), float("nan"), device="cuda")
    ws = torch.full((max(h2o.h2o_workspace_size(shape), 256),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    h2o.h2o_attn_chunk_q8(shape, dev_bf16(qb), _dev(kq), _dev(ks), _dev(vq), _dev(vs),
                          dev_bf16(knb), dev_bf16(vnb), out, lse, wsum, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), wsum.cpu().numpy()


def _check_attn(g, r, n, C, label):
    e_out = float(np.abs(g[0] - r[0]).max())
    e_lse = float(np.abs(g[1] - r[1]).max())
    e_w = float(np.abs(g[2] - r[2]).max())
    log(f"  {label}: out {e_out:.2e} lse {e_lse:.2e} wsum {e_w:.2e}")
    assert np.isfinite(g[0]).all() and np.isfinite(g[2]).all(), label
    assert e_out <= TOL_OUT and e_lse <= TOL_LSE and e_w <= TOL_WSUM, (label, e_out, e_lse, e_w)
    assert (g[2][..., n:C] == 0).all(), label


ATTN = [
    # name,            B, Hq, Hkv, D,   C,    S,   n
    ("ragged_rows",    1, 8,  2,   128, 300,  100, 250),
    ("head_dim_64",    2, 6,  2,   64,  200,  70,  200),
    ("empty_cache",    1, 4,  1,   128, 128,  64,  0),
    ("decode",         2, 8,  2,   128, 1000, 1,   1000),
    ("few_rows_chunk", 1, 8,  2,   128, 700,  8,   650),
    ("few_rows_d64",   1, 3,  3,   64,  257,  20,  257),
    ("g16_multi_tile", 1, 16, 1,   128, 520,  40,  333),
    # at most 16 rows (G * S): the 16-row kernel
    ("rows_16",        1, 4,  1,   128, 700,  4,   650),
    ("rows_15_d64",    2, 6,  2,   64,  333,  5,   300),
    ("rows_16_g16",    1, 16, 1,   128, 200,  1,   130),
    ("rows_8_empty",   1, 8,  2,   128, 64,   2,   0),
    ("rows_1",         1, 1,  1,   128, 100,  1,   100),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,C,S,n", ATTN)
def test_attention_q8_small(name, B, Hq, Hkv, D, C, S, n):
    log(f"q8 attention {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} C={C} S={S} n={n}")
    rng = np.random.default_rng(C + S + n + D)
    kq, ks, vq, vs, qb, knb, vnb = _q8_inputs(rng, B, Hq, Hkv, D, C, S, n)
    g = _gpu_attn_q8(shape_of(B, Hq, Hkv, D, C, S, n), kq, ks, vq, vs, qb, knb, vnb)
    r = oracle.attention_chunk_q8(f32(qb), kq, ks, vq, vs, f32(knb), f32(vnb), n)
    _check_attn(g, r, n, C, name)


@pytest.mark.parametrize("B,Hq,Hkv,D,C,S,n,slot,col", [
    (1, 4, 1, 128, 1024, 128, 1024, 700, 90),    # row-tile kernel
    (2, 8, 2, 128, 1000, 1, 1000, 300, -1),      # few-row (decode) kernel; the one
    (1, 4, 1, 64, 600, 2, 600, 100, -1),         # chunk key (each row's own) stays plain
])
def test_attention_q8_wide_logit_spread(B, Hq, Hkv, D, C, S, n, slot, col):
    """All-positive queries against one cache slot and one chunk key of
    constant 8.0 (int8 codes 127, scale 8/127): their base-2 logits exceed
    every row's own diagonal logit, and the first-tile maximum, by more than
    100, so pass 1 has to take its fallback sweeps and end with the exact
    row maxima."""
    log(f"q8 attention wide logit spread: C={C} S={S} heavy slot {slot} chunk column {col}")
    rng = np.random.default_rng(1301 + S)
    kq, ks, vq, vs, qb, knb, vnb = _q8_inputs(rng, B, Hq, Hkv, D, C, S, n, heavy=False,
                                             garbage=False)
    qb = synth.to_bf16(np.abs(f32(qb)) + np.float32(0.25))[0]
    big = np.full((1, D), 8.0, np.float32)
    bq, bs = oracle.quantize_rows_int8(big)
    kq[:, :, slot] = bq[0]
    ks[:, :, slot] = bs[0]
    if col >= 0:
        knb[:, :, col] = synth.to_bf16(big[0])[0]
    g = _gpu_attn_q8(shape_of(B, Hq, Hkv, D, C, S, n), kq, ks, vq, vs, qb, knb, vnb)
    r = oracle.attention_chunk_q8(f32(qb), kq, ks, vq, vs, f32(knb), f32(vnb), n)
    _check_attn(g, r, n, C, "wide_spread")
    # the heavy slot takes nearly all of the weight of every row
    assert r[2][0, 0, slot] > 0.25 * (Hq // Hkv) * S


def _gpu_step_q8(shape, kq, ks, vq, vs, scores, pos, qb, knb, vnb, p0):
    B, Hq, Hkv, D, C, S = (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.cache_len, shape.chunk_len)
    dk, dks, dv, dvs = _dev(kq), _dev(ks), _dev(vq), _dev(vs)
    dsc, dpos = _dev(scores.astype(np.float32)), _dev(pos)
    q, kn, vn = dev_bf16(qb), dev_bf16(knb), dev_bf16(vnb)
    out = torch.empty((B, Hq, S, D), device="cuda")
    lse = torch.empty((B, Hq, S), device="cuda")
    wsum = torch.empty((B, Hkv, C + S), device="cuda")
    new = torch.empty((B, Hkv, S), device="cuda")
    ev = torch.full((B, Hkv, S), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(h2o.h2o_workspace_size(shape), 256), dtype=torch.uint8, device="cuda")
    h2o.h2o_attn_chunk_q8(shape, q, dk, dks, dv, dvs, kn, vn, out, lse, wsum, ws)
    h2o.h2o_score_accumulate(shape, dsc, new, wsum)
    acc = dsc.clone()
    h2o.h2o_evict_select(shape, dsc, ev)
    h2o.kv_scatter_q8(shape, dk, dks, dv, dvs, dsc, dpos, kn, vn, new, ev, p0)
    torch.cuda.synchronize()
    c = lambda t: t.cpu().numpy()
    return dict(out=c(out), lse=c(lse), wsum=c(wsum), scores_acc=c(acc), evict_idx=c(ev),
                kq=c(dk), k_scale=c(dks), vq=c(dv), v_scale=c(dvs), scores=c(dsc), pos=c(dpos))


def _step_and_compare(shape, st, qb, knb, vnb, p0, heads=None, label=""):
    """st: dict kq, k_scale, vq, v_scale, scores, pos, n.  GPU on all heads,
    oracle on `heads` (all if None)."""
    n = st["n"]
    sh = shape.with_n(n)
    g = _gpu_step_q8(sh, st["kq"], st["k_scale"], st["vq"], st["v_scale"], st["scores"],
                     st["pos"], qb, knb, vnb, p0)
    Hkv = shape.n_kv_heads
    G = shape.n_q_heads // Hkv
    heads = list(range(Hkv)) if heads is None else heads
    qh = [h * G + x for h in heads for x in range(G)]
    sel = lambda a: a[:, heads]
    r = oracle.h2o_step_q8(sel(st["kq"]), sel(st["k_scale"]), sel(st["vq"]), sel(st["v_scale"]),
                           sel(st["scores"]).astype(np.float64), sel(st["pos"]), n,
                           f32(qb)[:, qh], f32(sel(knb)), f32(sel(vnb)), p0)
    _check_attn((g["out"][:, qh], g["lse"][:, qh], g["wsum"][:, heads]),
                (r["out"], r["lse"], r["wsum"]), n, shape.cache_len, label)
    C, S = shape.cache_len, shape.chunk_len
    acc_r = r["scores_acc"]
    acc_g = g["scores_acc"][:, heads]
    rel = np.abs(acc_g[..., :n] - acc_r[..., :n]) / np.maximum(np.abs(acc_r[..., :n]), 1e-6)
    assert (rel <= REL_SCORE).all(), label
    # quantised chunk rows, as the oracle quantises them
    ck, sk = oracle.quantize_rows_int8(f32(knb))
    cv, sv = oracle.quantize_rows_int8(f32(vnb))
    swaps = 0
    for b in range(shape.batch):
        for hi, h in enumerate(heads):
            ge = g["evict_idx"][b, h].astype(np.int64)
            ok, same = _evict_ok(ge, r["evict_idx"][b, hi], acc_r[b, hi], n, C, S)
            assert ok, (label, "evict", b, h)
            swaps += 0 if same else 1
            if same:
                np.testing.assert_array_equal(g["kq"][b, h], r["kq"][b, hi])
                np.testing.assert_array_equal(g["vq"][b, h], r["vq"][b, hi])
                np.testing.assert_array_equal(g["k_scale"][b, h], r["k_scale"][b, hi])
                np.testing.assert_array_equal(g["v_scale"][b, h], r["v_scale"][b, hi])
                np.testing.assert_array_equal(g["pos"][b, h], r["pos"][b, hi])
            for t, j in enumerate(ge):   # the GPU layout agrees with its own choice
                np.testing.assert_array_equal(g["kq"][b, h, j], ck[b, h, t])
                np.testing.assert_array_equal(g["vq"][b, h, j], cv[b, h, t])
                assert g["k_scale"][b, h, j] == sk[b, h, t] and g["v_scale"][b, h, j] == sv[b, h, t]
                assert g["pos"][b, h, j] == p0 + t
    log(f"  {label}: eviction sets outside the tie band identical; swaps {swaps}")
    return g, r


def _q8_state_from_synth(cs):
    kq, ks = oracle.quantize_rows_int8(cs.k)
    vq, vs = oracle.quantize_rows_int8(cs.v)
    return dict(kq=kq, k_scale=ks, vq=vq, v_scale=vs, scores=cs.scores.astype(np.float32),
                pos=cs.pos.copy(), n=cs.n_valid)


def test_q8_small_gqa_trajectory():
    """Fill and eviction steps of the small GQA workload with the 8-bit cache;
    the oracle's state is fed in before every step."""
    wl = synth.WORKLOADS["small_gqa"]
    cs = synth.empty_state(wl)
    st = _q8_state_from_synth(cs)
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, 0)
    for step in range(wl.fill_steps + 4):
        ch = synth.gen_chunk(wl, 0, step)
        _, r = _step_and_compare(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0,
                                 label=f"small_gqa q8 step {step}")
        st = dict(kq=r["kq"], k_scale=r["k_scale"], vq=r["vq"], v_scale=r["v_scale"],
                  scores=r["scores"].astype(np.float32), pos=r["pos"], n=r["n_valid"])


def test_q8_qwen3_128k_steady_step_one_head():
    wl = synth.WORKLOADS["qwen3_4b_128k"]
    cs = synth.steady_state(wl, layer=1)
    st = _q8_state_from_synth(cs)
    ch = synth.gen_chunk(wl, 1, wl.fill_steps + 2)
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st["n"])
    _step_and_compare(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0, heads=[4],
                      label="qwen3 128k q8 steady")


def test_q8_decode_step_all_heads():
    wl = synth.WORKLOADS["decode"]
    cs = synth.prefilled_state(wl)
    st = _q8_state_from_synth(cs)
    shape = shape_of(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.cache_len,
                     wl.chunk_len, st["n"])
    for step in range(2):
        ch = synth.gen_chunk(wl, 0, step)
        _, r = _step_and_compare(shape, st, ch.q_bits, ch.k_bits, ch.v_bits, ch.p0,
                                 label=f"decode q8 step {step}")
        st = dict(kq=r["kq"], k_scale=r["k_scale"], vq=r["vq"], v_scale=r["v_scale"],
                  scores=r["scores"].astype(np.float32), pos=r["pos"], n=r["n_valid"])
