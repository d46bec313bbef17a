"""Pins of the oracle's 8-bit cache (quantisation, attention over int8 rows,
quantising scatter) against facts other than its own code: exact codes for
rows whose scale is a power of two, round-half-even on ties, the half-step
error bound, and attention over exactly representable rows equal to the
unquantised attention.  CPU only."""
import math

import numpy as np
import pytest

import oracle


def test_power_of_two_scales_give_exact_codes():
    # amax = 127 * 2^e makes the float32 scale exactly 2^e, so x / scale is
    # exact and the codes are the integers themselves
    ints = np.array([127, -63, 1, 0, -127, 5, 64, -1], np.float32)
    for e in (-20, -3, 0, 4, 30):
        x = (ints * np.float32(2.0 ** e)).reshape(1, -1)
        codes, sc = oracle.quantize_rows_int8(x)
        assert sc[0] == np.float32(2.0 ** e)
        assert codes[0].tolist() == ints.astype(int).tolist()


def test_ties_round_to_even():
    codes, sc = oracle.quantize_rows_int8(np.array([[127, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5]],
                                                    np.float32))
    assert sc[0] == 1.0
    assert codes[0].tolist() == [127, 0, 2, 2, 0, -2, 126]


def test_zero_row_and_sign_of_the_largest():
    codes, sc = oracle.quantize_rows_int8(np.zeros((2, 3, 8), np.float32))
    assert (codes == 0).all() and (sc == 0).all()
    codes, sc = oracle.quantize_rows_int8(np.array([[-3.0, 1.0, 2.0]], np.float32))
    assert codes[0, 0] == -127 and sc[0] == np.float32(3.0) / np.float32(127.0)


def test_half_step_error_bound():
    # round to nearest: |x - code * scale| <= scale / 2 (plus float32 slack),
    # and the row's largest |x| maps to +-127
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((50, 128)) * rng.uniform(0.01, 100, (50, 1))).astype(np.float32)
    codes, sc = oracle.quantize_rows_int8(x)
    err = np.abs(x.astype(np.float64) - oracle.dequantize_rows_int8(codes, sc))
    assert (err <= sc[:, None].astype(np.float64) * (0.5 + 1e-5)).all()
    assert (np.abs(codes).max(axis=1) == 127).all()
    assert np.abs(codes.astype(int)).max() <= 127


def test_attention_over_representable_rows_equals_unquantised():
    # rows = integer vectors (amax 127) times 2^e with e per row and per
    # tensor: quantisation is exact, so the int8 attention must equal the
    # attention on the original values; a scale applied to the wrong row or
    # tensor breaks the equality
    rng = np.random.default_rng(22)
    B, Hq, Hkv, D, C, S, n = 1, 4, 2, 16, 24, 5, 19
    def rows(shape):
        ints = rng.integers(-127, 128, size=shape).astype(np.float32)
        ints[..., 0] = 127
        e = rng.integers(-8, 3, size=shape[:-1]).astype(np.float32)
        return ints * np.float32(2.0) ** e[..., None]
    kc, vc = rows((B, Hkv, C, D)), rows((B, Hkv, C, D))
    kq, ks = oracle.quantize_rows_int8(kc)
    vq, vs = oracle.quantize_rows_int8(vc)
    q = rng.standard_normal((B, Hq, S, D)) * 0.05
    kn, vn = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    want = oracle.attention_chunk(q, kc, vc, kn, vn, n)
    got = oracle.attention_chunk_q8(q, kq, ks, vq, vs, kn, vn, n)
    for w, g in zip(want, got):
        np.testing.assert_allclose(g, w, rtol=1e-13, atol=1e-13)
    # swapping the two scale arrays changes the result
    bad = oracle.attention_chunk_q8(q, kq, vs, vq, ks, kn, vn, n)
    assert np.abs(bad[0] - want[0]).max() > 1e-3


def test_scatter_writes_the_quantised_chunk():
    rng = np.random.default_rng(23)
    B, Hkv, C, D, S = 1, 2, 10, 8, 3
    kq = np.zeros((B, Hkv, C, D), np.int8)
    vq = np.zeros((B, Hkv, C, D), np.int8)
    ks = np.zeros((B, Hkv, C), np.float32)
    vs = np.zeros((B, Hkv, C), np.float32)
    sc = np.zeros((B, Hkv, C))
    pos = np.full((B, Hkv, C), -1, np.int64)
    kn = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    ev = np.array([[[1, 4, 9], [0, 2, 3]]])
    oracle.kv_scatter_q8(kq, ks, vq, vs, sc, pos, kn, vn, np.ones((B, Hkv, S)), ev, p0=40)
    for h in range(Hkv):
        for t in range(S):
            j = ev[0, h, t]
            x = kn[0, h, t]
            assert ks[0, h, j] == np.float32(np.abs(x).max()) / np.float32(127)
            assert np.abs(x - kq[0, h, j] * np.float64(ks[0, h, j])).max() <= ks[0, h, j] * 0.50001
            assert pos[0, h, j] == 40 + t
        untouched = [j for j in range(C) if j not in ev[0, h]]
        assert (kq[0, h, untouched] == 0).all() and (pos[0, h, untouched] == -1).all()


def _representable_rows(rng, shape, e_lo, e_hi):
    """Rows that the 8-bit format stores exactly: integer vectors whose
    largest magnitude is 127, times 2^e with one e per row.  Returns the
    values and, for an independent check of the stored rows, the integers
    and the exponents."""
    ints = rng.integers(-126, 127, size=shape).astype(np.float32)
    ints[..., 0] = np.where(rng.random(shape[:-1]) < 0.5, 127, -127)
    e = rng.integers(e_lo, e_hi, size=shape[:-1])
    return ints * np.float32(2.0) ** e[..., None].astype(np.float32), ints, e


def test_scatter_writes_codes_scale_and_score_of_every_token():
    # K and V rows exactly representable with different exponent ranges, so
    # every written code and scale is known in advance; distinct new scores
    # per (head, token), so a token or head index slip shows
    rng = np.random.default_rng(24)
    B, Hkv, C, D, S = 2, 2, 11, 8, 4
    kn, ki, ke = _representable_rows(rng, (B, Hkv, S, D), -6, -1)
    vn, vi, ve = _representable_rows(rng, (B, Hkv, S, D), 1, 5)
    kq = np.full((B, Hkv, C, D), 3, np.int8)
    vq = np.full((B, Hkv, C, D), -3, np.int8)
    ks = np.full((B, Hkv, C), 7.0, np.float32)
    vs = np.full((B, Hkv, C), 9.0, np.float32)
    sc = np.full((B, Hkv, C), -1.0)
    pos = np.full((B, Hkv, C), -1, np.int64)
    new_sc = np.arange(B * Hkv * S, dtype=np.float64).reshape(B, Hkv, S) + 0.25
    ev = np.array([[[0, 3, 4, 10], [1, 2, 7, 8]], [[5, 6, 9, 10], [0, 1, 2, 3]]])
    oracle.kv_scatter_q8(kq, ks, vq, vs, sc, pos, kn, vn, new_sc, ev, p0=100)
    for b in range(B):
        for h in range(Hkv):
            for t in range(S):
                j = ev[b, h, t]
                assert kq[b, h, j].tolist() == ki[b, h, t].astype(int).tolist()
                assert vq[b, h, j].tolist() == vi[b, h, t].astype(int).tolist()
                assert ks[b, h, j] == np.float32(2.0 ** ke[b, h, t])
                assert vs[b, h, j] == np.float32(2.0 ** ve[b, h, t])
                assert sc[b, h, j] == new_sc[b, h, t]
                assert pos[b, h, j] == 100 + t
            rest = [j for j in range(C) if j not in ev[b, h]]
            assert (kq[b, h, rest] == 3).all() and (vq[b, h, rest] == -3).all()
            assert (ks[b, h, rest] == 7).all() and (vs[b, h, rest] == 9).all()
            assert (sc[b, h, rest] == -1).all() and (pos[b, h, rest] == -1).all()


def test_whole_q8_step_equals_the_unquantised_step_on_representable_rows():
    # every K/V row (cache and chunk) is exactly representable, with per-row
    # power-of-two scales drawn from different ranges for K and V: the 8-bit
    # step must then equal the unquantised step bit for bit over a whole run
    # (fill, partial overflow and eviction steps), and the stored codes and
    # scales of every slot must be those of the token its position names
    rng = np.random.default_rng(25)
    B, Hq, Hkv, D, C, S, steps = 1, 4, 2, 16, 10, 4, 6
    T = S * steps
    kn_all, ki, ke = _representable_rows(rng, (B, Hkv, T, D), -5, 0)
    vn_all, vi, ve = _representable_rows(rng, (B, Hkv, T, D), 0, 4)
    q_all = rng.standard_normal((B, Hq, T, D)) * 0.02
    kc = np.zeros((B, Hkv, C, D))
    vc = np.zeros((B, Hkv, C, D))
    kq = np.zeros((B, Hkv, C, D), np.int8)
    vq = np.zeros((B, Hkv, C, D), np.int8)
    ks = np.zeros((B, Hkv, C), np.float32)
    vs = np.zeros((B, Hkv, C), np.float32)
    sc = np.zeros((B, Hkv, C))
    sc8 = np.zeros((B, Hkv, C))
    pos = np.full((B, Hkv, C), -1, np.int64)
    pos8 = pos.copy()
    n = n8 = 0
    for step in range(steps):
        sl = slice(step * S, (step + 1) * S)
        args = (q_all[:, :, sl], kn_all[:, :, sl], vn_all[:, :, sl], step * S)
        r = oracle.h2o_step(kc, vc, sc, pos, n, *args)
        r8 = oracle.h2o_step_q8(kq, ks, vq, vs, sc8, pos8, n8, *args)
        for key in ("out", "lse", "wsum", "scores_acc", "new_scores", "evict_idx", "scores",
                    "pos"):
            np.testing.assert_array_equal(r8[key], r[key], err_msg=f"step {step} {key}")
        assert r8["n_valid"] == r["n_valid"]
        np.testing.assert_array_equal(oracle.dequantize_rows_int8(r8["kq"], r8["k_scale"]),
                                      r["k_cache"])
        np.testing.assert_array_equal(oracle.dequantize_rows_int8(r8["vq"], r8["v_scale"]),
                                      r["v_cache"])
        for b in range(B):
            for h in range(Hkv):
                for j in range(C):
                    p = r8["pos"][b, h, j]
                    if p < 0:
                        continue
                    assert r8["kq"][b, h, j].tolist() == ki[b, h, p].astype(int).tolist()
                    assert r8["vq"][b, h, j].tolist() == vi[b, h, p].astype(int).tolist()
                    assert r8["k_scale"][b, h, j] == np.float32(2.0 ** ke[b, h, p])
                    assert r8["v_scale"][b, h, j] == np.float32(2.0 ** ve[b, h, p])
        kc, vc, sc, pos, n = r["k_cache"], r["v_cache"], r["scores"], r["pos"], r["n_valid"]
        kq, ks, vq, vs = r8["kq"], r8["k_scale"], r8["vq"], r8["v_scale"]
        sc8, pos8, n8 = r8["scores"], r8["pos"], r8["n_valid"]
    assert n == C   # the run reached eviction steps
