"""Pins of the oracle's attention backward against things other than its own
formula: central finite differences of the forward (float64), and the two
shift invariances of attention.  CPU only (no gpu mark)."""
import numpy as np
import pytest

import oracle



def _inputs(seed, B=1, Hq=4, Hkv=2, D=8, C=7, S=5, n=5, std=1.0):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s) * std
    return (f(B, Hq, S, D), f(B, Hkv, C, D), f(B, Hkv, C, D), f(B, Hkv, S, D),
            f(B, Hkv, S, D), n, f(B, Hq, S, D))


def _loss(q, kc, vc, kn, vn, n, dout, scale=None):
    out, _, _ = oracle.attention_chunk(q, kc, vc, kn, vn, n, scale)
    return float((out * dout).sum())


@pytest.mark.parametrize("seed,n,scale", [(0, 5, None), (1, 0, None), (2, 7, 0.3)])
def test_backward_matches_finite_differences(seed, n, scale):
    q, kc, vc, kn, vn, _, dout = _inputs(seed, n=n)
    grads = oracle.attention_chunk_backward(q, kc, vc, kn, vn, n, dout, scale)
    args = [q, kc, vc, kn, vn]
    h = 1e-5
    for which, (x, g) in enumerate(zip(args, grads)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(*args, n, dout, scale)
            x[idx] = keep - h
            dn = _loss(*args, n, dout, scale)
            x[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=2e-7, rtol=1e-6, err_msg=f"input {which}")
    # empty slots receive no gradient
    assert np.all(grads[1][:, :, n:] == 0) and np.all(grads[2][:, :, n:] == 0)


def test_key_gradients_sum_to_zero():
    # adding one vector to every visible key of a KV head shifts each row's
    # logits by a constant, which softmax ignores
    q, kc, vc, kn, vn, n, dout = _inputs(3, B=2, Hq=6, Hkv=2, D=16, C=9, S=6, n=8)
    dq, dkc, dvc, dkn, dvn = oracle.attention_chunk_backward(q, kc, vc, kn, vn, n, dout)
    total = dkc[:, :, :n].sum(axis=2) + dkn.sum(axis=2)
    np.testing.assert_allclose(total, 0.0, atol=1e-12)


def test_value_gradients_sum_to_upstream():
    # adding one vector to every value shifts every output row by it
    q, kc, vc, kn, vn, n, dout = _inputs(4, B=1, Hq=6, Hkv=3, D=8, C=4, S=7, n=4)
    dq, dkc, dvc, dkn, dvn = oracle.attention_chunk_backward(q, kc, vc, kn, vn, n, dout)
    G = 2
    total = dvc.sum(axis=2) + dvn.sum(axis=2)                  # [B, Hkv, D]
    up = dout.reshape(1, 3, G, 7, 8).sum(axis=(2, 3))
    np.testing.assert_allclose(total, up, atol=1e-12)


def test_identical_keys_give_zero_query_gradient():
    q, kc, vc, kn, vn, n, dout = _inputs(5, n=7)
    kc[:] = 0.7
    kn[:] = 0.7
    dq = oracle.attention_chunk_backward(q, kc, vc, kn, vn, n, dout)[0]
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
