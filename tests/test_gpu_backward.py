"""GPU parity of the attention backward (slot layout fixed) against the CPU
oracle, through the C ABI.  The forward's O and log-sum-exp are the oracle's,
rounded to fp32, so both sides differentiate the same forward.

Tolerance (no figure on the pages): the kernels feed P and dS to the MFMAs in
bf16 (relative rounding 2^-9) with dO, Q, K, V already bf16, and accumulate in
fp32.  Each gradient entry is a sum of such rounded products, so its error is
bounded by about 2^-9 times the sum of the magnitudes of its terms, which for
these inputs stays within a few times 2^-9 of the largest entry of that
gradient.  The test takes max|gpu - oracle| <= 2^-6 * max|oracle| per tensor
(and prints the measured ratio)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from h2o_harness import dev_bf16, log

pytestmark = pytest.mark.gpu

TOL_REL = 2.0 ** -6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import h2o_kv_cache_amd as h2o
    h2o.load_library()


def _bf16(rng, shape, std=1.0):
    return synth.to_bf16((rng.standard_normal(shape) * std).astype(np.float32))


def _run(B, Hq, Hkv, D, C, S, n, seed, heads=None, std=1.0, garbage=False):
    import h2o_kv_cache_amd as h2o
    rng = np.random.default_rng(seed)
    (qb, qf), (kcb, kcf), (vcb, vcf) = (_bf16(rng, (B, Hq, S, D), std),
                                        _bf16(rng, (B, Hkv, C, D), std),
                                        _bf16(rng, (B, Hkv, C, D), std))
    (knb, knf), (vnb, vnf), (dob, dof) = (_bf16(rng, (B, Hkv, S, D), std),
                                          _bf16(rng, (B, Hkv, S, D), std),
                                          _bf16(rng, (B, Hq, S, D)))
    if garbage:          # empty slots hold NaN / inf patterns: must not leak
        kcb[:, :, n:] = 0x7FC1
        vcb[:, :, n:] = 0xFF80
    G = Hq // Hkv
    hs = list(range(Hkv)) if heads is None else heads
    qh = np.concatenate([np.arange(h * G, (h + 1) * G) for h in hs])
    kcf_o, vcf_o = kcf[:, hs].astype(np.float64), vcf[:, hs].astype(np.float64)
    out, lse, _ = oracle.attention_chunk(qf[:, qh], kcf_o, vcf_o, knf[:, hs], vnf[:, hs], n)
    ref = oracle.attention_chunk_backward(qf[:, qh], kcf_o, vcf_o, knf[:, hs], vnf[:, hs], n,
                                          dof[:, qh])
    # device inputs: the full tensors; out / lse only needed for the checked heads,
    # the others get the oracle's values too when heads is None
    out_full = np.zeros((B, Hq, S, D), np.float32)
    lse_full = np.zeros((B, Hq, S), np.float32)
    out_full[:, qh] = out.astype(np.float32)
    lse_full[:, qh] = lse.astype(np.float32)
    shape = h2o.Shape(B, Hq, Hkv, D, C, S, n)
    dev = lambda a: torch.from_numpy(a).cuda()
    dq = torch.full((B, Hq, S, D), float("nan"), device="cuda")
    dkc = torch.full((B, Hkv, C, D), float("nan"), device="cuda")
    dvc = torch.full((B, Hkv, C, D), float("nan"), device="cuda")
    dkn = torch.full((B, Hkv, S, D), float("nan"), device="cuda")
    dvn = torch.full((B, Hkv, S, D), float("nan"), device="cuda")
    ws = torch.full((max(h2o.h2o_attn_bwd_workspace_size(shape), 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    log(f"[bwd] B={B} Hq={Hq} Hkv={Hkv} D={D} C={C} S={S} n={n} heads={hs}")
    h2o.h2o_attn_chunk_bwd(shape, dev_bf16(qb), dev_bf16(kcb), dev_bf16(vcb), dev_bf16(knb),
                           dev_bf16(vnb), dev(out_full), dev(lse_full), dev_bf16(dob), dq, dkc,
                           dvc, dkn, dvn, ws)
    torch.cuda.synchronize()
    got = [dq.cpu().numpy()[:, qh], dkc.cpu().numpy()[:, hs], dvc.cpu().numpy()[:, hs],
           dkn.cpu().numpy()[:, hs], dvn.cpu().numpy()[:, hs]]
    names = ["dq", "dk_cache", "dv_cache", "dk_new", "dv_new"]
    worst = {}
    for name, g, r in zip(names, got, ref):
        assert np.all(np.isfinite(g)), name
        scale = max(float(np.max(np.abs(r))), 1e-30)
        err = float(np.max(np.abs(g - r)))
        worst[name] = err / scale
        assert err <= TOL_REL * scale, (name, err, scale)
    assert np.all(got[1][:, :, n:] == 0) and np.all(got[2][:, :, n:] == 0)
    log(f"[bwd] max error / max magnitude: { {k: f'{v:.2e}' for k, v in worst.items()} }")
    return worst


CASES = [
    # B, Hq, Hkv, D, C, S, n
    (1, 4, 2, 64, 100, 20, 70),
    (2, 8, 2, 128, 300, 50, 300),
    (1, 4, 1, 128, 64, 64, 0),
    (1, 3, 3, 64, 257, 33, 200),
    (1, 6, 2, 128, 130, 1, 130),
    (1, 16, 1, 128, 520, 40, 333),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,C,S,n", CASES)
def test_backward_small(B, Hq, Hkv, D, C, S, n):
    _run(B, Hq, Hkv, D, C, S, n, seed=B * 1000 + C + S)


def test_backward_garbage_in_empty_slots():
    _run(1, 4, 2, 128, 200, 48, 120, seed=7, garbage=True)


def test_backward_qwen3_128k_one_head():
    # one KV head of the 128k-context shape (C = 16384 full, S = 1024)
    _run(1, 32, 8, 128, 16384, 1024, 16384, seed=11, heads=[5])
