"""The no-workspace attention entry point (h2o_attn_chunk_static, for callers
that cannot allocate) against h2o_attn_chunk with a caller workspace: same
kernels, same plan, so the outputs must agree bit for bit.  The calls run
largest scratch first, so every later call starts from the scratch contents
an earlier, larger call left behind."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

# name, B, Hq, Hkv, D, C, S, n_valid  (workspace sizes decreasing)
CASES = [
    ("decode_16x16384", 16, 32, 8, 128, 16384, 1, 16384),
    ("qwen3_128k_layer", 1, 32, 8, 128, 16384, 1024, 16384),
    ("small_gqa_partial", 1, 8, 2, 128, 2048, 256, 1280),
    ("tiny_from_empty", 1, 2, 1, 64, 256, 64, 0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import h2o_kv_cache_amd as h2o
    h2o.load_library()


def _inputs(B, Hq, Hkv, D, C, S, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16
    r = lambda *s: torch.randn(s, generator=g, device="cuda").to(bf)
    return r(B, Hq, S, D), r(B, Hkv, C, D), r(B, Hkv, C, D), r(B, Hkv, S, D), r(B, Hkv, S, D)


def _outputs(B, Hq, Hkv, D, C, S):
    return (torch.full((B, Hq, S, D), float("nan"), device="cuda"),
            torch.full((B, Hq, S), float("nan"), device="cuda"),
            torch.full((B, Hkv, C + S), float("nan"), device="cuda"))


def test_static_scratch_matches_workspace_entry_point():
    import h2o_kv_cache_amd as h2o
    for i, (name, B, Hq, Hkv, D, C, S, n) in enumerate(CASES):
        print(f"[no-alloc] {name} B={B} Hq={Hq} Hkv={Hkv} D={D} C={C} S={S} n={n}",
              flush=True)
        shape = h2o.Shape(B, Hq, Hkv, D, C, S, n, 0.0)
        need = h2o.h2o_workspace_size(shape)
        assert 0 < need <= h2o.STATIC_SCRATCH_BYTES
        if i > 0:
            assert need < h2o.h2o_workspace_size(h2o.Shape(*CASES[i - 1][1:8], 0.0))
        q, kc, vc, kn, vn = _inputs(B, Hq, Hkv, D, C, S, 1000 + i)
        st = _outputs(B, Hq, Hkv, D, C, S)
        h2o.h2o_attn_chunk_static(shape, q, kc, vc, kn, vn, *st)
        torch.cuda.synchronize()
        ref = _outputs(B, Hq, Hkv, D, C, S)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        h2o.h2o_attn_chunk(shape, q, kc, vc, kn, vn, *ref, ws)
        torch.cuda.synchronize()
        for label, a, b in zip(("out", "lse", "wsum"), st, ref):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert np.isfinite(a).all(), (name, label)
            assert np.array_equal(a, b), (name, label, float(np.abs(a - b).max()))
        # the summed weights of a (b, kv head) total G * S (each row sums to 1)
        tot = st[2].double().sum(dim=2).cpu().numpy()
        np.testing.assert_allclose(tot, (Hq // Hkv) * S, rtol=1e-4)
        print(f"[no-alloc] {name} bit-identical", flush=True)
