"""One step's four C-ABI calls captured in a HIP graph (through torch's graph
capture) and replayed.  The calls allocate nothing and record no memset, so
the graph holds only their kernels; every replay -- with eager work between
replays -- must match the eager step bit for bit (all reductions have a fixed
order)."""
import pytest
import torch

from h2o_harness import h2o, log, shape_of

pytestmark = pytest.mark.gpu


def _make(B, Hq, Hkv, D, C, S, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)
    init = dict(k=bf(B, Hkv, C, D), v=bf(B, Hkv, C, D),
                scores=torch.rand((B, Hkv, C), generator=g, device="cuda") * 4,
                pos=torch.arange(C, device="cuda").repeat(B, Hkv, 1).to(torch.int64))
    chunk = dict(q=bf(B, Hq, S, D), kn=bf(B, Hkv, S, D), vn=bf(B, Hkv, S, D))
    return init, chunk


def _buffers(B, Hq, Hkv, D, C, S, shape):
    return dict(out=torch.empty((B, Hq, S, D), device="cuda"),
                lse=torch.empty((B, Hq, S), device="cuda"),
                wsum=torch.empty((B, Hkv, C + S), device="cuda"),
                new_scores=torch.empty((B, Hkv, S), device="cuda"),
                evict=torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda"),
                ws=torch.empty(max(h2o.h2o_workspace_size(shape), 256), dtype=torch.uint8,
                               device="cuda"))


def _reset(st, init, buf):
    for name, t in init.items():
        st[name].copy_(t)
    for name in ("out", "lse", "wsum", "new_scores"):
        buf[name].fill_(float("nan"))
    buf["evict"].fill_(-7)


def _step(shape, st, ch, buf, p0):
    h2o.h2o_attn_chunk(shape, ch["q"], st["k"], st["v"], ch["kn"], ch["vn"], buf["out"],
                       buf["lse"], buf["wsum"], buf["ws"])
    h2o.h2o_score_accumulate(shape, st["scores"], buf["new_scores"], buf["wsum"])
    h2o.h2o_evict_select(shape, st["scores"], buf["evict"])
    h2o.kv_scatter(shape, st["k"], st["v"], st["scores"], st["pos"], ch["kn"], ch["vn"],
                   buf["new_scores"], buf["evict"], p0)


def _snapshot(st, buf):
    return {**{k: v.clone() for k, v in st.items()},
            **{k: v.clone() for k, v in buf.items() if k != "ws"}}


@pytest.mark.parametrize("B,Hq,Hkv,D,C,S", [
    (4, 8, 2, 128, 2048, 1),     # few-row path (one decode token per sequence)
    (1, 8, 2, 128, 2048, 128),   # chunk path: pass 1, merge, pass 2, reduce
])
def test_step_graph_replays_match_eager(B, Hq, Hkv, D, C, S):
    log(f"[graph] B={B} Hq={Hq} Hkv={Hkv} D={D} C={C} S={S}")
    shape = shape_of(B, Hq, Hkv, D, C, S, C)
    init, ch = _make(B, Hq, Hkv, D, C, S, seed=4242 + S)
    p0 = C + 7
    st = {k: torch.empty_like(v) for k, v in init.items()}
    buf = _buffers(B, Hq, Hkv, D, C, S, shape)

    _reset(st, init, buf)
    _step(shape, st, ch, buf, p0)
    torch.cuda.synchronize()
    ref = _snapshot(st, buf)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _reset(st, init, buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _step(shape, st, ch, buf, p0)
    torch.cuda.synchronize()

    for rep in range(3):
        _reset(st, init, buf)                 # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(st, buf)
        for name, t in ref.items():
            assert torch.equal(got[name], t), (rep, name)
        log(f"[graph] replay {rep} matches the eager step")
