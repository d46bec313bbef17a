"""Trajectory parity at full size: the oracle walks real steps from the
workload's initial cache (empty, or pre-filled for decode), so the scores it
feeds in are accumulated from real summed weights -- heavy hitters, ties,
slot reuse -- rather than drawn at random.  Before each compared step the
oracle's cache state of the sampled (batch row, KV head) pairs is uploaded
into the full-size device cache; the GPU then runs the workload's own launch
shape through the C ABI and its outputs for the sampled pairs are compared
with the oracle's at the usual tolerances.

Per-head work is independent (the choice is per batch row and KV head), so
the pairs that are not sampled hold a fixed synthetic cache of the same fill;
their outputs are not compared.

Cadence: the one-KV-head share of the 128k layers over all 128 steps of
layer 0 (steps 15, 16, 17, then every 8th and the last), the 8-head 128k
layer through the fill into three eviction steps on two heads, the 64k layer
over all 32 steps on one head, and decode on one sequence for 64 steps.
"""
import numpy as np
import pytest
import torch

import synth
from synth import WORKLOADS

from h2o_harness import HostState, compare, log, oracle_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import h2o_kv_cache_amd as h2o
    h2o.load_library()


def _dev_u16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda()


class SampledRun:
    """The oracle's trajectory of the sampled pairs, advanced step by step."""

    def __init__(self, wl, rows, heads, layer=0):
        import h2o_kv_cache_amd as h2o
        self.h2o = h2o
        self.wl, self.rows, self.heads, self.layer = wl, list(rows), list(heads), layer
        G = wl.group
        self.qheads = [h * G + g for h in self.heads for g in range(G)]
        init = synth.prefilled_state(wl, layer) if wl.prefilled else synth.empty_state(wl)
        ix = np.ix_(self.rows, self.heads)
        self.st = HostState(init.k_bits[ix].copy(), init.v_bits[ix].copy(),
                            init.scores[ix].astype(np.float32), init.pos[ix].copy(),
                            init.n_valid)
        # device cache of the full shape: valid synthetic rows for every pair
        # (the sampled pairs are overwritten before each compared step)
        base = init if wl.prefilled else synth.steady_state(wl, layer)
        self.kc = _dev_u16(base.k_bits)
        self.vc = _dev_u16(base.v_bits)
        self.scores = torch.from_numpy(base.scores.astype(np.float32)).cuda()
        self.pos = torch.from_numpy(base.pos.astype(np.int64)).cuda()
        B, Hq, Hkv, D, C, S = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                               wl.cache_len, wl.chunk_len)
        self.out = torch.empty((B, Hq, S, D), device="cuda")
        self.lse = torch.empty((B, Hq, S), device="cuda")
        self.wsum = torch.empty((B, Hkv, C + S), device="cuda")
        self.new_scores = torch.empty((B, Hkv, S), device="cuda")
        self.evict = torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda")
        shape = h2o.Shape(B, Hq, Hkv, D, C, S, 0, 0.0)
        self.ws = torch.empty(max(h2o.h2o_workspace_size(shape), 256), dtype=torch.uint8,
                              device="cuda")
        self.step = 0
        self.worst = {}

    def _sub_chunk(self, ch):
        r = self.rows
        return (ch.q_bits[r][:, self.qheads], ch.k_bits[r][:, self.heads],
                ch.v_bits[r][:, self.heads])

    def _gpu(self, ch):
        """The four calls at the full shape with the sampled pairs' state fed
        in; host copies of the sampled pairs' results."""
        h2o, wl, st = self.h2o, self.wl, self.st
        B, Hq, Hkv, D, C, S = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                               wl.cache_len, wl.chunk_len)
        rows = torch.tensor(self.rows, device="cuda")
        heads = torch.tensor(self.heads, device="cuda")
        qh = torch.tensor(self.qheads, device="cuda")
        # feed the oracle's state of the sampled pairs into the full cache
        for i, b in enumerate(self.rows):
            self.kc[b, heads] = _dev_u16(st.k_bits[i])
            self.vc[b, heads] = _dev_u16(st.v_bits[i])
            self.scores[b, heads] = torch.from_numpy(st.scores[i]).cuda()
            self.pos[b, heads] = torch.from_numpy(st.pos[i]).cuda()
        bf = torch.bfloat16
        kc, vc = self.kc.view(bf), self.vc.view(bf)
        q, kn, vn = (_dev_u16(ch.q_bits).view(bf), _dev_u16(ch.k_bits).view(bf),
                     _dev_u16(ch.v_bits).view(bf))
        for t in (self.out, self.lse, self.wsum, self.new_scores):
            t.fill_(float("nan"))
        self.evict.fill_(-7)
        self.ws.fill_(0xFF)
        shape = h2o.Shape(B, Hq, Hkv, D, C, S, st.n_valid, 0.0)
        h2o.h2o_attn_chunk(shape, q, kc, vc, kn, vn, self.out, self.lse, self.wsum, self.ws)
        h2o.h2o_score_accumulate(shape, self.scores, self.new_scores, self.wsum)
        acc = self.scores.clone()
        h2o.h2o_evict_select(shape, self.scores, self.evict)
        h2o.kv_scatter(shape, kc, vc, self.scores, self.pos, kn, vn, self.new_scores,
                       self.evict, ch.p0)
        torch.cuda.synchronize()

        def pick_kv(t):   # [B, Hkv, ...] -> sampled pairs
            return t.index_select(0, rows).index_select(1, heads).cpu().numpy()

        def pick_q(t):    # [B, Hq, ...] -> sampled pairs' query heads
            return t.index_select(0, rows).index_select(1, qh).cpu().numpy()

        return dict(out=pick_q(self.out), lse=pick_q(self.lse), wsum=pick_kv(self.wsum),
                    new_scores=pick_kv(self.new_scores), scores_acc=pick_kv(acc),
                    evict_idx=pick_kv(self.evict),
                    k_bits=pick_kv(self.kc).view(np.uint16),
                    v_bits=pick_kv(self.vc).view(np.uint16),
                    scores=pick_kv(self.scores), pos=pick_kv(self.pos))

    def advance(self, until, compare_at):
        """Run the oracle to step ``until`` (exclusive); compare the GPU at the
        steps in ``compare_at``."""
        wl = self.wl
        while self.step < until:
            step = self.step
            ch = synth.gen_chunk(wl, self.layer, step)
            qb, kb, vb = self._sub_chunk(ch)
            r = oracle_step(self.st, qb, kb, vb, ch.p0)
            if step in compare_at:
                log(f"[trajectory] {wl.name} layer {self.layer} step {step} "
                    f"n={self.st.n_valid} rows={self.rows} heads={self.heads}")
                g = self._gpu(ch)
                s = compare(g, r, self.st, kb, vb, ch.p0, f"{wl.name}:{step}")
                log(f"[trajectory] {wl.name} step {step} {s}")
                for k, v in s.items():
                    self.worst[k] = max(self.worst.get(k, 0), v)
            self.st = HostState(synth.to_bf16(r["k_cache"].astype(np.float32))[0],
                                synth.to_bf16(r["v_cache"].astype(np.float32))[0],
                                r["scores"].astype(np.float32), r["pos"].copy(),
                                r["n_valid"])
            self.step += 1
        log(f"[trajectory] {wl.name} worst so far {self.worst}")


_RUNS = {}


def _run(key, make):
    if key not in _RUNS:
        _RUNS[key] = make()
    return _RUNS[key]


# --- the one-KV-head share of the 128k layers, all 128 steps of layer 0 ---
HEAD = WORKLOADS["qwen3_4b_128k_head"]
HEAD_COMPARE = {15, 16, 17} | set(range(24, HEAD.steps, 8)) | {HEAD.steps - 1}


@pytest.mark.parametrize("part", range(4))
def test_qwen3_128k_head_trajectory(part):
    # four parts of 32 steps; a part run on its own replays the earlier ones
    run = _run("128k_head", lambda: SampledRun(HEAD, rows=[0], heads=[0], layer=0))
    run.advance(32 * (part + 1), HEAD_COMPARE)
    if part == 3:
        assert run.step == HEAD.steps
        # scores accumulated over real steps reach far beyond one step's weights
        assert float(run.st.scores.max()) > HEAD.group * 4


def test_qwen3_128k_eviction_after_real_fill():
    # all 8 KV heads on the device; the oracle follows heads 2 and 7 through
    # the 16 fill steps into three eviction steps
    wl = WORKLOADS["qwen3_4b_128k"]
    run = SampledRun(wl, rows=[0], heads=[2, 7], layer=0)
    fill = wl.fill_steps
    run.advance(fill + 3, {fill - 1, fill, fill + 1, fill + 2})


def test_qwen3_64k_trajectory():
    wl = WORKLOADS["qwen3_4b_64k"]
    run = SampledRun(wl, rows=[0], heads=[5], layer=0)
    run.advance(wl.steps, {3, 4, 5} | set(range(8, wl.steps, 4)) | {wl.steps - 1})


def test_decode_trajectory():
    # 16 sequences on the device; the oracle follows sequence 3 (all heads)
    # for 64 single-token steps from the pre-filled cache
    wl = WORKLOADS["decode"]
    run = SampledRun(wl, rows=[3], heads=list(range(wl.n_kv_heads)), layer=0)
    run.advance(64, set(range(64)))
