#!/usr/bin/env python3
"""Throughput of the H2O chunk step on one MI355X.

A step is one chunk of S new tokens pushed through every layer of the
workload: per layer, the four C-ABI calls (attention with summed weights,
score accumulation, slot choice, scatter) on that layer's full cache.  The
default workload is the Qwen3-4B-shaped 128k-context case: 32 query / 8 KV
heads, head_dim 128, 16384 cache slots, chunks of 1024 tokens, 36 layers, in
the steady state (cache full, every step evicts 1024 slots per KV head).
Inputs are synthetic (seeded, N(0,1) Q/K/V with 5% of K rows scaled x4) and
resident in device memory before the timed region starts.

Prints one JSON line.  ``value`` is tokens per second through all layers.
``roofline`` is for the dominant kernel (pass 1 of the attention: QK^T and PV
on MFMA), timed with HIP events around each of its launches inside the timed
region.  ``cpu_baseline`` is the CPU oracle on a bounded sample of the same
workload (one KV head of one layer-step), scaled to tokens/s.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps as one captured HIP graph replay (policy calls "
                         "on the attention stream only: one layer or --serial-policy)")
    ap.add_argument("--workload", default="qwen3_4b_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--whole-run", action="store_true",
                    help="every step of the workload from an empty cache (fill, then "
                         "eviction) through all layers; tokens/s over the summed step times")
    ap.add_argument("--calib-copy", action="store_true",
                    help="copy a 1 GiB buffer once before timing (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a summary of a rocprofv3 --stats csv run and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel FETCH_SIZE/WRITE_SIZE of a rocprofv3 --pmc csv run")
    ap.add_argument("--serial-policy", action="store_true",
                    help="issue the policy calls (accumulate, choice, scatter) on the same "
                         "stream as the attention instead of a second stream")
    ap.add_argument("--separate-calls", action="store_true",
                    help="with the policy calls on the attention stream, issue the four "
                         "calls of a layer-step separately instead of h2o_step")
    ap.add_argument("--kv8", action="store_true",
                    help="8-bit KV cache (int8 codes + one fp32 scale per row): attention "
                         "over the int8 cache and the quantising scatter")
    ap.add_argument("--backward", action="store_true",
                    help="time the attention backward (dQ, dK, dV with the slot layout "
                         "fixed) instead of the forward step")
    ap.add_argument("--mfma-summary", nargs="+", metavar="PMC_DIR",
                    help="print per-kernel SQ counters (MFMA ops and busy cycles, VALU and "
                         "MFMA instructions, waits, LDS) of rocprofv3 --pmc runs of the "
                         "default step, with the MFMA flops checked against the algorithmic "
                         "count and the busy fraction against the SQ busy cycles")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the copy-calibrated HBM bytes per dispatch of every h2o "
                         "kernel from a FETCH_SIZE and a WRITE_SIZE run (both with "
                         "--calib-copy); the file format measured_traffic() reads")
    return ap.parse_args()


CALIB_BYTES = 1 << 30


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].replace("h2o::", "")


def summarize_stats(d):
    """Kernel-time table from rocprofv3 --kernel-trace --stats --output-format csv."""
    import csv
    import glob
    path = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(path)))
    print(f"# rocprofv3 kernel stats ({os.path.basename(path)})")
    print(f"{'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for r in rows:
        print(f"{_short(r['Name'])[:48]:48s} {int(r['Calls']):6d} "
              f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
              f"{float(r['Percentage']):6.2f}")


def summarize_pmc(d):
    """Average per-dispatch counter values per kernel, plus the calibration
    factor from the 1 GiB copy (true bytes / counted bytes)."""
    import collections
    import csv
    import glob
    path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        acc[_short(r["Kernel_Name"])][r["Counter_Name"]].append(
            (int(r["Dispatch_Id"]), float(r["Counter_Value"]), int(r["Grid_Size"])))
    print(f"# rocprofv3 --pmc per-dispatch averages ({os.path.basename(path)})")
    for k, ctrs in acc.items():
        for c, vals in ctrs.items():
            per = collections.defaultdict(float)
            grid = {}
            for did, v, gsz in vals:
                per[did] += v
                grid[did] = gsz
            avg = sum(per.values()) / len(per)
            print(f"{k[:60]:60s} {c:12s} dispatches {len(per):5d} avg_KiB {avg:14.1f}")



def _pmc_kib(d, counter):
    """{kernel: average KiB per dispatch} of one rocprofv3 --pmc csv run."""
    import collections
    import csv
    import glob
    path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[_short(r["Kernel_Name"])][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def traffic_summary(fetch_dir, write_dir):
    """HBM bytes per dispatch of each h2o kernel: counter KiB x 1024, scaled by
    (true bytes / counted bytes) of the 1 GiB calibration copy."""
    fetch = _pmc_kib(fetch_dir, "FETCH_SIZE")
    write = _pmc_kib(write_dir, "WRITE_SIZE")
    copy = next(k for k in fetch if "copyBuffer" in k)
    f_scale = CALIB_BYTES / (fetch[copy][0] * 1024.0)
    w_scale = CALIB_BYTES / (write[copy][0] * 1024.0)
    print(f"# calibration: the 1 GiB copy reads FETCH_SIZE {fetch[copy][0]:.1f} KiB, "
          f"WRITE_SIZE {write[copy][0]:.1f} KiB")
    print(f"fetch_scale {f_scale:.5f}")
    print(f"write_scale {w_scale:.5f}")
    print("# bytes = counter KiB x 1024 x scale, averaged over the dispatches")
    print("# sources_sha1: attn.hip, h2o_tiles.h, h2o_device.h, h2o_launch.h")
    print(f"sources_sha1 {kernel_sources_sha1()}")
    for k in fetch:
        if k in write and "copyBuffer" not in k and not k.startswith("at::") \
                and not k.startswith("elementwise"):
            fb = fetch[k][0] * 1024.0 * f_scale
            wb = write[k][0] * 1024.0 * w_scale
            print(f"{k:28s} fetch_bytes {fb:14.0f} write_bytes {wb:14.0f}   "
                  f"dispatches {fetch[k][1]}")


def _pmc_avg(dirs):
    """{kernel: {counter: average per dispatch}} over rocprofv3 --pmc csv runs
    (counters summed over their instances within a dispatch)."""
    import collections
    import csv
    import glob
    out = collections.defaultdict(dict)
    for d in dirs:
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(path)):
            per[(_short(r["Kernel_Name"]), r["Counter_Name"])][int(r["Dispatch_Id"])] += \
                float(r["Counter_Value"])
        for (k, c), v in per.items():
            out[k][c] = (sum(v.values()) / len(v), len(v))
    return out


def mfma_summary(dirs, workload="qwen3_4b_128k"):
    """MFMA evidence of the attention kernels from SQ counters.

    flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, against 4*D*pairs (pass 1) and
    2*D*pairs (pass 2) of the steady layer-step; MFMA busy fraction =
    SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES / shader engines x SIMDs),
    i.e. over the cycles the kernel had waves resident, at the clock it ran."""
    import synth
    wl = synth.WORKLOADS[workload]
    pairs = pairs_per_layer_step(wl.batch, wl.n_q_heads, wl.cache_len, wl.chunk_len,
                                 wl.cache_len)
    algo = {"attn_fwd_kernel<128>": 4 * wl.head_dim * pairs,
            "attn_colsum_kernel<128>": 2 * wl.head_dim * pairs}
    n_se, n_simd = 32, 1024    # 8 XCDs x 4 shader engines; 256 CUs x 4 SIMDs
    data = _pmc_avg(dirs)
    print(f"# SQ counters per dispatch, {workload} steady layer-step "
          f"(pairs {pairs:.4e}); sources_sha1 {kernel_sources_sha1()}")
    for k in sorted(data, key=lambda x: -data[x].get("SQ_BUSY_CYCLES", (0, 0))[0]):
        if k.startswith("at::") or "elementwise" in k or "copyBuffer" in k:
            continue
        c = {n: v[0] for n, v in data[k].items()}
        line = "  ".join(f"{n} {v:.0f}" for n, v in sorted(c.items()))
        print(f"{k}: {line}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c and c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] > 0:
            flop = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            msg = f"    mfma_flop {flop:.4e}"
            if k in algo:
                msg += f" = {flop / algo[k]:.4f} x algorithmic {algo[k]:.4e}"
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "SQ_BUSY_CYCLES" in c:
                cyc = c["SQ_BUSY_CYCLES"] / n_se
                msg += (f"; busy cycles per SE {cyc:.0f}; MFMA busy "
                        f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * n_simd):.3f} of SIMD-cycles")
            if "SQ_INSTS_MFMA" in c and "SQ_INSTS_VALU" in c:
                msg += f"; VALU/MFMA instructions {c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f}"
            print(msg)


def kernel_sources_sha1():
    """SHA-1 over the sources the attention kernels are built from (attn.hip
    and the headers it includes), in a fixed order."""
    import hashlib
    h = hashlib.sha1()
    for name in ("attn.hip", "h2o_tiles.h", "h2o_device.h", "h2o_launch.h"):
        h.update(open(os.path.join(ROOT, "h2o_kv_cache_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def pairs_per_layer_step(B, Hq, C, S, n):
    """Causally visible (query, key) pairs of one layer-step."""
    return B * Hq * S * (n + (S + 1) / 2.0)


def make_inputs(wl, steps, gen):
    import torch
    B, Hq, Hkv, D, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk_len
    std = wl.value_std
    out = []
    for _ in range(steps):
        per_layer = []
        for _ in range(wl.layers):
            q = (torch.randn((B, Hq, S, D), generator=gen, device="cuda") * std).to(torch.bfloat16)
            k = torch.randn((B, Hkv, S, D), generator=gen, device="cuda") * std
            heavy = torch.rand((B, Hkv, S, 1), generator=gen, device="cuda") < wl.heavy_frac
            k = torch.where(heavy, k * wl.heavy_scale, k).to(torch.bfloat16)
            v = (torch.randn((B, Hkv, S, D), generator=gen, device="cuda") * std).to(torch.bfloat16)
            per_layer.append((q, k, v))
        out.append(per_layer)
    return out


def make_layer_state(wl, gen):
    import torch
    B, Hkv, D, C = wl.batch, wl.n_kv_heads, wl.head_dim, wl.cache_len
    std = wl.value_std
    # A layer's K and V caches live in one allocation (kv[0], kv[1]), the
    # way a serving engine lays out its KV-cache slab.  The streaming pass
    # over separately allocated caches measured up to 15% slower on some
    # allocations (the same kernel and bytes; the placement of the pages
    # differs), and never faster.
    kv = torch.empty((2, B, Hkv, C, D), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((B, Hkv, C, D), generator=gen, device="cuda") * std
    heavy = torch.rand((B, Hkv, C, 1), generator=gen, device="cuda") < wl.heavy_frac
    kv[0].copy_(torch.where(heavy, k * wl.heavy_scale, k))
    del k, heavy
    kv[1].copy_(torch.randn((B, Hkv, C, D), generator=gen, device="cuda") * std)
    scores = torch.rand((B, Hkv, C), generator=gen, device="cuda") * 8.0
    pos = torch.arange(C, device="cuda", dtype=torch.int64).expand(B, Hkv, C).contiguous()
    return dict(k=kv[0], v=kv[1], scores=scores, pos=pos)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    none for this workload or the kernel source changed since it was taken."""
    import re
    name = {"qwen3_4b_128k": "attn_fwd_qwen3_4b_128k_hbm_bytes.txt",
            "decode": "attn_fwd_few_decode_hbm_bytes.txt"}.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else ""
    if name is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^sources_sha1 (\w+)", text, re.M)
    if not m or m.group(1) != kernel_sources_sha1():
        return None
    m = re.search(rf"^{re.escape(kernel)}\s+fetch_bytes\s+(\d+)\s+write_bytes\s+(\d+)",
                  text, re.M)
    if not m:
        return None
    return {"fetch": int(m.group(1)), "write": int(m.group(2)),
            "total": int(m.group(1)) + int(m.group(2)),
            "source": os.path.relpath(path, ROOT)}


def _host_info():
    """BLAS threads the oracle's matrix products use, the BLAS library behind
    NumPy, the CPU model and the host's core counts (after NumPy is loaded,
    so that its BLAS pool is visible)."""
    import numpy as np  # noqa: F401  (loads the BLAS pool)
    threads, blas = len(os.sched_getaffinity(0)), "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            threads = max(i.get("num_threads", 1) for i in pools)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in pools)
    except Exception:
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"threads": int(threads), "blas": blas, "cpu_model": model,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(wl, min_seconds=10.0, max_heads=4096, q8=False):
    """The oracle as it stands, run in float32 (its ``dtype`` argument), on
    single-KV-head slices of steady layer-steps, repeated until about
    ``min_seconds`` of CPU work; scaled to tokens/s of the whole workload.
    q8: the 8-bit cache step."""
    import numpy as np
    import oracle
    import synth
    host = _host_info()
    threads = host["threads"]
    f32 = np.float32
    G = wl.group
    sub = wl.with_(n_kv_heads=1, n_q_heads=G, batch=1)
    st = synth.steady_state(sub)
    k, v, sc = st.k, st.v, st.scores.astype(np.float32)
    if q8:
        kq, ks = oracle.quantize_rows_int8(k)
        vq, vs = oracle.quantize_rows_int8(v)
    spent, heads = 0.0, 0
    while heads < max_heads and (spent < min_seconds or heads == 0):
        ch = synth.gen_chunk(sub, 0, sub.fill_steps + 2 + heads)
        t0 = time.perf_counter()
        if q8:
            oracle.h2o_step_q8(kq, ks, vq, vs, sc, st.pos, st.n_valid, ch.q, ch.k, ch.v, ch.p0,
                               dtype=f32)
        else:
            oracle.h2o_step(k, v, sc, st.pos, st.n_valid, ch.q, ch.k, ch.v, ch.p0, dtype=f32)
        spent += time.perf_counter() - t0
        heads += 1
    per_head = spent / heads
    total = per_head * wl.n_kv_heads * wl.batch * wl.layers   # s per step, all heads/layers
    return {"value": wl.chunk_len * wl.batch / total, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "dtype": "float32", **host,
            "sample": (f"{heads} steady layer-steps of one KV head each ({G} query heads, "
                       f"C={wl.cache_len}, S={wl.chunk_len}), float32, {spent:.1f} s; "
                       f"scaled x{wl.n_kv_heads * wl.batch} heads x{wl.layers} layers")}


def run_backward(args, wl):
    """Time h2o_attn_chunk_bwd over all layers of a steady step.  Each layer
    keeps one chunk (its forward output and log-sum-exp computed once,
    untimed): the backward has no value-dependent work, so the timed steps
    repeat the same calls."""
    import torch
    import h2o_kv_cache_amd as h2o
    B, Hq, Hkv, D, C, S, L = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                              wl.cache_len, wl.chunk_len, wl.layers)
    shape = h2o.Shape(B, Hq, Hkv, D, C, S, C)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261204)
    layers = [make_layer_state(wl, gen) for _ in range(L)]
    chunk = make_inputs(wl, 1, gen)[0]
    ws_f = torch.empty(h2o.h2o_workspace_size(shape), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(h2o.h2o_attn_bwd_workspace_size(shape), dtype=torch.uint8, device="cuda")
    wsum = torch.empty((B, Hkv, C + S), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fw = []
    for li, st in enumerate(layers):
        q, kn, vn = chunk[li]
        out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        h2o.h2o_attn_chunk(shape, q, st["k"], st["v"], kn, vn, out, lse, wsum, ws_f, stream)
        dout = torch.randn((B, Hq, S, D), generator=gen, device="cuda").to(torch.bfloat16)
        fw.append((out, lse, dout))
    grads = dict(dq=torch.empty((B, Hq, S, D), device="cuda"),
                 dkc=torch.empty((B, Hkv, C, D), device="cuda"),
                 dvc=torch.empty((B, Hkv, C, D), device="cuda"),
                 dkn=torch.empty((B, Hkv, S, D), device="cuda"),
                 dvn=torch.empty((B, Hkv, S, D), device="cuda"))

    def run_step():
        for li, st in enumerate(layers):
            q, kn, vn = chunk[li]
            out, lse, dout = fw[li]
            h2o.h2o_attn_chunk_bwd(shape, q, st["k"], st["v"], kn, vn, out, lse, dout,
                                   grads["dq"], grads["dkc"], grads["dvc"], grads["dkn"],
                                   grads["dvn"], ws_b, stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    h2o.h2o_timing_start(args.steps * L)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        run_step()
    t_stop.record(stream)
    torch.cuda.synchronize()
    kernel_ms, calls = h2o.h2o_timing_stop()
    elapsed_ms = t_start.elapsed_time(t_stop)
    ms_per_step = elapsed_ms / args.steps
    pairs = pairs_per_layer_step(B, Hq, C, S, C)
    # D = 128: dK/dV and dQ share one grid (bwd_dkdv_dq_kernel), then the
    # split reduction of dQ; D = 64: dK/dV, then dQ and its reduction
    names = (("bwd_prep", "bwd_dkdv_dq", "bwd_dq_reduce") if D == 128 else
             ("bwd_prep", "bwd_dkdv", "bwd_dq"))
    per_layer = {n: kernel_ms[k] / calls for n, k in zip(names, h2o.ATTN_KERNELS)}
    dkdv_ms = per_layer[names[1]]
    # algorithmic, 2*D flop per pair each: dP = dO V^T, dV = P^T dO and
    # dK = dS^T Q (the key-major part), dQ = dS K (the query-major one).
    # Executed: the key-major part also recomputes S (8*D per pair), the
    # query-major one S and dP (6*D per pair).  At D = 128 the roofline
    # kernel runs both parts: 8*D algorithmic flop per pair
    dkdv_flop = (8.0 if D == 128 else 6.0) * D * pairs
    roof = {"bound": "mfma", "achieved": dkdv_flop / (dkdv_ms * 1e-3) / 1e12,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "per_launch_flop": dkdv_flop}
    roof["frac"] = roof["achieved"] / roof["peak"]
    result = {
        "metric": "H2O chunk-step attention backward tokens/s (dQ, dK, dV; slot layout fixed)",
        "value": B * S * args.steps / (elapsed_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
            "cache_len": C, "chunk_len": S, "layers": L, "pass": "backward",
            "ms_per_layer_step": per_layer,
            "algorithmic_flop_per_layer_step": 8.0 * D * pairs,
            "algorithmic_tflops_whole_step": 8.0 * D * pairs * L / (ms_per_step * 1e-3) / 1e12,
        },
        "roofline": dict(kernel=("bwd_dkdv_dq_kernel<128> (dK/dV key tiles: S, P, dP, dV, dK; "
                                 "dQ row tiles: S, P, dP, dQ)" if D == 128
                                 else "bwd_dkdv_kernel<%d> (S, P, dP, dV, dK)" % D), traffic=None,
                         avg_launch_ms=dkdv_ms, launches=calls, **roof),
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_snapkv(wl):
    """The oracle (float32) on one KV head of one layer of the SnapKV-style
    one-shot choice (window attention over the prompt cache, keep choice,
    compaction), scaled to window tokens/s of the whole workload."""
    import numpy as np
    import oracle
    import synth
    host = _host_info()
    threads = host["threads"]
    G = wl.group
    sub = wl.with_(n_kv_heads=1, n_q_heads=G, batch=1)
    st = synth.prefilled_state(sub)
    ch = synth.gen_chunk(sub, 0, 0)
    k, v = st.k, st.v
    t0 = time.perf_counter()
    _, _, wsum = oracle.attention_chunk(ch.q, k, v, ch.k, ch.v, st.n_valid, dtype=np.float32)
    keep = oracle.snapkv_keep(wsum, st.n_valid, wl.keep_budget)
    oracle.snapkv_compact(k, v, st.pos, ch.k, ch.v, wsum, keep,
                          wl.keep_budget + wl.chunk_len, ch.p0)
    spent = time.perf_counter() - t0
    total = spent * wl.n_kv_heads * wl.batch * wl.layers
    return {"value": wl.chunk_len * wl.batch / total, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "dtype": "float32", **host,
            "sample": (f"one KV head ({G} query heads) of one layer: window attention over "
                       f"{wl.cache_len} slots, keep choice, compaction; float32, {spent:.1f} s; "
                       f"scaled x{wl.n_kv_heads * wl.batch} heads x{wl.layers} layers")}


def run_whole(args, wl):
    """The whole run of a chunked workload: every step from an empty cache --
    the fill steps (the choice appends), then the eviction steps -- through
    all layers, with the policy calls on a second stream as in the steady-state
    line.  Each step's inputs are generated before it, outside its events;
    tokens/s = all tokens / the summed step times."""
    import torch
    import h2o_kv_cache_amd as h2o
    B, Hq, Hkv, D, C, S, L = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                              wl.cache_len, wl.chunk_len, wl.layers)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203)
    bf16 = torch.bfloat16

    def empty_layer():
        return dict(k=torch.zeros((B, Hkv, C, D), dtype=bf16, device="cuda"),
                    v=torch.zeros((B, Hkv, C, D), dtype=bf16, device="cuda"),
                    scores=torch.zeros((B, Hkv, C), device="cuda"),
                    pos=torch.full((B, Hkv, C), -1, dtype=torch.int64, device="cuda"),
                    wsum=torch.empty((B, Hkv, C + S), device="cuda"),
                    new_scores=torch.empty((B, Hkv, S), device="cuda"),
                    evict=torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda"))
    layers = [empty_layer() for _ in range(L)]
    steps = wl.steps
    ns = [min(C, i * S) for i in range(steps)]
    ws = torch.empty(max(h2o.h2o_workspace_size(h2o.Shape(B, Hq, Hkv, D, C, S, n))
                         for n in sorted(set(ns))), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, S, D), device="cuda")
    lse = torch.empty((B, Hq, S), device="cuda")
    stream = torch.cuda.current_stream()
    pstream = stream if (args.serial_policy or L == 1) else torch.cuda.Stream()
    ev_attn = [torch.cuda.Event() for _ in range(L)]
    ev_pol = [torch.cuda.Event() for _ in range(L)]

    def layer_step(shape, st, q, kn, vn, p0, li):
        if pstream is not stream:
            stream.wait_event(ev_pol[li])
        h2o.h2o_attn_chunk(shape, q, st["k"], st["v"], kn, vn, out, lse, st["wsum"], ws, stream)
        if pstream is not stream:
            ev_attn[li].record(stream)
            pstream.wait_event(ev_attn[li])
        h2o.h2o_score_accumulate(shape, st["scores"], st["new_scores"], st["wsum"], pstream)
        h2o.h2o_evict_select(shape, st["scores"], st["evict"], pstream)
        h2o.kv_scatter(shape, st["k"], st["v"], st["scores"], st["pos"], kn, vn,
                       st["new_scores"], st["evict"], p0, pstream)
        if pstream is not stream:
            ev_pol[li].record(pstream)

    # untimed: one fill-phase and one eviction-phase step on a scratch layer
    scratch = empty_layer()
    warm = make_inputs(wl.with_(layers=1), 1, gen)[0][0]
    for n in (0, C):
        layer_step(h2o.Shape(B, Hq, Hkv, D, C, S, n), scratch, *warm, n, 0)
    torch.cuda.synchronize()
    del scratch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    step_ms = []
    for i in range(steps):
        chunk = make_inputs(wl, 1, gen)[0]
        torch.cuda.synchronize()
        shape = h2o.Shape(B, Hq, Hkv, D, C, S, ns[i])
        e0.record(stream)
        for li, st in enumerate(layers):
            layer_step(shape, st, *chunk[li], i * S, li)
        stream.wait_stream(pstream)
        e1.record(stream)
        torch.cuda.synchronize()
        step_ms.append(e0.elapsed_time(e1))
        del chunk
    total_ms = float(sum(step_ms))
    fill = [t for t, n in zip(step_ms, ns) if n + S <= C]
    evict = [t for t, n in zip(step_ms, ns) if n + S > C]
    pct = lambda x: [float(np.percentile(x, q)) for q in (10, 50, 90)] if x else None
    result = {
        "metric": "H2O chunk-step tokens/s over the whole run (fill + eviction steps), "
                  "all layers",
        "value": B * S * steps / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 0,
        "ms_per_step": total_ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
            "cache_len": C, "chunk_len": S, "layers": L, "context": wl.seq_len,
            "fill_steps": len(fill), "eviction_steps": len(evict),
            "fill_step_ms_p10_p50_p90": pct(fill),
            "eviction_step_ms_p10_p50_p90": pct(evict),
            "policy_stream": ("same stream" if pstream is stream else
                              "second stream, overlapped with the next layer's attention"),
            "calls": "h2o_attn_chunk, h2o_score_accumulate, h2o_evict_select, kv_scatter",
            "timing": "events around each step; inputs generated between steps",
        },
    }
    print(json.dumps(result), flush=True)


def run_snapkv(args, wl):
    """Time the SnapKV-style one-shot choice at the end of a prompt, over all
    layers: per layer the window chunk's attention over the prompt cache
    (h2o_attn_chunk, unchanged), the keep choice and the compaction into a
    cache of budget + S slots.  The input caches are not modified, so every
    timed step repeats the same work."""
    import torch
    import h2o_kv_cache_amd as h2o
    B, Hq, Hkv, D, C, S, L = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                              wl.cache_len, wl.chunk_len, wl.layers)
    budget = wl.keep_budget
    out_len = budget + S
    shape = h2o.Shape(B, Hq, Hkv, D, C, S, C)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261205)
    layers = [make_layer_state(wl, gen) for _ in range(L)]
    chunk = make_inputs(wl, 1, gen)[0]
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    wsum = torch.empty((B, Hkv, C + S), dtype=torch.float32, device="cuda")
    keep = torch.empty((B, Hkv, budget), dtype=torch.int32, device="cuda")
    ws = torch.empty(h2o.h2o_workspace_size(shape), dtype=torch.uint8, device="cuda")
    outs = [dict(k=torch.empty((B, Hkv, out_len, D), dtype=torch.bfloat16, device="cuda"),
                 v=torch.empty((B, Hkv, out_len, D), dtype=torch.bfloat16, device="cuda"),
                 pos=torch.empty((B, Hkv, out_len), dtype=torch.int64, device="cuda"),
                 scores=torch.empty((B, Hkv, out_len), dtype=torch.float32, device="cuda"))
            for _ in range(L)]
    stream = torch.cuda.current_stream()
    p0 = C

    def attn(li):
        q, kn, vn = chunk[li]
        st = layers[li]
        h2o.h2o_attn_chunk(shape, q, st["k"], st["v"], kn, vn, out, lse, wsum, ws, stream)

    def select(li):
        h2o.h2o_snapkv_select(shape, wsum, budget, keep, stream)

    def compact(li):
        q, kn, vn = chunk[li]
        st, o = layers[li], outs[li]
        h2o.h2o_snapkv_compact(shape, st["k"], st["v"], st["pos"], kn, vn, wsum, keep, budget,
                               out_len, p0, o["k"], o["v"], o["pos"], o["scores"], stream)

    def run_step():
        for li in range(L):
            attn(li)
            select(li)
            compact(li)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    h2o.h2o_timing_start(args.steps * L)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        run_step()
    t_stop.record(stream)
    torch.cuda.synchronize()
    kernel_ms, calls = h2o.h2o_timing_stop()
    elapsed_ms = t_start.elapsed_time(t_stop)
    ms_per_step = elapsed_ms / args.steps

    # per-call times of the choice and the compaction (one untimed pass each,
    # bracketed by events on the same stream; the wsum of the last layer)
    part_ms = {}
    for name, fn in (("snapkv_select", select), ("snapkv_compact", compact)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for li in range(L):
            fn(li)
        e1.record(stream)
        torch.cuda.synchronize()
        part_ms[name] = e0.elapsed_time(e1) / L

    pairs = pairs_per_layer_step(B, Hq, C, S, C)
    per_layer = {k: v / calls for k, v in kernel_ms.items()}
    per_layer.update(part_ms)
    fwd_ms = per_layer["attn_fwd"]
    fwd_flop = 4.0 * D * pairs
    roof = {"bound": "mfma", "achieved": fwd_flop / (fwd_ms * 1e-3) / 1e12,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "per_launch_flop": fwd_flop}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # compaction moves budget + S rows of K and V per KV head (read + write)
    cp_bytes = 2.0 * 2 * B * Hkv * out_len * D * 2
    result = {
        "metric": ("SnapKV-style one-shot choice at the end of a 128k prompt: window tokens/s "
                   "(window attention + keep choice + compaction, all layers)"),
        "value": B * S * args.steps / (elapsed_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
            "prompt_len": wl.seq_len, "cache_len": C, "window": S, "keep_budget": budget,
            "out_len": out_len, "layers": L,
            "ms_per_layer": per_layer,
            "compact_gbs": cp_bytes / (part_ms["snapkv_compact"] * 1e-3) / 1e9,
        },
        "roofline": dict(kernel="attn_fwd_kernel<%d> (pass 1: QK^T, online softmax, PV)" % D,
                         traffic=None, avg_launch_ms=fwd_ms, launches=calls, **roof),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_snapkv(wl)
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the H2O step shards by KV head or by "
              "sequence with no exchange, so a run on more than one GPU measures "
              "nothing a single GPU does not (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import h2o_kv_cache_amd as h2o

    wl = synth.WORKLOADS[args.workload]
    h2o.load_library()
    torch.cuda.set_device(0)
    if args.backward:
        run_backward(args, wl)
        return
    if args.whole_run:
        if wl.prefilled or wl.keep_budget > 0:
            print("--whole-run covers chunked workloads that start from an empty cache",
                  file=sys.stderr)
            sys.exit(2)
        run_whole(args, wl)
        return
    if wl.keep_budget > 0:
        run_snapkv(args, wl)
        return
    B, Hq, Hkv, D, C, S, L = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                              wl.cache_len, wl.chunk_len, wl.layers)
    shape = h2o.Shape(B, Hq, Hkv, D, C, S, C)   # steady state: cache full
    tok_per_step = B * S
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203)
    layers = [make_layer_state(wl, gen) for _ in range(L)]
    if args.kv8:   # the same caches, quantised on the device
        for st in layers:
            for name in ("k", "v"):
                codes = torch.empty((B, Hkv, C, D), dtype=torch.int8, device="cuda")
                scales = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
                h2o.h2o_quantize_rows_q8(st[name], codes, scales)
                st[name + "q"], st[name + "s"] = codes, scales
                del st[name]
        torch.cuda.synchronize()
    inputs = make_inputs(wl, args.warmup + args.steps * (2 if args.graph else 1), gen)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    # per layer: the policy calls of a layer may still run while the next
    # layer's attention writes its own summed weights
    for st in layers:
        st["wsum"] = torch.empty((B, Hkv, C + S), dtype=torch.float32, device="cuda")
        st["new_scores"] = torch.empty((B, Hkv, S), dtype=torch.float32, device="cuda")
        st["evict"] = torch.empty((B, Hkv, S), dtype=torch.int32, device="cuda")
    ws = torch.empty(h2o.h2o_workspace_size(shape), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # The policy calls of layer l (accumulate, choice, scatter) need only that
    # layer's summed weights; the attention of layer l+1 does not depend on
    # them, and the attention of layer l at the next step needs the scatter.
    # They run on a second stream (default priority), ordered by events.
    # With one layer there is nothing to overlap (the next step's attention
    # waits for the scatter), and the events only add latency.
    pstream = stream if (args.serial_policy or L == 1) else torch.cuda.Stream()
    main_stream, policy_stream = stream, pstream
    if args.graph and pstream is not stream:
        print("--graph captures the policy calls on the attention stream: use it with one "
              "layer or --serial-policy", file=sys.stderr)
        sys.exit(2)
    ev_attn = [torch.cuda.Event() for _ in range(L)]
    ev_pol = [torch.cuda.Event() for _ in range(L)]
    p0_base = (C // S + 2) * S

    # one stream and a bf16 cache: the whole layer-step in one call (for
    # one-token chunks the work after the streaming pass is one kernel)
    single_call = pstream is stream and not args.kv8 and not args.separate_calls

    def run_step(i, s_main=None):
        stream = s_main if s_main is not None else main_stream
        pstream = stream if policy_stream is main_stream else policy_stream
        p0 = p0_base + i * S
        for li, st in enumerate(layers):
            q, kn, vn = inputs[i][li]
            wsum, new_scores, evict = st["wsum"], st["new_scores"], st["evict"]
            if single_call:
                h2o.h2o_step(shape, q, st["k"], st["v"], kn, vn, out, lse, wsum, st["scores"],
                             new_scores, evict, st["pos"], p0, ws, stream)
                continue
            if pstream is not stream:
                stream.wait_event(ev_pol[li])        # the cache after last step's scatter
            if args.kv8:
                h2o.h2o_attn_chunk_q8(shape, q, st["kq"], st["ks"], st["vq"], st["vs"], kn, vn,
                                      out, lse, wsum, ws, stream)
            else:
                h2o.h2o_attn_chunk(shape, q, st["k"], st["v"], kn, vn, out, lse, wsum, ws,
                                   stream)
            if pstream is not stream:
                ev_attn[li].record(stream)
                pstream.wait_event(ev_attn[li])
            h2o.h2o_score_accumulate(shape, st["scores"], new_scores, wsum, pstream)
            h2o.h2o_evict_select(shape, st["scores"], evict, pstream)
            if args.kv8:
                h2o.kv_scatter_q8(shape, st["kq"], st["ks"], st["vq"], st["vs"], st["scores"],
                                  st["pos"], kn, vn, new_scores, evict, p0, pstream)
            else:
                h2o.kv_scatter(shape, st["k"], st["v"], st["scores"], st["pos"], kn, vn,
                               new_scores, evict, p0, pstream)
            if pstream is not stream:
                ev_pol[li].record(pstream)

    if args.calib_copy:   # a copy of known size, to scale the HBM byte counters
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    h2o.h2o_timing_start(args.steps * L)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # step boundaries on the attention stream (the policy calls of a step
    # overlap the next step's attention; the last step ends when they do)
    marks = [t_start] + [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    t_start.record(stream)
    for i in range(args.steps):
        if i > 0:
            marks[i].record(stream)
        run_step(args.warmup + i)
    stream.wait_stream(pstream)               # the last policy calls end the step
    t_stop.record(stream)
    torch.cuda.synchronize()
    kernel_ms, calls = h2o.h2o_timing_stop()
    elapsed_ms = t_start.elapsed_time(t_stop)
    marks.append(t_stop)
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    eager_ms = elapsed_ms
    if args.graph:
        # the next K steps (their own inputs and positions) captured once,
        # replayed once untimed, then timed as one replay
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                run_step(args.warmup + args.steps + i, cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        graph.replay()
        t_stop.record(stream)
        torch.cuda.synchronize()
        elapsed_ms = t_start.elapsed_time(t_stop)

    ms_per_step = elapsed_ms / args.steps
    tokens_per_s = B * S * args.steps / (elapsed_ms / 1e3)
    pairs = pairs_per_layer_step(B, Hq, C, S, C)
    fwd_ms = kernel_ms["attn_fwd"] / calls
    per_layer = {k: v / calls for k, v in kernel_ms.items()}
    if single_call and Hq // Hkv * S <= 32 and S == 1:
        # h2o_step's decode path: the streaming pass, then the tail kernels
        # (weights, scores and running minimum; choice and scatter)
        per_layer = {"attn_fwd": per_layer["attn_fwd"], "decode_tail": per_layer["attn_combine"]}
    # pass 1 reads every cached K/V row once plus the chunk's Q/K/V
    cache_row_bytes = (D + 4) if args.kv8 else 2 * D   # int8 codes + scale, or bf16
    fwd_bytes = (2.0 * B * Hkv * (C * cache_row_bytes + S * D * 2)) + B * Hq * S * D * 2
    fwd_flop = 4.0 * D * pairs                   # QK^T + PV, 2 flop per MAC
    if fwd_flop / fwd_bytes >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:   # above the ridge
        roof = {"bound": "mfma", "achieved": fwd_flop / (fwd_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "per_launch_flop": fwd_flop}
    else:
        roof = {"bound": "hbm", "achieved": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "per_launch_bytes": fwd_bytes}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rows = Hq // Hkv * S   # packed query rows per (b, kv head)
    small = rows <= 32
    if args.kv8:
        fwd_kernel = ("attn_fwd_few_q8_kernel<%d>" if rows <= 16 else
                      "attn_fwd_small_q8_kernel<%d>" if small else "attn_fwd_q8_kernel<%d>") % D
    else:
        fwd_kernel = ("attn_fwd_few_kernel<%d>" if rows <= 16 else
                      "attn_fwd_small_kernel<%d>" if small else "attn_fwd_kernel<%d>") % D
    traffic = None if args.kv8 else measured_traffic(wl.name, fwd_kernel)
    per_layer["policy_and_gaps"] = ms_per_step / L - sum(per_layer.values())
    total_flop_exec = 6.0 * D * pairs
    step_tflops = total_flop_exec * L / (ms_per_step * 1e-3) / 1e12

    result = {
        "metric": "H2O chunk-step tokens/s (attn+scores+evict) at 128k ctx; % MFMA/HBM peak",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" + (" (int8 KV cache)" if args.kv8 else ""),
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
            "cache_len": C, "chunk_len": S, "layers": L, "context": wl.seq_len,
            "kv_cache": "int8 codes + fp32 row scales" if args.kv8 else "bf16",
            "phase": "steady state: cache full, S slots evicted per KV head per layer",
            "ms_per_layer_step": per_layer,
            "policy_stream": ("same stream" if pstream is stream else
                              "second stream, overlapped with the next layer's attention"),
            "calls": "h2o_step (one call per layer-step)" if single_call else
                     "h2o_attn_chunk, h2o_score_accumulate, h2o_evict_select, kv_scatter",
            "executed_mfma_tflops_whole_step": step_tflops,
            "executed_mfma_frac_whole_step": step_tflops / PEAK_BF16_TFLOPS,
            "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
            "timing": ("one HIP graph replay of the K steps; per-kernel split and step "
                       "percentiles from the eager loop (%.4f ms/step eager)"
                       % (eager_ms / args.steps)) if args.graph else "eager launches",
        },
        "roofline": dict(
            kernel=fwd_kernel + " (pass 1: QK^T, online softmax, PV)",
            traffic=(traffic["total"] if traffic else None), traffic_detail=traffic,
            avg_launch_ms=fwd_ms, launches=calls, **roof),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, q8=args.kv8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
