#!/usr/bin/env python3
"""Benchmark: k8v4 decode attention at 118,750 cells x 48 layers on one MI355X.

One step = one decoded token across 48 layers: for every layer, append the
token's K/V at cell 118,749 and attend over cells [0, 118,750), in one
fused call (attn_decode_append; the two-call form kv_append_k8v4 +
attn_decode is timed beside it in extra).  Each layer has its own pool (96.9 MB of k8v4
pages, 4.65 GB in all, far beyond the 256 MB Infinity Cache), so every step
streams its KV from HBM.  The step is captured once per step index in a HIP
graph (torch.cuda.CUDAGraph) and replayed; W untimed steps, then K timed
steps between two synchronizations.

Prints one JSON line on stdout:
  value = KV bytes read per second over the whole step (GB/s, 1e9 B/s),
  ms_per_step, us_per_layer, hbm_frac (value / 8 TB/s),
  roofline: the decode kernel alone, algorithmic bytes (cells x 816 B per
            launch) over its mean duration from start/stop events recorded
            by hipExtLaunchKernelGGL around each launch,
  cpu_baseline: the CPU oracle on the host's cores on a bounded sample (one
            layer's decode, 1 thread and the default thread count; append,
            verify and a prefill sample under extra.cpu_oracle),
  extra: decode / verify at 240,000 cells and the 8,192-query prefill chunk.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
CELL_BYTES = 816               # k8v4, 2 KV heads x 256 dims
METRIC = "decode-attn µs/step and KV-read GB/s (% of HBM peak) at 119K/240K ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (copy-calibrated), or None when the kernel source has
    changed since those counters were taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "attn_splitk_decode_118750_traffic.json")
    try:
        rec = json.load(open(rec_path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["bytes_per_launch"]


def fill_pool(k8, synth, pool, pt, seed, layer, ctx, dev):
    for c, s in enumerate(range(0, ctx, synth.CHUNK)):
        n = min(synth.CHUNK, ctx - s)
        k, v = synth.kv_chunk_device(seed, layer, c, n, 2, 256, dev)
        k8.kv_append_k8v4(pool, pt, k, v, s)


def make_table(torch, synth, seed, layer, n_table, n_pages, dev):
    pt = synth.page_table(seed * 1000 + layer, n_table, n_pages)
    return torch.from_numpy(pt).to(dev)


def event_mean_ms(torch, pairs):
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in pairs]
    return sum(ts) / len(ts), ts


def spread_us(ts):
    """Median, 10th and 90th percentile (nearest rank) of per-launch times
    given in ms, in us."""
    s = sorted(ts)

    def q(p):
        return round(s[min(len(s) - 1, int(p * (len(s) - 1) + 0.5))] * 1e3, 3)

    return {"launches": len(s), "median_us": q(0.5), "p10_us": q(0.1), "p90_us": q(0.9)}


LEAD_CYCLES_PER_LAUNCH = 300_000


def timed_launches(torch, k8, fn, n):
    """Run fn() n times, each single kernel bracketed by start/stop events.
    A spin kernel enqueued first holds the GPU until the host has queued all
    n calls, so the launches run back to back, as the kernels of a replayed
    graph do, not each after an idle gap the host's enqueue time left (the
    launch after such a gap runs up to ~20 % slower)."""
    torch.cuda._sleep(LEAD_CYCLES_PER_LAUNCH * n)
    pairs = []
    for i in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()  # torch creates the HIP event on first record
        e1.record()
        k8.time_next_launch(e0, e1)
        fn(i)
        pairs.append((e0, e1))
    return event_mean_ms(torch, pairs)


def timed_calls(torch, fn, n):
    """Run fn() n times, each call (all its kernels) bracketed by events."""
    pairs = []
    for i in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        pairs.append((e0, e1))
    return event_mean_ms(torch, pairs)


def graph_calls_ms(torch, fn, n_calls, replays=4):
    """Device time per call of fn(0..n_calls-1) captured back to back in one
    HIP graph (so host launch overhead is excluded), mean over replays."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(n_calls):
                fn(i)
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * n_calls)


def stream_read_ceiling(torch, k8, dev):
    """Attainable read bandwidth: a plain streaming read of 1 GiB (beyond the
    Infinity Cache) by the library's yardstick kernel."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    k8.probe_read(buf, sink)
    ms = graph_calls_ms(torch, lambda i: k8.probe_read(buf, sink), 5)
    del buf
    return {"gbs": round((1 << 30) / ms / 1e6, 1), "bytes": 1 << 30,
            "kernel": "probe_read_kernel: 512 workgroups, each streaming its own contiguous 2 MiB with 256 lanes x 4 non-temporal 16 B loads per round"}


def stream_read_same_size(torch, k8, dev, n_bufs=6):
    """A plain streaming read of exactly one decode's KV bytes (118,750 and
    240,000 cells x 816 B), one launch at a time over n_bufs rotated buffers
    (beyond the Infinity Cache), timed like the split kernel (start/stop
    events around each launch): what a single launch of that size attains,
    start-up and tail included."""
    out = {}
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    for cells in (118750, 240000):
        b = cells * CELL_BYTES
        bufs = [torch.empty(b, dtype=torch.uint8, device=dev).fill_(1) for _ in range(n_bufs)]
        for i in range(n_bufs):
            k8.probe_read(bufs[i], sink)
        ms, _ = timed_launches(torch, k8, lambda i: k8.probe_read(bufs[i % n_bufs], sink), 8 * n_bufs)
        out[str(cells)] = {"us": round(ms * 1e3, 3), "gbs": round(b / ms / 1e6, 1), "bytes": b}
        del bufs
    return out


def cpu_info():
    """CPU model, logical CPUs of the host and those this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count() or 1, "usable_cpus": usable}


def cpu_baseline():
    """The oracle on the host's cores, on bounded samples of the workloads:
    one 240,000-cell oracle pool built by appends of 8,192-token chunks
    (timed per chunk), then decode at 118,750 cells with 1 thread and with
    the oracle's default thread count (the headline value), decode at the
    sweep's other lengths (1,024 .. 131,072 cells), decode and the 5-query
    verify at 240,000 cells, and 32 sampled rows of the 8,192-query
    prefill chunk at [231,808, 240,000) (first 8, last 8, 16 seeded others),
    extrapolated to the whole chunk.  Inputs follow the numpy stream of the
    same recipe."""
    import numpy as np

    import oracle
    from long_context_decode_append_amd import synth
    P, ctx, n_pages = 256, 240000, 1024
    threads = oracle.default_threads()
    pt = synth.page_table(4, (ctx + P - 1) // P, n_pages)
    pool = oracle.OraclePool(3, n_pages, P, 2)
    app = []
    for s in range(0, ctx, synth.CHUNK):
        n = min(synth.CHUNK, ctx - s)
        k, v = synth.kv_tokens(4, 0, s, n, 2, 256, np.float16)
        t0 = time.perf_counter()
        pool.append(pt, k, v, s)
        if n == synth.CHUNK:
            app.append(time.perf_counter() - t0)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    q1 = synth.queries(3, 0, 0, 1, 16, 256, np.float16)
    d1 = timed(lambda: oracle.attention_from_pool(pool, pt, q1, [118750], threads=1))
    dn = timed(lambda: oracle.attention_from_pool(pool, pt, q1, [118750], threads=threads))
    d240 = timed(lambda: oracle.attention_from_pool(pool, pt, q1, [ctx], threads=threads))
    # the decode context sweep's other lengths, same threads
    sweep = {n: timed(lambda n=n: oracle.attention_from_pool(pool, pt, q1, [n], threads=threads))
             for n in (1024, 4096, 16384, 32768, 65536, 131072)}
    q5 = synth.queries(4, 0, 1, 5, 16, 256, np.float16)
    v5 = timed(lambda: oracle.attention_from_pool(pool, pt, q5, [ctx - 4 + i for i in range(5)], threads=threads))
    pos0, n_new = 231808, 8192
    rows = list(range(8)) + list(range(n_new - 8, n_new)) + sorted(
        np.random.default_rng(5).choice(np.arange(8, n_new - 8), 16, replace=False).tolist())
    qp = synth.queries(5, 0, 0, n_new, 16, 256, np.float16)[rows]
    pf = timed(lambda: oracle.attention_from_pool(pool, pt, qp, [pos0 + r + 1 for r in rows], threads=threads))
    flops_rows = sum(1024.0 * 16 * (pos0 + r + 1) for r in rows)
    flops_all = sum(1024.0 * 16 * (pos0 + i + 1) for i in range(n_new))
    b118 = 118750 * CELL_BYTES
    info = cpu_info()
    base = {"value": round(b118 / dn / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"one layer of the 48: a 118,750-cell decode step (gather, dequantize, fp64 attention "
                      f"for 16 heads) by the C oracle with {threads} threads, {dn:.2f} s",
            "single_thread_gbs": round(b118 / d1 / 1e9, 4), "single_thread_s": round(d1, 3),
            **info}
    extra = {"threads": threads, **info,
             "append_8192_tokens_s": round(float(np.mean(app)), 4),
             "append_tokens_per_s": round(synth.CHUNK / float(np.mean(app)), 1),
             "decode_118750_s": {"1_thread": round(d1, 3), f"{threads}_threads": round(dn, 3)},
             "decode_240000_s": round(d240, 3), "decode_240000_gbs": round(ctx * CELL_BYTES / d240 / 1e9, 4),
             "decode_sweep_s": {str(n): round(t, 4) for n, t in sweep.items()},
             "verify5_240000_s": round(v5, 3),
             "prefill_32_sampled_rows_s": round(pf, 3),
             "prefill_8192_at_231808_s_extrapolated": round(pf * flops_all / flops_rows, 1),
             "prefill_extrapolation": "time of the 32 sampled rows scaled by the chunk's flops over theirs"}
    return base, extra


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode240000", "copy", "prefill", "verify"], default=None,
                    help="profiling aids: 'decode' runs 24 eager fused append + decode calls at "
                         "118,750 cells (8 layer pools); 'decode240000' runs 12 decode calls at "
                         "240,000 cells over 3 pools; 'copy' runs 4 plain 1 GiB device copies "
                         "(calibrates the HBM byte counters); 'prefill' runs the 8,192-query chunk "
                         "at 231,808 twice; 'verify' runs 4 five-query verify calls at 240,000")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the k8v4 attention path here is a single-GPU "
              "kernel library (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_decode_append_amd as k8
    from long_context_decode_append_amd import synth

    dev = torch.device("cuda:0")
    k8.lib()
    if args.only is not None:
        profile_only(args.only, torch, k8, synth, dev)
        return
    layers, ctx, P = 48, 118750, 256
    n_pages = (ctx + P - 1) // P                     # 464 pages, the last one partly used
    seed = 3
    W, K = args.warmup, args.steps

    log(f"filling {layers} layer pools of {ctx} cells ...")
    pools, tables = [], []
    for l in range(layers):
        pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, seed, l, n_pages, n_pages, dev)
        fill_pool(k8, synth, pool, pt, seed, l, ctx, dev)
        pools.append(pool)
        tables.append(pt)
    ws = k8.attn_workspace(pools[0], 1, ctx)
    outs = [torch.empty((16, 256), dtype=torch.float32, device=dev) for _ in range(layers)]
    n_steps = W + K
    q_all = [[synth.queries_device(seed, l, s, 1, 16, 256, dev)[0] for l in range(layers)]
             for s in range(n_steps)]
    kv_new = [[synth.kv_chunk_device(seed, l, 10_000 + s, 1, 2, 256, dev) for l in range(layers)]
              for s in range(n_steps)]
    torch.cuda.synchronize()

    def step(s):
        for l in range(layers):
            kn, vn = kv_new[s][l]
            k8.attn_decode_append(pools[l], tables[l], kn[0], vn[0], q_all[s][l], ctx - 1, ws,
                                  out=outs[l])

    # eager run of every step once (also warms the library's device cache)
    log("eager pass ...")
    t0 = time.perf_counter()
    for s in range(n_steps):
        step(s)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_steps

    log("capturing graphs ...")
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for s in range(n_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(s)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    log(f"warmup {W}, timed {K} steps ...")
    for s in range(W):
        graphs[s].replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record()
    for s in range(W, W + K):
        graphs[s].replay()
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = ev0.elapsed_time(ev1) / K
    kv_bytes_step = layers * ctx * CELL_BYTES
    value = kv_bytes_step / (step_ms * 1e-3) / 1e9

    # the decode kernel on its own: start/stop events around each launch
    log("per-kernel timing ...")
    dec_ms, dec_ts = timed_launches(torch, k8, lambda i: k8.attn_decode_append(
        pools[i % layers], tables[i % layers], kv_new[0][i % layers][0][0], kv_new[0][i % layers][1][0],
        q_all[0][i % layers], ctx - 1, ws, out=outs[i % layers]), 2 * layers)
    app_ms, _ = timed_launches(torch, k8, lambda i: k8.kv_append_k8v4(
        pools[i % layers], tables[i % layers], kv_new[0][i % layers][0],
        kv_new[0][i % layers][1], ctx - 1), layers)
    dec_gbs = ctx * CELL_BYTES / (dec_ms * 1e-3) / 1e9
    traffic_bytes = measured_traffic()
    traffic = None if traffic_bytes is None else round(traffic_bytes / (dec_ms * 1e-3) / 1e9, 2)

    extra = {}
    if not args.no_extra:
        del graphs
        extra = bench_extra(torch, k8, synth, dev, log)
        extra["stream_read_ceiling"] = stream_read_ceiling(torch, k8, dev)
        extra["stream_read_same_size"] = stream_read_same_size(torch, k8, dev)
        dc_ms = graph_calls_ms(torch, lambda i: k8.attn_decode(
            pools[i % layers], tables[i % layers], q_all[0][i % layers], ctx, ws,
            out=outs[i % layers]), layers, replays=2)
        extra["decode_118750_split_plus_combine"] = {
            "us": round(dc_ms * 1e3, 3),
            "hbm_frac": round(ctx * CELL_BYTES / dc_ms / 1e6 / HBM_PEAK_GBS, 4)}

        def two_call(i):
            l = i % layers
            kn, vn = kv_new[0][l]
            k8.kv_append_k8v4(pools[l], tables[l], kn, vn, ctx - 1)
            k8.attn_decode(pools[l], tables[l], q_all[0][l], ctx, ws, out=outs[l])

        def fused(i):
            l = i % layers
            kn, vn = kv_new[0][l]
            k8.attn_decode_append(pools[l], tables[l], kn[0], vn[0], q_all[0][l], ctx - 1, ws,
                                  out=outs[l])
        extra["layer_118750_append_and_decode_us"] = {
            "fused (attn_decode_append)": round(graph_calls_ms(torch, fused, layers, replays=2) * 1e3, 3),
            "two calls (kv_append_k8v4 + attn_decode)": round(
                graph_calls_ms(torch, two_call, layers, replays=2) * 1e3, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu, extra["cpu_oracle"] = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_118750x48", "ctx": ctx, "layers": layers, "batch": 1,
                   "q_heads": 16, "kv_heads": 2, "head_dim": 256, "page_size": P,
                   "kv_format": "k8v4 (816 B/cell)", "per_step": "48 x (append 1 token + decode), fused (attn_decode_append)",
                   "launch": "HIP graph per step"},
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_layer": round(step_ms * 1e3 / layers, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "eager_ms_per_step": round(eager_ms, 3),
        "wall_s_timed": round(t_wall, 4),
        "roofline": {"kernel": "attn_splitk_kernel (decode with fused append, 1 query)", "bound": "hbm",
                     "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": ctx * CELL_BYTES, "traffic_bytes_per_launch": traffic_bytes,
                     "mean_us": round(dec_ms * 1e3, 3), "spread": spread_us(dec_ts),
                     "append_mean_us": round(app_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def profile_only(what, torch, k8, synth, dev):
    """Short, fixed workloads for counter collection under rocprofv3."""
    if what in ("prefill", "verify"):
        ctx, P, n_pages = 240000, 256, 1024
        pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, 4, 0, (ctx + P - 1) // P, n_pages, dev)
        fill_pool(k8, synth, pool, pt, 4, 0, ctx, dev)
        if what == "prefill":
            pos0, n_new = 231808, 8192
            q = synth.queries_device(4, 0, 0, n_new, 16, 256, dev)
            out = torch.empty((n_new, 16, 256), dtype=torch.float32, device=dev)
            pws = k8.attn_prefill_workspace(pool, pos0 + n_new)
            for _ in range(2):
                k8.attn_prefill_chunk(pool, pt, q, pos0, out=out, ws=pws)
            log(f"2 prefill chunks of {n_new} at {pos0}")
        else:
            nv = [ctx - 4 + i for i in range(5)]
            q = synth.queries_device(4, 0, 0, 5, 16, 256, dev)
            ws = k8.attn_workspace(pool, 5, ctx)
            for _ in range(4):
                k8.attn_verify(pool, pt, q, nv, ws)
            log(f"4 verify calls of 5 queries at {ctx}")
        torch.cuda.synchronize()
        return
    if what == "decode240000":
        ctx, P, n_pages, n_pools = 240000, 256, 1024, 3
        pools, tables = [], []
        for i in range(n_pools):
            pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
            pt = make_table(torch, synth, 4, i, (ctx + P - 1) // P, n_pages, dev)
            fill_pool(k8, synth, pool, pt, 4, i, ctx, dev)
            pools.append(pool)
            tables.append(pt)
        q = synth.queries_device(4, 0, 0, 1, 16, 256, dev)[0]
        ws = k8.attn_workspace(pools[0], 1, ctx)
        for i in range(4 * n_pools):
            k8.attn_decode(pools[i % n_pools], tables[i % n_pools], q, ctx, ws)
        torch.cuda.synchronize()
        log(f"{4 * n_pools} decode calls at {ctx} cells over {n_pools} pools")
        return
    if what == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(7)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x 4")
        return
    ctx, P, layers = 118750, 256, 8
    n_pages = (ctx + P - 1) // P
    pools, tables = [], []
    for l in range(layers):
        pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, 3, l, n_pages, n_pages, dev)
        fill_pool(k8, synth, pool, pt, 3, l, ctx, dev)
        pools.append(pool)
        tables.append(pt)
    ws = k8.attn_workspace(pools[0], 1, ctx)
    q = synth.queries_device(3, 0, 0, 1, 16, 256, dev)[0]
    out = torch.empty((16, 256), dtype=torch.float32, device=dev)
    kn, vn = synth.kv_chunk_device(3, 0, 10_000, 1, 2, 256, dev)
    for i in range(3 * layers):
        # the bench step's call: the token of cell ctx - 1, then attention over [0, ctx)
        k8.attn_decode_append(pools[i % layers], tables[i % layers], kn[0], vn[0], q, ctx - 1, ws, out=out)
    torch.cuda.synchronize()
    log(f"{3 * layers} decode calls (fused append) at {ctx} cells")


def bench_extra(torch, k8, synth, dev, log):
    """Decode and verify at 240,000 cells (6 rotated 262,144-cell pools,
    1.28 GB, beyond the Infinity Cache), the 8,192-query prefill chunk and
    the append of an 8,192-token chunk."""
    out = {}
    ctx, P, n_pages, n_pools = 240000, 256, 1024, 6
    n_table = (ctx + P - 1) // P
    log(f"extra: filling {n_pools} pools of {ctx} cells ...")
    pools, tables = [], []
    for i in range(n_pools):
        pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, 4, i, n_table, n_pages, dev)
        fill_pool(k8, synth, pool, pt, 4, i, ctx, dev)
        pools.append(pool)
        tables.append(pt)
    q1 = synth.queries_device(4, 0, 0, 1, 16, 256, dev)[0]
    q5 = synth.queries_device(4, 0, 1, 5, 16, 256, dev)
    ws1 = k8.attn_workspace(pools[0], 1, ctx)
    ws5 = k8.attn_workspace(pools[0], 5, ctx)
    nv = [ctx - 4, ctx - 3, ctx - 2, ctx - 1, ctx]
    for i in range(n_pools):  # warm
        k8.attn_decode(pools[i], tables[i], q1, ctx, ws1)
        k8.attn_verify(pools[i], tables[i], q5, nv, ws5)
    reps = 9 * n_pools  # at least 50 launches over the pool rotation
    d_ms, d_ts = timed_launches(torch, k8, lambda i: k8.attn_decode(
        pools[i % n_pools], tables[i % n_pools], q1, ctx, ws1), reps)
    dc_ms = graph_calls_ms(torch, lambda i: k8.attn_decode(
        pools[i % n_pools], tables[i % n_pools], q1, ctx, ws1), 2 * n_pools)
    v_ms, v_ts = timed_launches(torch, k8, lambda i: k8.attn_verify(
        pools[i % n_pools], tables[i % n_pools], q5, nv, ws5), reps)
    vc_ms = graph_calls_ms(torch, lambda i: k8.attn_verify(
        pools[i % n_pools], tables[i % n_pools], q5, nv, ws5), 2 * n_pools)
    b = ctx * CELL_BYTES
    out["decode_240000"] = {"us": round(d_ms * 1e3, 3), "gbs": round(b / d_ms / 1e6, 2),
                            "hbm_frac": round(b / d_ms / 1e6 / HBM_PEAK_GBS, 4),
                            "pools_rotated": n_pools, "kernel": "split kernel alone",
                            "spread": spread_us(d_ts),
                            "us_split_plus_combine": round(dc_ms * 1e3, 3),
                            "hbm_frac_split_plus_combine": round(b / dc_ms / 1e6 / HBM_PEAK_GBS, 4)}
    # context sweep on the same pools: whole decode call (split + combine),
    # calls replayed back to back from a graph
    sweep = {}
    for n in (1024, 4096, 16384, 32768, 65536, 118750, 131072, 240000):
        s_ms = graph_calls_ms(torch, lambda i, n=n: k8.attn_decode(
            pools[i % n_pools], tables[i % n_pools], q1, n, ws1), 2 * n_pools)
        sweep[str(n)] = {"us": round(s_ms * 1e3, 2), "gbs": round(n * CELL_BYTES / s_ms / 1e6, 1),
                         "hbm_frac": round(n * CELL_BYTES / s_ms / 1e6 / HBM_PEAK_GBS, 4)}
    out["decode_sweep_split_plus_combine"] = sweep
    out["verify5_240000"] = {"us": round(v_ms * 1e3, 3), "gbs": round(b / v_ms / 1e6, 2),
                             "hbm_frac": round(b / v_ms / 1e6 / HBM_PEAK_GBS, 4),
                             "kernel": "split kernel alone", "spread": spread_us(v_ts),
                             "us_split_plus_combine": round(vc_ms * 1e3, 3),
                             "hbm_frac_split_plus_combine": round(b / vc_ms / 1e6 / HBM_PEAK_GBS, 4),
                             "n_visible": nv}
    # batched decode: 4 sequences of 59,904 cells (234 pages; their tables
    # are quarters of each 240,000-cell table) in one call, against 4 single
    # calls
    nb, cb = 4, 234 * 256
    pps = (cb + P - 1) // P
    sub = [[tables[p][i * pps:(i + 1) * pps] for i in range(nb)] for p in range(n_pools)]
    qb = synth.queries_device(4, 0, 1, nb, 16, 256, dev)
    wsb = k8.attn_workspace(pools[0], nb, cb)
    ms_b = graph_calls_ms(torch, lambda i: k8.attn_decode_batch(
        pools[i % n_pools], sub[i % n_pools], qb, [cb] * nb, wsb), 2 * n_pools)
    ws1b = k8.attn_workspace(pools[0], 1, cb)

    def four_singles(i):
        for j in range(nb):
            k8.attn_decode(pools[i % n_pools], sub[i % n_pools][j], qb[j], cb, ws1b)
    ms_s = graph_calls_ms(torch, four_singles, 2 * n_pools)
    bb = nb * cb * CELL_BYTES
    out["decode_batch_4x59904"] = {"us": round(ms_b * 1e3, 3), "gbs": round(bb / ms_b / 1e6, 2),
                                   "hbm_frac": round(bb / ms_b / 1e6 / HBM_PEAK_GBS, 4),
                                   "four_single_calls_us": round(ms_s * 1e3, 3)}
    # prefill chunk: 8,192 queries at [231,808, 240,000)
    pos0, n_new = 231808, 8192
    qp = synth.queries_device(5, 0, 0, n_new, 16, 256, dev)
    outp = torch.empty((n_new, 16, 256), dtype=torch.float32, device=dev)
    pws = k8.attn_prefill_workspace(pools[0], pos0 + n_new)
    k8.attn_prefill_chunk(pools[0], tables[0], qp, pos0, out=outp, ws=pws)
    # one call = the staging kernel (each 32-cell tile dequantized once per KV
    # head) and the attention kernel; the timing pair brackets both
    p_ms, p_ts = timed_launches(torch, k8, lambda i: k8.attn_prefill_chunk(
        pools[i % 2], tables[i % 2], qp, pos0, out=outp, ws=pws), 6)
    flops = sum(1024.0 * 16 * (pos0 + i + 1) for i in range(n_new))
    out["prefill_8192_at_231808"] = {"ms": round(p_ms, 3), "tflops": round(flops / p_ms / 1e9, 2),
                                     "mfma_frac": round(flops / p_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                                     "flop": flops, "spread": spread_us(p_ts)}
    # append of one 8,192-token chunk (quantize K, rotate and quantize V,
    # write the three runs): chunk 28 of each pool again, with the values it
    # was filled with, so the pools keep their bytes
    chunks = [synth.kv_chunk_device(4, i, 28, synth.CHUNK, 2, 256, dev) for i in range(n_pools)]
    a_ms, a_ts = timed_launches(torch, k8, lambda i: k8.kv_append_k8v4(
        pools[i % n_pools], tables[i % n_pools], chunks[i % n_pools][0], chunks[i % n_pools][1],
        28 * synth.CHUNK), reps)
    ab = synth.CHUNK * 2 * 256 * 2 * 2 + synth.CHUNK * CELL_BYTES  # fp16 K and V in, the cells out
    out["append_8192_tokens"] = {"us": round(a_ms * 1e3, 3), "bytes": ab, "gbs": round(ab / a_ms / 1e6, 2),
                                 "hbm_frac": round(ab / a_ms / 1e6 / HBM_PEAK_GBS, 4),
                                 "spread": spread_us(a_ts)}
    del chunks
    # the same chunk over the comparison formats (one 240,000-cell pool each)
    fm = {}
    for fmt, name in ((1, "int8"), (2, "q4_0"), (0, "fp16")):
        log(f"extra: prefill chunk over a {name} pool ...")
        pool = k8.KvPool(fmt, n_pages, P, 2, device=dev)
        for c, s in enumerate(range(0, ctx, synth.CHUNK)):
            n = min(synth.CHUNK, ctx - s)
            kk, vv = synth.kv_chunk_device(4, 0, c, n, 2, 256, dev)
            k8.kv_append(pool, tables[0], kk, vv, s)
        k8.attn_prefill_chunk(pool, tables[0], qp, pos0, out=outp, ws=pws)
        f_ms, _ = timed_launches(torch, k8, lambda i: k8.attn_prefill_chunk(
            pool, tables[0], qp, pos0, out=outp, ws=pws), 2)
        fm[name] = {"ms": round(f_ms, 3), "mfma_frac": round(flops / f_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4)}
        del pool
        torch.cuda.empty_cache()
    out["prefill_8192_formats"] = fm
    out["formats_32768"] = bench_formats_32768(torch, k8, synth, dev, log)
    out["decode_240000_fp16"] = bench_fp16_240000(torch, k8, synth, dev, log)
    out["decode_240000_formats"] = bench_formats_240000(torch, k8, synth, dev, log)
    out["decode_stream_240000"] = bench_stream_240000(torch, k8, synth, dev, log)
    out["decode_1048576"] = bench_decode_1m(torch, k8, synth, dev, log)
    out["page_copy_k8v4"] = bench_page_copy(torch, k8, pools[0], tables[0], dev, log)
    log(f"extra: {json.dumps(out)}")
    return out


def bench_page_copy(torch, k8, pool, table, dev, log):
    """The streamed cache's page moves (kv_copy_pages): 128 pages of 256
    cells (26.7 MB of k8v4) between a pinned host mirror and device pools,
    each direction graph-timed."""
    n = 128
    log("extra: page copies between host and device ...")
    host = k8.KvPool(3, pool.n_pages, pool.page_size, pool.n_kv_heads, host=True)
    win = k8.K8V4Pool(n, pool.page_size, pool.n_kv_heads, device=dev)
    src = table[:n].contiguous()
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    b = n * int(k8.lib().kv_cell_bytes(3, pool.n_kv_heads, 256)) * pool.page_size
    d2h = graph_calls_ms(torch, lambda i: k8.kv_copy_pages(host, pool, src, src), 4)
    h2d = graph_calls_ms(torch, lambda i: k8.kv_copy_pages(win, host, slots, src), 4)
    d2d = graph_calls_ms(torch, lambda i: k8.kv_copy_pages(win, pool, slots, src), 4)
    return {"bytes": b, "host_to_device_gbs": round(b / h2d / 1e6, 2),
            "device_to_host_gbs": round(b / d2h / 1e6, 2), "device_to_device_gbs": round(b / d2d / 1e6, 2)}


def bench_formats_32768(torch, k8, synth, dev, log):
    """Decode at 32,768 cells for the four formats on the same raw inputs:
    3 outlier channels per KV head (x8 on K and V), P = 256, 128 pages drawn
    from a 256-page pool, 16 layer pools per format rotated (beyond the
    Infinity Cache).  Whole calls replayed from a graph."""
    ctx, P, n_pages, n_table, layers = 32768, 256, 256, 128, 16
    outl = synth.outlier_channels(2, 2, 256, 0.01)
    q = synth.queries_device(2, 0, 0, 1, 16, 256, dev)[0]
    res = {}
    for fmt, name in ((3, "k8v4"), (1, "int8"), (2, "q4_0"), (0, "fp16")):
        log(f"formats: filling {layers} {name} pools of {ctx} cells ...")
        pools, tables = [], []
        for l in range(layers):
            pool = k8.KvPool(fmt, n_pages, P, 2, device=dev)
            pt = make_table(torch, synth, 2, l, n_table, n_pages, dev)
            for c, s in enumerate(range(0, ctx, synth.CHUNK)):
                n = min(synth.CHUNK, ctx - s)
                kk, vv = synth.kv_chunk_device(2, l, c, n, 2, 256, dev, outliers=outl)
                k8.kv_append(pool, pt, kk, vv, s)
            pools.append(pool)
            tables.append(pt)
        ws = k8.attn_workspace(pools[0], 1, ctx)
        ms = graph_calls_ms(torch, lambda i: k8.attn_decode(pools[i % layers], tables[i % layers], q, ctx, ws),
                            layers)
        cell = int(k8.lib().kv_cell_bytes(fmt, 2, 256))
        b = ctx * cell
        res[name] = {"us": round(ms * 1e3, 2), "mb_per_step": round(b / 1e6, 2),
                     "gbs": round(b / ms / 1e6, 1), "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
                     "cell_bytes": cell}
        del pools, tables
        torch.cuda.empty_cache()
    return res


def bench_stream_240000(torch, k8, synth, dev, log):
    """The streamed cache at 240,000 cells: a pinned host mirror holding every
    page and a device window of the newest 128 pages (32,768 cells); the
    streamed decode reads the window where a page is resident and the mirror
    across the host link where not (whole call: the lookup kernel, the split
    kernel and the combine, replayed from a graph).  Also a window of every
    page (no misses): the streamed path's own cost against the resident
    decode."""
    ctx, P, n_mirror = 240000, 256, 1024
    n_table = (ctx + P - 1) // P
    mt = make_table(torch, synth, 4, 0, n_table, n_mirror, dev)
    q = synth.queries_device(4, 0, 0, 1, 16, 256, dev)[0]
    res = {}
    for n_window in (128, n_mirror):
        log(f"extra: streamed cache, window of {n_window} pages ...")
        s = k8.KvStream(3, n_window, n_mirror, P, mt, fill=0)
        for c, st in enumerate(range(0, ctx, synth.CHUNK)):
            kk, vv = synth.kv_chunk_device(4, 0, c, min(synth.CHUNK, ctx - st), 2, 256, dev)
            k8.kv_stream_append(s, kk, vv, st)
        first = max(0, n_table - n_window)
        k8.kv_stream_fetch(s, first, n_table - first)
        ws = k8.attn_workspace(s.window, 1, ctx)
        k8.attn_decode_stream(s, q, ctx, ws)
        torch.cuda.synchronize()
        s.stats.zero_()
        reps = 4 if n_window < n_table else 16
        ms = graph_calls_ms(torch, lambda i: k8.attn_decode_stream(s, q, ctx, ws), reps, replays=2)
        lookups, misses = (x / (3 * reps) for x in s.stats.cpu().tolist())  # a warm-up and 2 timed replays
        miss_bytes = misses * P * CELL_BYTES
        res[f"window_{n_window}_pages"] = {
            "us": round(ms * 1e3, 3), "lookups_per_call": lookups, "misses_per_call": misses,
            "missed_bytes_per_call": int(miss_bytes),
            "host_link_gbs_missed": round(miss_bytes / ms / 1e6, 2) if misses else None}
        del s
        torch.cuda.empty_cache()
    return res


def bench_formats_240000(torch, k8, synth, dev, log):
    """Decode at 240,000 cells over the int8 and q4_0 comparison formats (4
    pools each, rotated beyond the Infinity Cache), timed like the k8v4
    decode: split kernel alone (events) and the whole call (graph)."""
    ctx, P, n_pages, n_pools = 240000, 256, 1024, 4
    q = synth.queries_device(4, 0, 0, 1, 16, 256, dev)[0]
    res = {}
    for fmt, name in ((1, "int8"), (2, "q4_0")):
        log(f"extra: filling {n_pools} {name} pools of {ctx} cells ...")
        pools, tables = [], []
        for i in range(n_pools):
            pool = k8.KvPool(fmt, n_pages, P, 2, device=dev)
            pt = make_table(torch, synth, 4, i, (ctx + P - 1) // P, n_pages, dev)
            for c, s in enumerate(range(0, ctx, synth.CHUNK)):
                kk, vv = synth.kv_chunk_device(4, i, c, min(synth.CHUNK, ctx - s), 2, 256, dev)
                k8.kv_append(pool, pt, kk, vv, s)
            pools.append(pool)
            tables.append(pt)
        ws = k8.attn_workspace(pools[0], 1, ctx)
        for i in range(n_pools):
            k8.attn_decode(pools[i], tables[i], q, ctx, ws)
        ms, ts = timed_launches(torch, k8, lambda i: k8.attn_decode(
            pools[i % n_pools], tables[i % n_pools], q, ctx, ws), 12 * n_pools)
        wc = graph_calls_ms(torch, lambda i: k8.attn_decode(
            pools[i % n_pools], tables[i % n_pools], q, ctx, ws), 2 * n_pools)
        cell = int(k8.lib().kv_cell_bytes(fmt, 2, 256))
        b = ctx * cell
        res[name] = {"us": round(ms * 1e3, 3), "gbs": round(b / ms / 1e6, 2),
                     "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "spread": spread_us(ts),
                     "us_split_plus_combine": round(wc * 1e3, 3), "cell_bytes": cell,
                     "kernel": "split kernel alone"}
        del pools, tables
        torch.cuda.empty_cache()
    return res


def bench_fp16_240000(torch, k8, synth, dev, log):
    """The no-dequantization reference: decode at 240,000 cells of the fp16
    format (2,048 B/cell, 491.5 MB per pool, 3 pools rotated), split kernel
    alone, timed like the k8v4 decode."""
    ctx, P, n_pages, n_pools = 240000, 256, 1024, 3
    log(f"extra: filling {n_pools} fp16 pools of {ctx} cells ...")
    pools, tables = [], []
    for i in range(n_pools):
        pool = k8.KvPool(0, n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, 4, i, (ctx + P - 1) // P, n_pages, dev)
        for c, s in enumerate(range(0, ctx, synth.CHUNK)):
            n = min(synth.CHUNK, ctx - s)
            kk, vv = synth.kv_chunk_device(4, i, c, n, 2, 256, dev)
            k8.kv_append(pool, pt, kk, vv, s)
        pools.append(pool)
        tables.append(pt)
    q = synth.queries_device(4, 0, 0, 1, 16, 256, dev)[0]
    ws = k8.attn_workspace(pools[0], 1, ctx)
    for i in range(n_pools):
        k8.attn_decode(pools[i], tables[i], q, ctx, ws)
    ms, _ = timed_launches(torch, k8, lambda i: k8.attn_decode(pools[i % n_pools], tables[i % n_pools], q, ctx, ws),
                           8 * n_pools)
    b = ctx * 2048
    del pools, tables
    torch.cuda.empty_cache()
    return {"us": round(ms * 1e3, 3), "gbs": round(b / ms / 1e6, 1), "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
            "cell_bytes": 2048, "kernel": "split kernel alone"}


def bench_decode_1m(torch, k8, synth, dev, log):
    """Decode at 1,048,576 cells (the longest context the pages run k8v4 at),
    2 pools of 856 MB rotated, split kernel alone and whole call."""
    ctx, P, n_pools = 1 << 20, 256, 2
    n_pages = ctx // P
    log(f"extra: filling {n_pools} k8v4 pools of {ctx} cells ...")
    pools, tables = [], []
    for i in range(n_pools):
        pool = k8.K8V4Pool(n_pages, P, 2, device=dev)
        pt = make_table(torch, synth, 6, i, n_pages, n_pages, dev)
        fill_pool(k8, synth, pool, pt, 6, i, ctx, dev)
        pools.append(pool)
        tables.append(pt)
    q = synth.queries_device(6, 0, 0, 1, 16, 256, dev)[0]
    ws = k8.attn_workspace(pools[0], 1, ctx)
    for i in range(n_pools):
        k8.attn_decode(pools[i], tables[i], q, ctx, ws)
    ms, _ = timed_launches(torch, k8, lambda i: k8.attn_decode(pools[i % n_pools], tables[i % n_pools], q, ctx, ws),
                           8 * n_pools)
    wc_ms = graph_calls_ms(torch, lambda i: k8.attn_decode(pools[i % n_pools], tables[i % n_pools], q, ctx, ws),
                           2 * n_pools)
    b = ctx * CELL_BYTES
    del pools, tables
    torch.cuda.empty_cache()
    return {"us": round(ms * 1e3, 3), "gbs": round(b / ms / 1e6, 1), "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
            "kernel": "split kernel alone", "us_split_plus_combine": round(wc_ms * 1e3, 3),
            "hbm_frac_split_plus_combine": round(b / wc_ms / 1e6 / HBM_PEAK_GBS, 4)}


if __name__ == "__main__":
    main()
