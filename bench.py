"""Benchmark: sparse decode steps/s (all layers) at 196k context, top-2048.

Workload c3 (synthetic): 12 sparse-attention layers, batch 1, 32 query heads
/ 4 KV heads, head_dim 128, 64-token pages, context 196,608 tokens (3,072
pages per layer), top-32 pages (2,048 tokens), fp8 e4m3 KV with per-token
fp32 scales, a 256-slot GPU pool over a pinned host mirror, log-Zipf(1.1)
page bias, AR(1) queries.  One step = decode_layer for all 12 layers
(indexer + compact + LRU ensure, fused host->device fetch of the missed pages
across all layers, sparse paged attention).

Timing: W untimed steps, then K steps bracketed by synchronize + HIP events
on the stream the kernels run on.  A separate measurement pass then times
the fetch and attention kernels one launch at a time with HIP events for the
roofline figures.  The oracle (CPU) is timed on a bounded sample of the same
workload as the cpu_baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LINK_PEAK_GBPS = 63.0   # PCIe Gen5 x16: 32 GT/s * 16 lanes * 128/130 / 8, per direction


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--measure-steps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=3)
    return ap.parse_args()


def calibrate(torch):
    """Pinned host->device memcpy and device copy ceilings (context only)."""
    n = 256 << 20
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(n, dtype=torch.uint8, device="cuda")
    d2 = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        d.copy_(h, non_blocking=True)
        d2.copy_(d)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        d.copy_(h, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d = 5 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record()
    for _ in range(5):
        d2.copy_(d)
    e1.record()
    torch.cuda.synchronize()
    d2d = 5 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del h, d, d2
    return dict(h2d_memcpy_GBps=round(h2d, 1), d2d_copy_GBps=round(d2d, 1))


def measure_kernels(torch, g, start_step, nsteps):
    """Run `nsteps` decode steps through the unfused entry points with HIP
    events around every fetch and attention launch (same stream)."""
    wl, t = g.wl, g.tier
    rs = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = []
    c0 = t.read_counters()
    for s in range(start_step, start_step + nsteps):
        for layer in range(wl.num_layers):
            q = g.q[s % g.q.shape[0], layer]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            e[0].record(stream)
            t.select_pages(layer, q, rs, g.bt, g.n_pages, wl.topk, g.sel[layer], g.needed[layer],
                           page_bias=g.bias)
            t.lru_ensure(g.needed[layer].view(-1), g.out_slots[layer], g.miss[layer], g.miss_count[layer])
            e[1].record(stream)
            t.fetch_pages(g.miss[layer], g.miss_count[layer])
            e[2].record(stream)
            t.sparse_paged_attn(layer, q, rs, g.ctx_len, g.sel[layer], g.bt, g.out[layer])
            e[3].record(stream)
            ev.append(e)
    torch.cuda.synchronize()
    c1 = t.read_counters()
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in ev)
    fetch_ms = sum(e[1].elapsed_time(e[2]) for e in ev)
    attn_ms = sum(e[2].elapsed_time(e[3]) for e in ev)
    n = len(ev)
    fetched = c1["bytes_fetched"] - c0["bytes_fetched"]
    misses = c1["misses"] - c0["misses"]
    # algorithmic bytes
    lay = t.layer_bytes
    qo = 2 * wl.batch * wl.num_q_heads * wl.head_dim * 2
    attn_bytes = wl.batch * wl.topk * lay + qo
    slab_bytes = int(g.npg_np.sum()) * wl.num_kv_heads * wl.head_dim * 2 + qo // 2
    return dict(
        launches=n,
        select_ensure_us=1e3 * sel_ms / n,
        fetch_us=1e3 * fetch_ms / n,
        attn_us=1e3 * attn_ms / n,
        fetch_bytes_per_launch=fetched / n,
        misses_per_step=misses / nsteps,
        fetch_GBps=fetched / (fetch_ms * 1e-3) / 1e9 if fetch_ms > 0 else 0.0,
        attn_bytes_per_launch=attn_bytes,
        attn_GBps=attn_bytes * n / (attn_ms * 1e-3) / 1e9,
        select_bytes_per_launch=slab_bytes,
        select_ensure_GBps=slab_bytes * n / (sel_ms * 1e-3) / 1e9,
    )


def cpu_baseline(wl, nsteps):
    """The oracle, as written, on a bounded sample: its setup (slab of every
    page) is untimed; then `nsteps` full decode steps (12 layers: select,
    compact, LRU, fetch copy, fp64 attention).  Rebuilding page bytes from the
    input generator (the lazy mirror) is input generation and is excluded."""
    import numpy as np

    from oracle import run
    from workload import gen

    t0 = time.perf_counter()
    tier = run.make_tier(wl, materialize=False)
    run.setup(wl, tier)
    setup_s = time.perf_counter() - t0
    builder = tier.row_builder
    spent = [0.0]

    def timed_builder(page):
        a = time.perf_counter()
        r = builder(page)
        spent[0] += time.perf_counter() - a
        return r

    tier.row_builder = timed_builder
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    q = gen.decode_queries(wl)
    rs = np.arange(wl.batch + 1)
    tier.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for s in range(nsteps):
            for layer in range(wl.num_layers):
                tier.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
        wall = time.perf_counter() - t0
    work = wall - spent[0]
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    return dict(value=round(nsteps / work, 3), unit="steps/s", cores=1, kind="oracle",
                sample=(f"first {nsteps} decode steps of {wl.name} (all {wl.num_layers} layers: "
                        f"select, compact, LRU ensure, fetch, fp64 attention), NumPy with BLAS limited to 1 thread; "
                        f"untimed: setup {setup_s:.1f}s, lazy page-row rebuild {spent[0]:.1f}s; "
                        f"host has {cores} cores"))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by request, one tier per GPU, with no exchange)", file=sys.stderr)
        sys.exit(2)
    import dataclasses

    import torch

    from workload import get_workload
    from workload.gpu_run import GpuWorkload

    base = get_workload(args.config)
    total = args.warmup + args.steps + args.measure_steps
    wl = dataclasses.replace(base, steps=max(base.steps, total))
    torch.cuda.set_device(0)
    calib = calibrate(torch)
    log(f"[bench] calibration {calib}")
    t0 = time.perf_counter()
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f}s ({wl.name})")
    stream = torch.cuda.current_stream()
    for s in range(args.warmup):
        g.decode_step(s)
    torch.cuda.synchronize()
    c0 = g.tier.read_counters()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(args.warmup, args.warmup + args.steps):
        g.decode_step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    c1 = g.tier.read_counters()
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step")
    k = measure_kernels(torch, g, args.warmup + args.steps, args.measure_steps)
    log(f"[bench] kernels {k}")
    misses_step = (c1["misses"] - c0["misses"]) / args.steps
    link_bytes_step = (c1["bytes_fetched"] - c0["bytes_fetched"]) / args.steps
    err = c1["error_word"]
    fetch_share = k["fetch_us"] * wl.num_layers / (ms * 1e3)
    result = {
        "metric": "sparse decode steps/s (all layers) at 196k ctx, top-2048; achieved HBM GB/s",
        "value": round(1e3 / ms, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 KV, bf16 q/out, fp32 math",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.num_layers, "batch": wl.batch,
                   "context_tokens": list(wl.contexts), "topk_pages": wl.topk,
                   "budget_tokens": wl.topk * wl.page_size, "page_size": wl.page_size,
                   "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "pool_slots": wl.num_slots, "kv_format": wl.kv_format},
        "roofline": {"kernel": "k_fetch (fused host->device page copy)", "bound": "host_link",
                     "achieved": round(k["fetch_GBps"], 2), "peak": LINK_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k["fetch_GBps"] / LINK_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": round(k["fetch_bytes_per_launch"]),
                     "avg_launch_us": round(k["fetch_us"], 2), "step_time_share": round(fetch_share, 3)},
        "roofline_hbm": {"kernel": "k_attn (sparse paged attention)", "bound": "hbm",
                         "achieved": round(k["attn_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(k["attn_GBps"] / HBM_PEAK_GBPS, 4), "traffic": None,
                         "bytes_per_launch": k["attn_bytes_per_launch"],
                         "avg_launch_us": round(k["attn_us"], 2)},
        "select_ensure": {"avg_us": round(k["select_ensure_us"], 2),
                          "slab_GBps": round(k["select_ensure_GBps"], 1)},
        "link": {"misses_per_step": round(misses_step, 1),
                 "bytes_per_step": round(link_bytes_step),
                 "step_GBps": round(link_bytes_step / (ms * 1e-3) / 1e9, 2)},
        "calibration": calib,
        "error_word": err,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(base, args.cpu_steps)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
