"""Benchmark: sparse decode steps/s (all layers) at 196k context, top-2048.

Headline workload c3 (synthetic): 12 sparse-attention layers, batch 1, 32
query heads / 4 KV heads, head_dim 128, 64-token pages, context 196,608
tokens (3,072 pages per layer), top-32 pages (2,048 tokens), fp8 e4m3 KV with
per-token fp32 scales, a 256-slot GPU pool over a pinned host mirror,
log-Zipf(1.1) page bias, AR(1) queries.  One step = one decode call for each
of the 12 layers (indexer + compact + LRU ensure, fused host->device copy of
the missed pages across all layers, sparse paged attention).  When the warmup
steps miss pages, the calls are decode_layer_split: each miss's slices of the
decoded layer and the next one are copied on the decode stream, the rest of
its row on a second stream, beside the attention and the next layer's
selection; otherwise decode_layer (one stream).

Timing: W untimed steps, then K steps bracketed by synchronize + HIP events
on the decode stream (the copy stream joined before the closing event).
Separate passes then time, with HIP events, every rest-of-rows copy on the
copy stream, and select+ensure, the whole-row copy and the attention one
launch at a time.

The same JSON line carries, under "configs", the other four workloads (c1
tiny bf16, c2 64k resident, c4 batch-4 mixed, c5 prefill chunk), each with
its own steps (the same W and K), roofline and CPU baseline, and cold-pool
figures for c3 (a step from an empty pool) and c5 (a chunk from an empty
pool: the bulk fetch of the cached context).  The oracle (CPU) is timed in a
child process started before this process touches the GPU, on its own
cores, on a bounded sample of each workload: the first steps of the same
timed window the GPU measured.
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
ATTN_MFMA_PEAK = 3333.3  # TFLOP/s: fp8 Q.K^T (5.0 PFLOP/s) and bf16 P.V (2.5) in equal parts
LINK_PEAK_GBPS = 63.0   # PCIe Gen5 x16: 32 GT/s * 16 lanes * 128/130 / 8, per direction


def fetch_traffic():
    """Bytes per k_fetch launch from the committed PMC summary (FETCH_SIZE and
    WRITE_SIZE scaled by the calibration copy), or None when the fetch kernel
    has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "c3_pmc_traffic.json")
    src = os.path.join(ROOT, "tiered_kv_cache_indexer_amd", "csrc", "tkv_fetch.hip")
    try:
        rec = json.load(open(path))["k_fetch"]
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except Exception:
        return None, None
    if rec.get("source_sha256_16") != sha:
        return None, None
    return round(rec["fetch_KiB"] * 1024), round(rec["write_KiB"] * 1024)


def pmc_traffic(summary, kernel, source):
    """Bytes per launch of `kernel` past L2 (FETCH_SIZE and WRITE_SIZE scaled
    by the calibration copy) from a committed PMC summary, or None when the
    kernel's source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    src = os.path.join(ROOT, "tiered_kv_cache_indexer_amd", "csrc", source)
    try:
        doc = json.load(open(path))
        rec = doc[kernel]
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except Exception:
        return None
    if rec.get("source_sha256_16") != sha:
        return None
    return round((rec["fetch_KiB"] * doc.get("fetch_scale", 2.0) + rec["write_KiB"] * doc.get("write_scale", 1.0))
                 * 1024)


def split_traffic(misses_per_call):
    """HBM-side bytes of one split copy (k_fetch_slice + k_fetch_rest) from the
    committed PMC summary, scaled to `misses_per_call` misses, or None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "c3_pmc_traffic.json")
    src = os.path.join(ROOT, "tiered_kv_cache_indexer_amd", "csrc", "tkv_fetch.hip")
    try:
        doc = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        parts = [doc["k_fetch_slice"], doc["k_fetch_rest"]]
    except Exception:
        return None
    if any(p.get("source_sha256_16") != sha or not p.get("misses_per_launch") for p in parts):
        return None
    b = sum((p["fetch_KiB"] * doc["fetch_scale"] + p["write_KiB"] * doc["write_scale"]) * 1024
            / p["misses_per_launch"] for p in parts)
    return round(b * misses_per_call)


def prefill_attn_traffic():
    return pmc_traffic("c5_pmc_traffic.json", "k_attn_mfma_rows", "tkv_attn_mfma.hip")


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
    ap.add_argument("--graph", action="store_true", help="replay each decode step as a captured HIP graph")
    ap.add_argument("--decode", choices=["auto", "split", "plain"], default="auto",
                    help="split: decode_layer_split (each miss's other layers copied on a second stream); "
                         "plain: decode_layer; auto: split when the warmup steps missed pages")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the preload, host-tail, prefix and append figures (profiling runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the --config workload: no other configs, no cold-pool figures")
    ap.add_argument("--cpu-deadline", type=float, default=480.0,
                    help="seconds from the start after which unfinished CPU baselines are dropped")
    ap.add_argument("--cpu-baseline-child", default=None, help=argparse.SUPPRESS)
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
    # a plain elementwise kernel of known size (reads n bytes, writes n bytes):
    # the reference the HBM byte counters of a profiled run are scaled by
    x = d.view(torch.float32)
    y = d2.view(torch.float32)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    del h, d, d2
    return dict(h2d_memcpy_GBps=round(h2d, 1), d2d_copy_GBps=round(d2d, 1))


def measure_kernels(torch, g, start_step, nsteps):
    """Run `nsteps` decode steps through the unfused entry points with HIP
    events around every select+ensure, fetch and attention launch (same
    stream, launched back to back).  Durations are the median over the
    launches: now and then one window reads 0.7-1.4 ms where the others read
    30 us (whether the queue runs full or drains between layers), and the
    mean would be that outlier's."""
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
    import numpy as np
    n = len(ev)
    sel_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * n
    fetch_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * n
    attn_ms = float(np.median([e[2].elapsed_time(e[3]) for e in ev])) * n
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


# ------------------------------------------------------------ CPU baseline --
# The oracle, as written, timed on this host in a child process (started
# before the parent touches the GPU and pinned to cores the parent does not
# use).  Decode workloads: untimed setup and untimed steps 0..W-1, then the
# first n of the GPU's timed steps W..W+K-1, all layers (select, compact,
# LRU ensure, fetch copy, fp64 attention).  Rebuilding page rows from the
# input generator (the oracle's lazy mirror) is input generation and is
# subtracted.  Prefill: the chunk's store, selection, ensure and fetch for all
# rows and layers, attention for a stated sample of rows, scaled to the chunk.

CPU_SAMPLE_STEPS = {"c1": 20, "c2": 6, "c3": 4, "c4": 2}
CPU_PREFILL_ROWS = 128


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_decode_baseline(key, warmup, steps):
    import dataclasses

    import numpy as np

    from oracle import run
    from workload import gen, get_workload

    base = get_workload(key)
    n = min(steps, CPU_SAMPLE_STEPS.get(key, 3))
    wl = dataclasses.replace(base, steps=max(base.steps, warmup + steps))
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

    def step(s):
        for layer in range(wl.num_layers):
            tier.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)

    a = time.perf_counter()
    for s in range(warmup):
        step(s)
    warm_s = time.perf_counter() - a
    spent[0] = 0.0
    a = time.perf_counter()
    for s in range(warmup, warmup + n):
        step(s)
    wall = time.perf_counter() - a
    work = wall - spent[0]
    threads = _oracle_threads()
    return dict(value=round(n / work, 3), unit="steps/s", cores=threads, kind="oracle",
                sample=(f"decode steps {warmup}..{warmup + n - 1} of {wl.name} (the first {n} of the GPU's "
                        f"timed steps {warmup}..{warmup + steps - 1}), all {wl.num_layers} layers: select, "
                        f"compact, LRU ensure, fetch copy, fp64 attention; timed {work:.2f}s; untimed: setup "
                        f"{setup_s:.1f}s, steps 0..{warmup - 1} {warm_s:.1f}s, page-row rebuild from the input "
                        f"generator {spent[0]:.1f}s; NumPy with BLAS on {threads} threads (the step loop is "
                        f"single-threaded Python)"),
                max_score_bits=round(float(tier.max_score_bits), 2),
                max_score_abs_sum=round(float(tier.max_certificate), 3))


def cpu_prefill_baseline(key):
    import numpy as np

    from oracle import run
    from workload import get_workload

    wl = get_workload(key)
    t0 = time.perf_counter()
    tier = run.make_tier(wl, materialize=False)
    run.setup(wl, tier)
    setup_s = time.perf_counter() - t0
    n = wl.prefill_tokens
    rows = list(range(0, n, max(1, n // CPU_PREFILL_ROWS)))
    spent = {"rebuild": 0.0, "attn": 0.0}
    builder, attend_row = tier.row_builder, tier.attention_row

    def timed_builder(page):
        a = time.perf_counter()
        r = builder(page)
        spent["rebuild"] += time.perf_counter() - a
        return r

    def timed_attention_row(*args, **kw):
        a = time.perf_counter()
        r0 = spent["rebuild"]
        out = attend_row(*args, **kw)
        spent["attn"] += time.perf_counter() - a - (spent["rebuild"] - r0)
        return out

    tier.row_builder = timed_builder
    tier.attention_row = timed_attention_row
    a = time.perf_counter()
    run.prefill(wl, tier, attention_rows=rows)
    wall = time.perf_counter() - a
    base_s = wall - spent["rebuild"] - spent["attn"]
    est = base_s + spent["attn"] * n / len(rows)
    threads = _oracle_threads()
    return dict(value=round(n / est, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=(f"{wl.name}: the {n}-token chunk's store, selection (all rows), ensure and fetch for all "
                        f"{wl.num_layers} layers ({base_s:.1f}s), attention for {len(rows)} of the {n} rows of "
                        f"every layer (every {n // len(rows)}th, {spent['attn']:.1f}s), scaled to the chunk: "
                        f"{est:.1f}s; untimed: setup {setup_s:.1f}s, page-row rebuild {spent['rebuild']:.1f}s; "
                        f"NumPy with BLAS on {threads} threads"),
                max_score_bits=round(float(tier.max_score_bits), 2),
                max_score_abs_sum=round(float(tier.max_certificate), 3))


def cpu_child_main(spec_path):
    """Child process: run the CPU baselines the spec lists, in order, writing
    the results file after each (so a parent that stops waiting keeps what
    finished)."""
    spec = json.load(open(spec_path))
    sys.stdin.readline()          # the parent says "go" once its GPU measurements are done
    cores = spec.get("cores")
    if cores:
        os.sched_setaffinity(0, cores)
    from threadpoolctl import threadpool_limits
    out = {}
    with threadpool_limits(limits=max(1, len(cores) if cores else os.cpu_count())):
        for item in spec["runs"]:
            key = item["key"]
            t0 = time.perf_counter()
            try:
                if item.get("prefill"):
                    out[key] = cpu_prefill_baseline(key)
                else:
                    out[key] = cpu_decode_baseline(key, item["warmup"], item["steps"])
            except Exception as e:   # reported, never silently dropped
                out[key] = {"error": f"{type(e).__name__}: {e}"}
            out[key]["wall_s"] = round(time.perf_counter() - t0, 1)
            tmp = spec["out"] + ".tmp"
            json.dump(out, open(tmp, "w"))
            os.replace(tmp, spec["out"])
            print(f"[cpu] {key} done in {out[key]['wall_s']}s", file=sys.stderr, flush=True)


def start_cpu_child(args, keys):
    """Starts the CPU-baseline child process before this process uses the GPU
    (it waits for go_cpu_child, so the oracle never shares the host with the
    GPU measurements: a busy host slowed the launch-bound passes up to 20x).
    Returns (process, results path, start time) or None."""
    import subprocess
    import tempfile
    try:
        cores = sorted(os.sched_getaffinity(0))
    except Exception:
        cores = list(range(os.cpu_count() or 1))
    d = tempfile.mkdtemp(prefix="tkv_cpu_")
    spec = {"out": os.path.join(d, "cpu.json"), "cores": cores,
            "runs": [{"key": k, "warmup": args.warmup, "steps": args.steps, "prefill": k == "c5"} for k in keys]}
    spec_path = os.path.join(d, "spec.json")
    json.dump(spec, open(spec_path, "w"))
    proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", spec_path],
                            stdin=subprocess.PIPE, stdout=subprocess.DEVNULL, stderr=sys.stderr, text=True)
    return proc, spec["out"], time.perf_counter()


def go_cpu_child(child):
    if child is not None:
        child[0].stdin.write("go\n")
        child[0].stdin.flush()


def collect_cpu_child(child, t_start, deadline):
    """Waits for the child until `deadline` seconds after the bench started;
    then stops it (its own PID) and returns whatever finished."""
    if child is None:
        return {}
    proc, path, _ = child
    go_cpu_child(child)
    try:
        proc.wait(timeout=max(1.0, deadline - (time.perf_counter() - t_start)))
    except Exception:
        log("[bench] CPU baselines past the deadline: stopping the child")
        proc.kill()
        proc.wait()
    try:
        return json.load(open(path))
    except Exception:
        return {}


def bench_append(torch, key, steps, warmup):
    """Decode steps that append one token per request (write-ensure + store
    with write-through + fused decode layer, per layer) on a fresh tier of the
    appending variant of the workload.  New tokens' K/V are generated before
    the timed region."""
    import dataclasses

    from workload import get_workload
    from workload.gpu_run import GpuWorkload
    wl = dataclasses.replace(get_workload(key), steps=warmup + steps)
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    kv = g.append_kv()
    for s in range(warmup):
        g.decode_step_append(s, kv)
    torch.cuda.synchronize()
    c0 = g.tier.read_counters()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(warmup, warmup + steps):
        g.decode_step_append(s, kv)
    e1.record(stream)
    torch.cuda.synchronize()
    c1 = g.tier.read_counters()
    ms = e0.elapsed_time(e1) / steps
    out = {"workload": wl.name, "ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 2),
           "misses_per_step": round((c1["misses"] - c0["misses"]) / steps, 1),
           "fresh_allocs": c1["fresh_allocs"] - c0["fresh_allocs"],
           "mirrored_bytes_per_step": round((c1["bytes_mirrored"] - c0["bytes_mirrored"]) / steps),
           "error_word": c1["error_word"],
           "note": "per layer: ensure_write_pages + store_kv_mirror (1 token/request) + decode_layer"}
    del g
    torch.cuda.empty_cache()
    return out


def bench_prefetch(torch, g, s0, steps, base_ms, base_misses, link_util):
    """Decode steps with the top-k preload: layer l preloads the page list
    layer l+1 needed last time, its copy on a second stream under layer l's
    selection (tkv_decode_layer_prefetch).  Continues from the tier state the
    fetch path left.  Also the gate the runner applies: the preload is used
    only when the link has idle time (the timed steps moved less than 0.85
    of the measured pinned-copy ceiling), it does not add link bytes (misses
    per step with it at most 2% above those without) and its timed steps ran
    faster than those without it; otherwise the steps run without it, at the
    speed of the path the workload's own figure uses."""
    wl, t = g.wl, g.tier
    n_q = g.q.shape[0]
    side = torch.cuda.Stream()
    for i in range(2):
        g.decode_step_prefetch((s0 + i) % n_q, side)
    torch.cuda.synchronize()
    c0 = t.read_counters()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        g.decode_step_prefetch((s0 + 2 + i) % n_q, side)
    e1.record(stream)
    torch.cuda.synchronize()
    c1 = t.read_counters()
    ms = e0.elapsed_time(e1) / steps
    # how good the prediction is: share of a layer's needed pages that were in
    # its needed list of the step before (untimed extra steps)
    import numpy as np
    prev = g.needed.cpu().numpy()
    shares = []
    for i in range(4):
        g.decode_step_prefetch((s0 + 2 + steps + i) % n_q, side)
        cur = g.needed.cpu().numpy()
        for layer in range(wl.num_layers):
            a = set(cur[layer].ravel().tolist()) - {-1}
            b = set(prev[layer].ravel().tolist()) - {-1}
            if a:
                shares.append(len(a & b) / len(a))
        prev = cur
    misses = (c1["misses"] - c0["misses"]) / steps
    enabled = link_util < 0.85 and misses <= 1.02 * base_misses and ms < base_ms
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 2),
            "misses_per_step": round(misses, 1),
            "link_bytes_per_step": round((c1["bytes_fetched"] - c0["bytes_fetched"]) / steps),
            "prediction_hit_share": round(float(np.mean(shares)), 3),
            "note": "misses include the preloads'; prediction = the next layer's last needed list",
            "gated": {"link_util": round(link_util, 3), "misses_per_step_without": round(base_misses, 1),
                      "enabled": bool(enabled),
                      "ms_per_step": round(ms if enabled else base_ms, 4),
                      "steps_per_s": round(1e3 / (ms if enabled else base_ms), 2),
                      "rule": "preload only when the link moved < 0.85 of the pinned-copy ceiling, the preload "
                              "adds at most 2% misses and its steps ran faster; else the steps run without it"}}


def bench_prefix(g, n):
    """Cold-prefix records of n pages of request 0 (n = 375: a 24k-token
    prefix) saved and restored in place: rows host to host, slab entries
    over the link.  Wall time of each call (both synchronise)."""
    t = g.tier
    pages = g.bt_np[0, :n]
    t.prefix_save(pages)                                    # warm the threads and the staging path
    a = time.perf_counter()
    recs = t.prefix_save(pages)
    b = time.perf_counter()
    t.prefix_restore(pages, recs)
    c = time.perf_counter()
    row_bytes = n * t.row_bytes
    return {"pages": n, "record_bytes": int(recs.nbytes), "save_ms": round((b - a) * 1e3, 2),
            "restore_ms": round((c - b) * 1e3, 2),
            "save_rows_GBps": round(row_bytes / (b - a) / 1e9, 2),
            "restore_rows_GBps": round(row_bytes / (c - b) / 1e9, 2),
            "note": "rows host to host (8 threads), slab entries via the GPU in 128-page slices"}


def bench_host_tail(torch, g, s0, steps):
    """Decode steps with the host tail read in place (tkv_select_pages +
    tkv_sparse_paged_attn_host_tail per layer; no ensure, no fetch), on the
    pool as the fetch path left it.  Host bytes per step = selected pages that
    are not resident x one layer's block of the row."""
    import numpy as np
    wl, t = g.wl, g.tier
    n_q = g.q.shape[0]
    for i in range(2):
        g.decode_step_host_tail((s0 + i) % n_q)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        g.decode_step_host_tail((s0 + 2 + i) % n_q)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    p2s = t.read_state()["page_to_slot"]
    sel = g.sel.cpu().numpy()
    bt = g.bt_np
    host_pages = 0
    for layer in range(wl.num_layers):
        for b in range(wl.batch):
            for i in sel[layer, b]:
                if i >= 0 and p2s[bt[b][i]] < 0:
                    host_pages += 1
    host_bytes = host_pages * t.layer_bytes
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 2),
            "host_pages_last_step": host_pages, "host_bytes_last_step": host_bytes,
            "host_read_GBps_lower_bound": round(host_bytes / (ms * 1e-3) / 1e9, 2),
            "note": "select_pages + sparse_paged_attn_host_tail per layer (no ensure, no fetch); "
                    "pool as the fetch path left it; GB/s = last step's host bytes / mean step time"}


def bench_prefill(torch, key, warmup, steps, cold_reps=0, split_store=True):
    """c5: one 4,096-token prefill chunk over 65,536 cached tokens, 12 layers:
    write-ensure, then per layer store (write-through) -> select (matrix-core
    indexer, causal per-query top-32) -> ensure -> fetch -> causal sparse
    attention.  Keys, values and queries are generated on the GPU before the
    timed region; the tier is reset and the context rewritten (untimed)
    before every repetition.  With `cold_reps`, that many more repetitions
    start from an empty pool (residency reset after the context is written):
    layer 0's ensure then misses the cached pages its rows select and its
    fetch moves them all over the host link.  `split_store` (the default):
    the stores through tkv_store_kv_mirror_split (the pool written on the
    chunk's stream, the mirror writes of whole pages deferred to a second
    stream beside the layer's attention); else tkv_store_kv_mirror (pool and
    mirror written by the store kernel)."""
    import numpy as np

    from workload import gen, get_workload, gpu_gen
    from workload.gpu_run import GpuWorkload

    wl = get_workload(key)
    L, n, start = wl.num_layers, wl.prefill_tokens, wl.contexts[0]
    g = GpuWorkload(wl)
    t = g.tier
    bufs = g.prefill_buffers()
    K = torch.empty((L, n, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    Q = torch.empty((L, n, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    for layer in range(L):
        gpu_gen.tokens(wl, gen.KIND_K, layer, 0, start, n, out=K[layer])
        gpu_gen.tokens(wl, gen.KIND_V, layer, 0, start, n, out=V[layer])
        gpu_gen.tokens(wl, gen.KIND_Q, layer, 0, 0, n, out=Q[layer])
    run_req = torch.tensor([0], dtype=torch.int32, device="cuda")
    run_start = torch.tensor([start], dtype=torch.int32, device="cuda")
    run_len = torch.tensor([n], dtype=torch.int32, device="cuda")
    run_off = torch.zeros(1, dtype=torch.int32, device="cuda")
    old_len = torch.tensor([start], dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    names = ("store", "select", "ensure", "fetch", "attn")
    reps, colds, copy_ms, totals = [], [], [], []
    # timed repetitions carry events at the chunk's ends only (an event
    # between two launches costs the stream a few microseconds); then as
    # many repetitions with events around every phase give the split
    n_timed = warmup + steps
    for rep in range(n_timed + steps + cold_reps):
        cold = rep >= n_timed + steps
        phases = rep >= n_timed and not cold
        t.reset_residency()
        t.set_select_width(1, wl.topk, 2 * wl.topk + 8)
        g.setup()
        if cold:
            t.reset_residency()
        torch.cuda.synchronize()
        t.set_select_width(1, wl.topk, wl.max_sel_pages)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 + 5 * L)]   # the last: chunk end
        evc = [torch.cuda.Event(enable_timing=True) for _ in range(L)]
        ev[0].record(stream)
        t.ensure_write_pages(run_req, run_start, run_len, n, g.bt, old_len)
        if phases or cold:
            ev[1].record(stream)
        for layer in range(L):
            e = ev[2 + 5 * layer: 7 + 5 * layer]
            t.store_kv_mirror(layer, K[layer], V[layer], run_req, run_start, run_len, run_off, n, g.bt,
                              copy_stream=side if split_store else None)
            if phases or cold:
                e[0].record(stream)
            t.select_pages(layer, Q[layer], bufs["row_start"], g.bt, g.n_pages, wl.topk, bufs["sel"],
                           bufs["needed"], row_pos=bufs["row_pos"])
            if phases:
                e[1].record(stream)
            t.lru_ensure(bufs["needed"].view(-1), bufs["out_slots"], bufs["miss"], bufs["miss_count"])
            if phases or cold:
                e[2].record(stream)
            t.fetch_pages(bufs["miss"], bufs["miss_count"])
            if phases or cold:
                e[3].record(stream)
            t.sparse_paged_attn(layer, Q[layer], bufs["row_start"], bufs["ctx_len"], bufs["sel"], g.bt,
                                bufs["out"], row_pos=bufs["row_pos"])
            if phases:
                e[4].record(stream)
                evc[layer].record(side)               # after this layer's mirror copy (enqueued beside the attention)
        stream.wait_stream(side)
        ev[-1].record(stream)
        torch.cuda.synchronize()
        if warmup <= rep < n_timed:
            totals.append(ev[0].elapsed_time(ev[-1]))
            continue
        if cold:
            c = t.read_counters()
            e = ev[2:7]
            fetch0 = e[2].elapsed_time(e[3])
            colds.append(dict(total_ms=ev[0].elapsed_time(ev[-1]), layer0_fetch_ms=fetch0,
                              misses=c["misses"], bytes_fetched=c["bytes_fetched"]))
            continue
        if rep < n_timed:
            continue
        split = dict(write_ensure=ev[0].elapsed_time(ev[1]))
        for i, nm in enumerate(names):
            split[nm] = 0.0
        for layer in range(L):
            prev = ev[1] if layer == 0 else ev[1 + 5 * layer]
            e = ev[2 + 5 * layer: 7 + 5 * layer]
            split["store"] += prev.elapsed_time(e[0])
            split["select"] += e[0].elapsed_time(e[1])
            split["ensure"] += e[1].elapsed_time(e[2])
            split["fetch"] += e[2].elapsed_time(e[3])
            split["attn"] += e[3].elapsed_time(e[4])
        split["total"] = ev[0].elapsed_time(ev[-1])
        reps.append(split)
        # each layer's mirror copy starts with its attention
        copy_ms.append(sum(ev[5 + 5 * layer].elapsed_time(evc[layer]) for layer in range(L)))
    ms = {k: float(np.mean([r[k] for r in reps])) for k in reps[0]}
    ms["total_with_phase_events"] = ms["total"]
    ms["total"] = float(np.mean(totals))
    # algorithmic work of the last repetition's last layer, scaled by layers
    sel = bufs["sel"].cpu().numpy()
    pos = bufs["row_pos"].cpu().numpy()
    ctxl = start + n
    toks = 0
    for r in range(n):
        for i in sel[r]:
            if i >= 0:
                toks += max(0, min(wl.page_size, min(ctxl, int(pos[r]) + 1) - int(i) * wl.page_size))
    toks = int(toks)
    attn_flop_layer = toks * wl.num_q_heads * wl.head_dim * 4
    pages_read = int(sum(1 for r in range(n) for i in sel[r]
                         if i >= 0 and int(i) * wl.page_size <= min(ctxl - 1, int(pos[r]))))
    attn_bytes_layer = pages_read * wl.num_kv_heads * (2 * wl.page_size * wl.head_dim + 8 * wl.page_size)
    attn_traffic = prefill_attn_traffic()
    gemm_flop_layer = 2 * n * wl.pages_of(0) * wl.num_kv_heads * wl.head_dim
    tok_bytes = t.layer_bytes // wl.page_size
    c = t.read_counters()
    return {
        "metric": "prefill chunk tokens/s (4,096 new over 65,536 cached, 12 layers)",
        "value": round(n / (ms["total"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms["total"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 KV, bf16 q/out, bf16 MFMA indexer, fp32 math", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "chunk_tokens": n, "cached_tokens": start,
                   "topk_pages": wl.topk, "pool_slots": wl.num_slots},
        "split_ms": {k: round(v, 3) for k, v in ms.items()},
        "roofline": {"kernel": "k_attn_mfma_rows (causal sparse attention, one wave per row and KV head)",
                     "bound": "mfma",
                     "achieved": round(attn_flop_layer * L / (ms["attn"] * 1e-3) / 1e12, 2),
                     "peak": ATTN_MFMA_PEAK, "unit": "TFLOP/s",
                     "frac": round(attn_flop_layer * L / (ms["attn"] * 1e-3) / 1e12 / ATTN_MFMA_PEAK, 4),
                     "traffic": attn_traffic,
                     "flop_per_launch": attn_flop_layer,
                     "peak_note": "half the flops are S = Q.K^T on fp8 (5.0 PFLOP/s), half P.V on bf16 "
                                  "(2.5 PFLOP/s): 3.33 PFLOP/s for the mix",
                     "cache_bytes_per_launch": attn_bytes_layer,
                     "cache_GBps": round(attn_bytes_layer * L / (ms["attn"] * 1e-3) / 1e9, 1),
                     "note": "the kernel reads K+V codes and scales of every (row, KV head, selected page): "
                             "cache_bytes per launch, 123x the layer's unique KV; most come from the L2s and "
                             "the Infinity Cache (traffic: what passed the L2s), and one page in flight per "
                             "wave leaves it bound by that path's latency, not by the matrix cores"},
        "roofline_mfma": {"kernel": "k_prefill_scores (+ per-row top-k, compaction)", "bound": "mfma",
                          "achieved": round(gemm_flop_layer * L / (ms["select"] * 1e-3) / 1e12, 2),
                          "peak": 2500.0, "unit": "TFLOP/s",
                          "frac": round(gemm_flop_layer * L / (ms["select"] * 1e-3) / 1e12 / 2500.0, 5)},
        "mirror_write_GBps": round(n * tok_bytes * L / (float(np.mean(copy_ms) if split_store else ms["store"])
                                                        * 1e-3) / 1e9, 2),
        "store_path": ("tkv_store_kv_mirror_split: split_ms.store is the pool part on the chunk's stream; the "
                       "mirror copy runs on a second stream beside the layer's attention (its time from the "
                       "attention's start: mirror_copy_ms; mirror_write_GBps = mirror bytes / that time)"
                       if split_store else
                       "tkv_store_kv_mirror: pool and mirror written by the store kernel "
                       "(mirror_write_GBps = mirror bytes / store time)"),
        "mirror_copy_ms": round(float(np.mean(copy_ms)), 3) if split_store else None,
        "error_word": c["error_word"],
        "cold_chunk": ({"ms_per_chunk": round(float(np.mean([x["total_ms"] for x in colds])), 3),
                        "tokens_per_s": round(n / (float(np.mean([x["total_ms"] for x in colds])) * 1e-3), 1),
                        "misses": colds[-1]["misses"], "bytes_fetched": colds[-1]["bytes_fetched"],
                        "layer0_fetch_ms": round(float(np.mean([x["layer0_fetch_ms"] for x in colds])), 3),
                        "roofline": {"kernel": "k_fetch (layer 0's fetch of the cached pages, all layers' rows)",
                                     "bound": "host_link",
                                     "achieved": round(colds[-1]["bytes_fetched"] / (float(np.mean(
                                         [x["layer0_fetch_ms"] for x in colds])) * 1e-3) / 1e9, 2),
                                     "peak": LINK_PEAK_GBPS, "unit": "GB/s",
                                     "frac": round(colds[-1]["bytes_fetched"] / (float(np.mean(
                                         [x["layer0_fetch_ms"] for x in colds])) * 1e-3) / 1e9 / LINK_PEAK_GBPS,
                                         4),
                                     "traffic": None},
                        "note": "residency reset after the context is written: the chunk's rows select cached "
                                "pages that are not resident, layer 0's ensure misses them and one fetch moves "
                                "their rows (every layer) host to device"} if colds else None),
        "cpu_baseline": None,
    }


def bench_decode(torch, key, args, headline):
    """Decode steps of workload `key`: W untimed, K timed (HIP events on the
    decode stream), then the per-launch passes.  Returns (result, workload
    runner, split flag, copy stream)."""
    import dataclasses

    from workload import get_workload
    from workload.gpu_run import GpuWorkload

    base = get_workload(key)
    total = args.warmup + args.steps + 2 * args.measure_steps
    wl = dataclasses.replace(base, steps=max(base.steps, total))
    t0 = time.perf_counter()
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f}s ({wl.name})")
    stream = torch.cuda.current_stream()
    # warmup: the first half through decode_layer decides the path (split when
    # it missed pages), the second half runs the chosen path (its first use of
    # the copy stream costs milliseconds once)
    cw = g.tier.read_counters()
    w1 = (args.warmup + 1) // 2
    for s in range(w1):
        g.decode_step(s)
    torch.cuda.synchronize()
    warm_misses = g.tier.read_counters()["misses"] - cw["misses"]
    # (one layer: a missed row is the layer's slice, nothing is left to split)
    split = wl.num_layers > 1 and (args.decode == "split" or (args.decode == "auto" and warm_misses > 0))
    side = torch.cuda.Stream() if split else None
    log(f"[bench] decode path: {'split' if split else 'plain'} ({warm_misses} misses in {w1} warmup steps)")
    for s in range(w1, args.warmup):
        if split:
            g.decode_step_split(s, side, join=False)
        else:
            g.decode_step(s)
    if split:
        stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    if args.graph:
        for s in range(args.warmup, args.warmup + args.steps):
            cg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cg):
                if split:
                    g.decode_step_split(s, side)
                else:
                    g.decode_step(s)
            graphs[s] = cg
        torch.cuda.synchronize()
    L = wl.num_layers
    c0 = g.tier.read_counters()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i, s in enumerate(range(args.warmup, args.warmup + args.steps)):
        if args.graph:
            graphs[s].replay()
        elif split:
            g.decode_step_split(s, side, join=False)
        else:
            g.decode_step(s)
    if split:
        stream.wait_stream(side)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    c1 = g.tier.read_counters()
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step")
    s_next = args.warmup + args.steps
    snap = {k_: getattr(g, k_).clone() for k_ in ("sel", "out_slots", "miss_count", "out")}
    rest = None
    if split:
        # HIP events on the copy stream around each call's rest-of-rows copy, in
        # steps of their own (markers between the copies add gaps to the timed
        # steps).  The marker before a call runs when the copy stream reaches it,
        # after the previous call's copy: the span is the copy plus any wait for
        # its own slice copy.
        ev = []
        cr0 = g.tier.read_counters()
        for s in range(s_next, s_next + args.measure_steps):
            for layer in range(L):
                ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ea.record(side)
                g.tier.decode_layer_split(layer, g.q[s, layer], g.bt, g.n_pages, g.ctx_len, wl.topk, g.sel[layer],
                                          g.needed[layer], g.out_slots[layer], g.miss[layer], g.miss_count[layer],
                                          g.out[layer], side, page_bias=g.bias)
                eb.record(side)
                ev.append((ea, eb))
        stream.wait_stream(side)
        torch.cuda.synchronize()
        cr1 = g.tier.read_counters()
        s_next += args.measure_steps
        import numpy as np
        rest_us = 1e3 * float(np.median([a.elapsed_time(b) for a, b in ev]))   # median: see measure_kernels
        rest_bytes = (cr1["bytes_fetched"] - cr0["bytes_fetched"]) * (L - 2) / L / len(ev)
        rest = dict(us=rest_us, bytes=rest_bytes, GBps=rest_bytes / (rest_us * 1e-6) / 1e9, launches=len(ev))
        log(f"[bench] rest copy {rest}")
    plain = None
    if split and headline and not args.no_extras:
        # the same steps from the same state through decode_layer, on a second tier
        g2 = GpuWorkload(wl)
        g2.setup()
        g2.upload_queries()
        for s in range(args.warmup):
            g2.decode_step(s)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(args.warmup, args.warmup + args.steps):
            g2.decode_step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / args.steps
        same = all(torch.equal(snap[k_], getattr(g2, k_)) for k_ in snap)
        plain = {"ms_per_step": round(pms, 4), "steps_per_s": round(1e3 / pms, 2),
                 "split_speedup": round(pms / ms, 4),
                 "note": "decode_layer (one stream: select+ensure, whole-row copy, attention) over the same "
                         "steps from the same state, on a second tier; last step's selections, slot maps, misses and "
                         "attention outputs " + ("equal" if same else "DIFFER")}
        log(f"[bench] plain decode {plain}")
        del g2
        torch.cuda.empty_cache()
    k = measure_kernels(torch, g, s_next, args.measure_steps)
    log(f"[bench] kernels {k}")
    misses_step = (c1["misses"] - c0["misses"]) / args.steps
    link_bytes_step = (c1["bytes_fetched"] - c0["bytes_fetched"]) / args.steps
    err = c1["error_word"]
    fetch_share = k["fetch_us"] * wl.num_layers / (ms * 1e3)
    t_read, t_write = fetch_traffic() if key == "c3" else (None, None)
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
        "roofline": ({"kernel": "k_fetch_slice + k_fetch_rest (each call's missed rows: the decoded and next "
                                "layers' slices on the decode stream, the rest on the copy stream; the two share the "
                                "host link, so the figure is the link's over the timed steps)",
                      "bound": "host_link",
                      "achieved": round(link_bytes_step / (ms * 1e-3) / 1e9, 2), "peak": LINK_PEAK_GBPS,
                      "unit": "GB/s", "frac": round(link_bytes_step / (ms * 1e-3) / 1e9 / LINK_PEAK_GBPS, 4),
                      "traffic": split_traffic(misses_step / wl.num_layers) if key == "c3" else None,
                      "traffic_note": "FETCH_SIZE (the host reads, which pass the L2s) + WRITE_SIZE (the HBM "
                                      "writes): every copied byte counts twice, so 2 x bytes_per_launch is the "
                                      "floor",
                      "bytes_per_launch": round(link_bytes_step / wl.num_layers),
                      "avg_launch_us": round(ms * 1e3 / wl.num_layers, 2),
                      "launch": "one decode_layer_split call (a slice copy and a rest copy); avg = step time / layers"}
                     if rest else
                     {"kernel": "k_fetch (fused host->device page copy)", "bound": "host_link",
                      "achieved": round(k["fetch_GBps"], 2), "peak": LINK_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(k["fetch_GBps"] / LINK_PEAK_GBPS, 4), "traffic": t_read,
                      "traffic_hbm_write": t_write,
                      "bytes_per_launch": round(k["fetch_bytes_per_launch"]),
                      "avg_launch_us": round(k["fetch_us"], 2), "step_time_share": round(fetch_share, 3)}),
        "rest_copy": ({"kernel": "k_fetch_rest", "achieved_GBps": round(rest["GBps"], 2),
                       "bytes_per_launch": round(rest["bytes"]), "avg_launch_us": round(rest["us"], 2),
                       "launches": rest["launches"],
                       "traffic": pmc_traffic("c3_pmc_traffic.json", "k_fetch_rest", "tkv_fetch.hip")
                       if key == "c3" else None,
                       "note": "HIP events on the copy stream around each call, in steps of their own: there "
                               "the copies do not overlap the next call's slice copy, as they do in the timed "
                               "steps"} if rest else None),
        "whole_row_copy": {"kernel": "k_fetch (decode_layer's one-launch copy, timed one launch at a time)",
                           "achieved_GBps": round(k["fetch_GBps"], 2),
                           "bytes_per_launch": round(k["fetch_bytes_per_launch"]),
                           "avg_launch_us": round(k["fetch_us"], 2), "traffic": t_read,
                           "traffic_hbm_write": t_write},
        "decode_path": "split" if split else "plain",
        "plain_decode": plain,
        "roofline_hbm": {"kernel": "k_attn_mfma_split (sparse paged attention, split pages + merge)",
                         "bound": "hbm",
                         "achieved": round(k["attn_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(k["attn_GBps"] / HBM_PEAK_GBPS, 4),
                         "traffic": pmc_traffic("c3_pmc_traffic.json", "k_attn_mfma_split", "tkv_attn_mfma.hip")
                         if key == "c3" else None,
                         "bytes_per_launch": k["attn_bytes_per_launch"],
                         "avg_launch_us": round(k["attn_us"], 2)},
        "select_ensure": {"avg_us": round(k["select_ensure_us"], 2),
                          "slab_GBps": round(k["select_ensure_GBps"], 1)},
        "link": {"misses_per_step": round(misses_step, 1),
                 "bytes_per_step": round(link_bytes_step),
                 "step_GBps": round(link_bytes_step / (ms * 1e-3) / 1e9, 2)},
        "launch": ("hip graph per step" if args.graph else "eager, one C call per layer")
                  + (" (decode_layer_split: copy stream joined once, after the timed steps; rest-copy "
                     "events in %d steps of their own)" % args.measure_steps if split else ""),
        "error_word": err,
    }
    # per-step HBM bytes the method needs (slab of every visible page, the
    # selected pages' K/V codes and scales, queries and outputs), all layers
    qo = 2 * wl.batch * wl.num_q_heads * wl.head_dim * 2
    step_bytes = wl.num_layers * (int(g.npg_np.sum()) * wl.num_kv_heads * wl.head_dim * 2
                                  + wl.batch * wl.topk * g.tier.layer_bytes + qo)
    result["_kernels"] = k
    result["step_hbm"] = {"bytes_per_step": step_bytes, "achieved": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                          "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5)}
    return result, g, split, side


def bench_cold_step(torch, g, s0, reps):
    """c3 from an empty pool: residency reset, then one decode step (all
    layers through decode_layer: every selected page misses); `reps` times.
    Link rate = bytes fetched / step time (the copies dominate it)."""
    import numpy as np
    wl, t = g.wl, g.tier
    stream = torch.cuda.current_stream()
    rec = []
    for i in range(reps + 1):
        t.reset_residency()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.decode_step((s0 + i) % g.q.shape[0])
        e1.record(stream)
        torch.cuda.synchronize()
        c = t.read_counters()
        if i:
            rec.append((e0.elapsed_time(e1), c["misses"], c["bytes_fetched"]))
    ms = float(np.mean([r[0] for r in rec]))
    b = float(np.mean([r[2] for r in rec]))
    return {"ms_per_step": round(ms, 4), "misses_per_step": round(float(np.mean([r[1] for r in rec])), 1),
            "bytes_per_step": round(b),
            "roofline": {"kernel": "each layer's whole-row copy of its misses (folded into the k_attn_mfma_split "
                                   "launch), over the step",
                         "bound": "host_link", "achieved": round(b / (ms * 1e-3) / 1e9, 2),
                         "peak": LINK_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(b / (ms * 1e-3) / 1e9 / LINK_PEAK_GBPS, 4), "traffic": None},
            "note": f"residency reset before each of {reps} steps (decode_layer, one stream): every page the "
                    "step selects misses; achieved = bytes fetched / step time"}


def pcie_link(torch):
    """Negotiated PCIe link of the GPU and of the bridges above it (sysfs)."""
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except Exception as e:
        return {"error": f"no PCI address: {e}"}
    out = {"device": bdf, "chain": []}
    path = os.path.realpath(os.path.join("/sys/bus/pci/devices", bdf))
    for _ in range(6):
        rec = {"bdf": os.path.basename(path)}
        for f in ("current_link_speed", "current_link_width", "max_link_speed", "max_link_width"):
            try:
                rec[f] = open(os.path.join(path, f)).read().strip()
            except Exception:
                pass
        if len(rec) == 1:
            break
        out["chain"].append(rec)
        path = os.path.dirname(path)
    return out


def decode_summary(r, cpu):
    """The sub-object of one decode workload in the default line.  Workloads
    whose timed steps are link-bound (the copies take most of the step: c4)
    keep the host-link roofline; the others (c1, c2: few or no misses) are
    priced against HBM on their dominant kernel, the indexer launch or the
    attention launch, whichever took longer."""
    keep = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "decode_path", "roofline",
            "roofline_hbm", "select_ensure", "link", "step_hbm", "rest_copy", "error_word")
    out = {"workload": r["config"]["workload"], **{k: r.get(k) for k in keep}}
    out["metric"] = "decode steps/s (all layers)"
    link_share = r["link"]["bytes_per_step"] / (r["ms_per_step"] * 1e-3) / 1e9 / LINK_PEAK_GBPS
    if link_share < 0.25:
        k = r["_kernels"]
        sel = {"kernel": "k_select_scan + k_ensure (indexer scan, top-k, compaction; LRU ensure)", "bound": "hbm",
               "achieved": round(k["select_ensure_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": round(k["select_ensure_GBps"] / HBM_PEAK_GBPS, 5), "traffic": None,
               "bytes_per_launch": k["select_bytes_per_launch"], "avg_launch_us": round(k["select_ensure_us"], 2)}
        att = dict(r["roofline_hbm"])
        out["roofline_link"] = out["roofline"]
        if k["select_ensure_us"] >= k["attn_us"]:
            out["roofline"], out["roofline_hbm"] = sel, att
        else:
            out["roofline"], out["roofline_hbm"] = att, sel
    out["cpu_baseline"] = cpu
    return out


def main():
    t_start = time.perf_counter()
    args = parse()
    if args.cpu_baseline_child:
        cpu_child_main(args.cpu_baseline_child)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by request, one tier per GPU, with no exchange)", file=sys.stderr)
        sys.exit(2)
    others = [] if args.headline_only else [k for k in ("c1", "c2", "c4", "c5") if k != args.config]
    # the CPU baselines start before this process touches the GPU
    child = None if args.no_cpu_baseline else start_cpu_child(args, [args.config] + others)

    import torch

    from workload import get_workload

    torch.cuda.set_device(0)
    base = get_workload(args.config)
    if base.prefill_tokens:
        result = bench_prefill(torch, args.config, args.warmup, args.steps, cold_reps=0 if args.headline_only else 2)
        cpu = collect_cpu_child(child, t_start, args.cpu_deadline)
        result["cpu_baseline"] = cpu.get(args.config)
        print(json.dumps(result), flush=True)
        return
    calib = calibrate(torch)
    calib["pcie_link"] = pcie_link(torch)
    log(f"[bench] calibration {calib}")
    result, g, split, side = bench_decode(torch, args.config, args, headline=True)
    result["calibration"] = calib
    if args.no_extras:
        result.update(prefetch=None, host_tail=None, prefix_rehydrate=None, decode_append=None)
    else:
        link_util = result["link"]["step_GBps"] / max(1e-9, calib["h2d_memcpy_GBps"])
        result["prefetch"] = bench_prefetch(torch, g, args.warmup + args.steps + args.measure_steps,
                                            min(args.steps, 50), result["ms_per_step"],
                                            result["link"]["misses_per_step"], link_util)
        log(f"[bench] prefetch {result['prefetch']}")
        result["host_tail"] = bench_host_tail(torch, g, args.warmup + args.steps + args.measure_steps,
                                              min(args.steps, 50))
        log(f"[bench] host tail {result['host_tail']}")
        result["prefix_rehydrate"] = bench_prefix(g, 375)
        log(f"[bench] prefix {result['prefix_rehydrate']}")
    if not args.headline_only:
        result["cold_step"] = bench_cold_step(torch, g, args.warmup + args.steps, 3)
        log(f"[bench] cold step {result['cold_step']}")
    if not args.no_extras and args.config == "c3":
        del g
        torch.cuda.empty_cache()
        result["decode_append"] = bench_append(torch, "c3a", min(args.steps, 40), 4)
        log(f"[bench] decode append {result['decode_append']}")
    else:
        result["decode_append"] = None
        del g
        torch.cuda.empty_cache()
    subs = {}
    for key in others:
        if key == "c5":
            r = bench_prefill(torch, key, 1, 3, cold_reps=2)
            subs[key] = {"workload": r["config"]["workload"], **{k: r[k] for k in (
                "metric", "value", "unit", "ms_per_step", "steps", "warmup", "split_ms", "roofline",
                "roofline_mfma", "mirror_write_GBps", "mirror_copy_ms", "store_path", "cold_chunk",
                "error_word")}}
            rs = bench_prefill(torch, key, 1, 3, split_store=False)
            subs[key]["plain_store"] = {k: rs[k] for k in ("ms_per_step", "split_ms", "mirror_write_GBps",
                                                           "store_path")}
            subs[key]["plain_store"]["note"] = ("the same chunk with the store kernel writing pool and mirror: "
                                                "the mirror writes on the chunk's critical path")
            subs[key]["roofline_link"] = {"kernel": "k_mirror_copy (mirror writes of the chunk's new K/V, all "
                                                    "layers, beside the attention: off the critical path)",
                                          "bound": "host_link", "achieved": r["mirror_write_GBps"],
                                          "peak": LINK_PEAK_GBPS, "unit": "GB/s",
                                          "frac": round(r["mirror_write_GBps"] / LINK_PEAK_GBPS, 4),
                                          "traffic": None}
        else:
            r, gk, _, _ = bench_decode(torch, key, args, headline=False)
            subs[key] = decode_summary(r, None)
            if key == "c4" and not args.no_extras:
                lu = r["link"]["step_GBps"] / max(1e-9, calib["h2d_memcpy_GBps"])
                subs[key]["prefetch"] = bench_prefetch(torch, gk, args.warmup + args.steps + 2 * args.measure_steps,
                                                       min(args.steps, 50), r["ms_per_step"],
                                                       r["link"]["misses_per_step"], lu)
                log(f"[bench] {key} prefetch {subs[key]['prefetch']}")
            del gk
            torch.cuda.empty_cache()
        log(f"[bench] {key}: {subs[key]['value']} {subs[key]['unit']}")
    cpu = collect_cpu_child(child, t_start, args.cpu_deadline)
    result["cpu_baseline"] = cpu.get(args.config)
    for key in subs:
        subs[key]["cpu_baseline"] = cpu.get(key)
    result.pop("_kernels", None)
    result["configs"] = subs
    result["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
