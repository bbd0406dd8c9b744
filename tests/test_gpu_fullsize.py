"""Parity at the full workload sizes, in the launch configurations bench.py
times: fused decode_layer per layer (eager launches on one stream), and for
the workloads whose steps miss pages (196k-context thrash, batch 4) the split
decode the bench times there (decode_layer_split: slice copies on the decode
stream, the rest of the rows on a copy stream).

Exact for every layer of the steps run: selections, compaction, slot maps,
miss lists, LRU state and counters; the slab of every page; attention on
sampled layers (every head of every row); mirror and pool bytes on sampled
pages.  The oracle keeps no page bytes at these sizes: it rebuilds a page's
row from the input generator when a sampled check reads it.
"""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import assert_close, bf16_to_f64, compare_state, say

pytestmark = pytest.mark.gpu


def _decode_fullsize(key, steps, attn_layers, split=False):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[fullsize] {key}: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    say(f"[fullsize] {key}: gpu setup done")
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    say(f"[fullsize] {key}: oracle setup done")
    rng = np.random.default_rng(7)
    sample_pages = sorted(set(rng.integers(0, wl.num_logical_pages, 6).tolist()))
    compare_state(g, o, f"{key} after setup", sample_pages=sample_pages)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    side = torch.cuda.Stream() if split else None
    for s in range(steps):
        if split:
            g.decode_step_split(s, side)
        else:
            g.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            where = f"{key} step {s} layer {layer}"
            with_attn = layer in attn_layers
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias,
                                 with_attention=with_attn)
            assert np.array_equal(g.sel[layer].cpu().numpy(), rec["sel"]), f"{where}: sel"
            assert np.array_equal(g.needed[layer].cpu().numpy(), rec["needed"]), f"{where}: needed"
            assert np.array_equal(g.out_slots[layer].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
            m = int(g.miss_count[layer].item())
            assert np.array_equal(g.miss[layer].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
            if with_attn:
                assert_close(bf16_to_f64(g.out[layer]), rec["out"], f"{where}: attention")
        say(f"[fullsize] {key}: step {s} ok")
        compare_state(g, o, f"{key} step {s}", sample_pages=sample_pages)
        if split:
            # pool rows of pages the step's copies brought in (resident now)
            resident = [int(p) for p in o.lru.slot_to_page if p >= 0]
            picked = sorted(rng.choice(resident, size=min(4, len(resident)), replace=False).tolist())
            compare_state(g, o, f"{key} step {s} (copied rows)", sample_pages=picked)
    c = g.tier.read_counters()
    assert c["error_word"] == 0 and c["drops"] == 0
    return wl, g, o


def test_c2_fullsize():
    _decode_fullsize("c2", steps=3, attn_layers={0, 7})


def test_c3_fullsize():
    wl, g, o = _decode_fullsize("c3", steps=3, attn_layers={0, 11})
    c = g.tier.read_counters()
    assert c["misses"] > 0 and c["evictions"] > 0


def test_c4_fullsize():
    _decode_fullsize("c4", steps=2, attn_layers={5})


def test_c3_fullsize_split():
    wl, g, o = _decode_fullsize("c3", steps=3, attn_layers={1, 6, 11}, split=True)
    c = g.tier.read_counters()
    assert c["misses"] > 0 and c["evictions"] > 0


def test_c4_fullsize_split():
    _decode_fullsize("c4", steps=2, attn_layers={2, 9}, split=True)


def test_c5_fullsize_prefill():
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5")
    say(f"[fullsize] c5: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    got = []

    def on_layer(layer, bufs):
        got.append({k: bufs[k].clone() for k in ("sel", "needed", "out_slots", "miss", "miss_count", "out")})

    g.prefill(on_layer=on_layer, copy_stream=torch.cuda.Stream())   # split stores, as the bench runs the chunk
    torch.cuda.synchronize()
    say("[fullsize] c5: gpu chunk done")
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    # chunk edges, 64-row block edges and a seeded spread: every row holds
    # its own top-32 pages over the whole cached range plus the causal tail
    rng = np.random.default_rng(5)
    edges = {0, 1, 62, 63, 64, 65, 127, 128, 1000, 2047, 2048, 3000, 4094, 4095}
    rest = np.array(sorted(set(range(wl.prefill_tokens)) - edges))
    rows = sorted(edges | set(int(x) for x in rng.choice(rest, 34, replace=False)))
    assert len(rows) == 48
    recs = run.prefill(wl, o, attention_rows=rows)
    for layer, (gg, rec) in enumerate(zip(got, recs)):
        where = f"c5 layer {layer}"
        assert np.array_equal(gg["sel"].cpu().numpy(), rec["sel"]), f"{where}: sel"
        assert np.array_equal(gg["needed"].cpu().numpy(), rec["needed"]), f"{where}: needed"
        assert np.array_equal(gg["out_slots"].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
        m = int(gg["miss_count"].item())
        assert np.array_equal(gg["miss"].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
        out = bf16_to_f64(gg["out"][rows])
        ref = np.stack([rec["out"][r] for r in rows])
        assert_close(out, ref, f"{where}: attention")
    new_pages = list(range(wl.contexts[0] // wl.page_size, wl.num_logical_pages))
    compare_state(g, o, "c5 after the chunk", sample_pages=new_pages[:3] + new_pages[-2:])


def test_c5_fullsize_cold_chunk():
    """The chunk from an empty pool, as the bench's cold chunk runs it: the
    context written, residency reset, then the chunk -- layer 0's ensure
    misses every cached page its rows select and one fetch moves their rows
    (every layer).  Selections, slot maps and misses of every layer, the
    attention of sampled rows on every layer, LRU state, counters and the
    pool rows of sampled fetched pages."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5")
    say(f"[fullsize] c5 cold chunk: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    g.tier.reset_residency()
    torch.cuda.synchronize()
    got = []

    def on_layer(layer, bufs):
        got.append({k: bufs[k].clone() for k in ("sel", "needed", "out_slots", "miss", "miss_count", "out")})

    g.prefill(on_layer=on_layer, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    say("[fullsize] c5 cold chunk: gpu chunk done")
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    o.reset_residency()
    rng = np.random.default_rng(9)
    rows = sorted({0, 63, 64, 2047, 4095} | set(int(x) for x in rng.choice(wl.prefill_tokens, 11, replace=False)))
    recs = run.prefill(wl, o, attention_rows=rows)
    for layer, (gg, rec) in enumerate(zip(got, recs)):
        where = f"c5 cold layer {layer}"
        assert np.array_equal(gg["sel"].cpu().numpy(), rec["sel"]), f"{where}: sel"
        assert np.array_equal(gg["needed"].cpu().numpy(), rec["needed"]), f"{where}: needed"
        assert np.array_equal(gg["out_slots"].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
        m = int(gg["miss_count"].item())
        assert np.array_equal(gg["miss"].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
        out = bf16_to_f64(gg["out"][rows])
        ref = np.stack([rec["out"][r] for r in rows])
        assert_close(out, ref, f"{where}: attention")
    misses0 = recs[0]["misses"]
    assert len(misses0) > 900, len(misses0)            # layer 0 fetches the cached pages it selects
    picked = sorted(int(misses0[i][1]) for i in rng.choice(len(misses0), 4, replace=False))
    compare_state(g, o, "c5 cold chunk", sample_pages=picked)


def test_c3_fullsize_cold_steps():
    """The bench's cold step: residency reset, then one decode step through
    decode_layer (every selected page misses: the fetch folded into the
    attention launch moves ~360 whole rows), twice.  Every layer against the
    oracle, LRU state, counters and the pool rows of sampled fetched pages."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3")
    say(f"[fullsize] c3 cold steps: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    rng = np.random.default_rng(13)
    for s in (0, 1):
        g.tier.reset_residency()
        o.reset_residency()
        g.decode_step(s)
        torch.cuda.synchronize()
        fetched = []
        for layer in range(wl.num_layers):
            where = f"c3 cold step {s} layer {layer}"
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias,
                                 with_attention=layer in (0, 7))
            assert np.array_equal(g.sel[layer].cpu().numpy(), rec["sel"]), f"{where}: sel"
            assert np.array_equal(g.out_slots[layer].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
            m = int(g.miss_count[layer].item())
            assert np.array_equal(g.miss[layer].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
            if layer in (0, 7):
                assert_close(bf16_to_f64(g.out[layer]), rec["out"], f"{where}: attention")
            fetched += [int(p) for _, p in rec["misses"]]
        assert len(fetched) > 300, len(fetched)
        picked = sorted(int(fetched[i]) for i in rng.choice(len(fetched), 4, replace=False))
        compare_state(g, o, f"c3 cold step {s}", sample_pages=picked)
        say(f"[fullsize] c3 cold step {s} ok ({len(fetched)} misses)")


# bench.py's default decode run: 8 untimed steps (the first half through
# decode_layer, then the split path it chose), 100 timed steps
BENCH_WARMUP, BENCH_STEPS = 8, 100


def _steady_state_split(key, check_layers, check_state, attn_step, attn_layers, split=True):
    """The bench's decode window at full size, in its launch configuration:
    steps 0..3 through decode_layer, then (split) decode_layer_split with the
    copy stream joined only where a step is compared (the bench joins it
    once, after its timed steps), else decode_layer throughout.  Every layer of the steps in check_layers against
    the oracle (selections, compaction, slot maps, miss lists), LRU state,
    counters and the pool rows of sampled resident pages at check_state,
    attention on attn_layers of attn_step."""
    import dataclasses

    from workload.gpu_run import GpuWorkload
    base = get_workload(key)
    last = max(check_layers | check_state | {attn_step})
    wl = dataclasses.replace(base, steps=max(base.steps, BENCH_WARMUP + BENCH_STEPS))
    say(f"[fullsize] {key} steady state to step {last}: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    say(f"[fullsize] {key} steady state: setups done")
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    side = torch.cuda.Stream()
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(11)
    plain_steps = (BENCH_WARMUP + 1) // 2
    for s in range(last + 1):
        if s < plain_steps or not split:
            g.decode_step(s)
        else:
            g.decode_step_split(s, side, join=False)
        if s in check_state or s in check_layers:
            stream.wait_stream(side)
            torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            with_attn = s == attn_step and layer in attn_layers
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias, with_attention=with_attn)
            if s in check_layers:
                where = f"{key} steady step {s} layer {layer}"
                assert np.array_equal(g.sel[layer].cpu().numpy(), rec["sel"]), f"{where}: sel"
                assert np.array_equal(g.needed[layer].cpu().numpy(), rec["needed"]), f"{where}: needed"
                assert np.array_equal(g.out_slots[layer].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
                m = int(g.miss_count[layer].item())
                assert np.array_equal(g.miss[layer].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
                if with_attn:
                    assert_close(bf16_to_f64(g.out[layer]), rec["out"], f"{where}: attention")
        if s in check_state:
            resident = [int(p) for p in o.lru.slot_to_page if p >= 0]
            picked = sorted(rng.choice(resident, size=4, replace=False).tolist())
            compare_state(g, o, f"{key} steady step {s}", sample_pages=picked)
            say(f"[fullsize] {key} steady state: step {s} ok")
    c = g.tier.read_counters()
    assert c["error_word"] == 0 and c["drops"] == 0 and (c["misses"] > 0 or not split)


def test_c2_fullsize_steady_state():
    """The every-page-resident 64k decode through the bench's default window,
    all of it through decode_layer (the path the bench takes when the warmup
    misses nothing; the fetch folded into the attention launch)."""
    first, last = BENCH_WARMUP, BENCH_WARMUP + BENCH_STEPS - 1
    _steady_state_split("c2", {first, last}, {first, last}, last, (0, 11), split=False)


def test_c3_fullsize_steady_state_split():
    """The 196k-context thrash through the bench's whole default window: the
    first and last timed steps (8 and 107) and one between, every layer."""
    first, last = BENCH_WARMUP, BENCH_WARMUP + BENCH_STEPS - 1
    _steady_state_split("c3", {first, 57, last}, {first, 57, last}, last, (3, 10))


def test_c4_fullsize_steady_state_split():
    """The batch-4 mixed-context decode into the bench's default window: its
    first 21 timed steps (the oracle takes a few seconds per step here, so
    the whole window would hold the test for minutes)."""
    first, last = BENCH_WARMUP, BENCH_WARMUP + 20
    _steady_state_split("c4", {first, last}, {first, last}, last, (2, 9))
