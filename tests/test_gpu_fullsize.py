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


def test_c3_fullsize_steady_state_split():
    """The bench's timed window at full size: steps 0-2 through decode_layer,
    then decode_layer_split with the copy stream joined only where a step is
    compared (as the bench joins it once, after its timed steps); every layer
    of steps 5 and 24 (the first and last timed steps of the driver's
    5 warmup + 20 timed steps) against the oracle -- selections, compaction,
    slot maps, miss lists -- LRU state and counters at steps 5, 14 and 24,
    attention on two layers of step 24, pool rows of pages copied then."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3")
    say(f"[fullsize] c3 steady state: {wl.description}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=False)
    run.setup(wl, o)
    say("[fullsize] c3 steady state: setups done")
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    side = torch.cuda.Stream()
    stream = torch.cuda.current_stream()
    check_layers, check_state, attn_step = {5, 24}, {5, 14, 24}, 24
    rng = np.random.default_rng(11)
    for s in range(25):
        if s < 3:
            g.decode_step(s)
        else:
            g.decode_step_split(s, side, join=False)
        if s in check_state:
            stream.wait_stream(side)
            torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            with_attn = s == attn_step and layer in (3, 10)
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias, with_attention=with_attn)
            if s in check_layers:
                where = f"c3 steady step {s} layer {layer}"
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
            compare_state(g, o, f"c3 steady step {s}", sample_pages=picked)
            say(f"[fullsize] c3 steady state: step {s} ok")
    c = g.tier.read_counters()
    assert c["error_word"] == 0 and c["drops"] == 0 and c["misses"] > 0
