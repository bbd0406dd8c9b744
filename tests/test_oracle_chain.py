"""End-to-end pins of the oracle chain on small workloads.

* budget >= context: the chain's sparse output equals dense attention over
  every token of the context, computed straight from the generated keys and
  values quantised by the store (FreeToken PR #499: only the selection
  changes what is read);
* the pool row of every resident page equals the mirror row after every
  layer (drop-clean slots), the decode path never writes the mirror, each
  fetch moves exactly the missed pages and nothing is fetched twice per call;
* forced drops are counted, never silent.
"""
from dataclasses import replace

import numpy as np
import pytest

from oracle import run
from oracle.attention import dense_reference
from oracle.engine import CapacityError
from oracle.store import quantize_tokens
from oracle.codecs import e4m3_decode
from workload import gen, get_workload


def _check_drop_clean(tier):
    for s in range(tier.S):
        p = int(tier.lru.slot_to_page[s])
        if p >= 0:
            assert np.array_equal(tier.pool[s], tier.mirror_row(p)), (s, p)


def test_c1_chain_drop_clean_and_no_writeback():
    wl = get_workload("c1")
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    _check_drop_clean(tier)
    snapshot = {p: r.copy() for p, r in tier.mirror.items()}
    fetched = []

    def on_layer(s, layer, rec):
        _check_drop_clean(tier)
        m = rec["misses"]
        assert len({int(p) for p in m[:, 1]}) == len(m)   # nothing fetched twice
        fetched.append(len(m))

    b0 = tier.bytes_fetched
    run.decode(wl, tier, on_layer=on_layer, attention=True)
    assert tier.bytes_fetched - b0 == sum(fetched) * tier.lay.row_bytes
    for p, r in tier.mirror.items():
        assert np.array_equal(r, snapshot[p])
    assert tier.counters()["drops"] == 0 and tier.counters()["error_word"] == 0


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sparse_equals_dense_when_budget_covers_context(fmt):
    base = get_workload("c1")
    wl = replace(base, kv_format=fmt, contexts=(256,), topk=16, num_slots=48, steps=2)
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    tr = run.decode(wl, tier, attention=True)
    q = gen.decode_queries(wl)
    k = gen.kv_tokens(wl, gen.KIND_K, 0, 0, 0, 256)
    v = gen.kv_tokens(wl, gen.KIND_V, 0, 0, 0, 256)
    if fmt == "fp8":
        kc, ks = quantize_tokens(k)
        vc, vs = quantize_tokens(v)
        k = e4m3_decode(kc).astype(np.float64) * ks[:, None, None]
        v = e4m3_decode(vc).astype(np.float64) * vs[:, None, None]
    for s in range(2):
        assert tr[s][0]["sel"][0].tolist() == list(range(16))
        ref = dense_reference(q[s, 0, 0].astype(np.float64), k.transpose(1, 0, 2).astype(np.float64),
                              v.transpose(1, 0, 2).astype(np.float64))
        assert np.allclose(tr[s][0]["out"][0], ref, rtol=1e-12, atol=1e-12)


def test_partial_last_page_masked_by_context_length():
    wl = replace(get_workload("c1"), contexts=(250,), topk=16, num_slots=48, steps=1)
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    tr = run.decode(wl, tier, attention=True)
    q = gen.decode_queries(wl)
    k = gen.kv_tokens(wl, gen.KIND_K, 0, 0, 0, 250).transpose(1, 0, 2).astype(np.float64)
    v = gen.kv_tokens(wl, gen.KIND_V, 0, 0, 0, 250).transpose(1, 0, 2).astype(np.float64)
    ref = dense_reference(q[0, 0, 0].astype(np.float64), k, v)
    assert np.allclose(tr[0][0]["out"][0], ref, rtol=1e-12, atol=1e-12)


def test_forced_drops_counted():
    wl = replace(get_workload("c1"), steps=2)
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    bt, npg = gen.block_tables(wl)
    tier.set_select_width(1, wl.topk, 10)       # cap below top-k
    q = gen.decode_queries(wl)
    sel, needed = tier.select(0, q[0, 0], np.array([0, 1]), None, bt, npg, wl.topk)
    assert tier.drops == wl.topk - 10
    assert needed[0].tolist() == bt[0][sel[0][:10]].tolist()


def test_capacity_by_construction():
    wl = get_workload("c4")
    tier = run.make_tier(replace(wl, num_slots=200), materialize=False)
    with pytest.raises(CapacityError):
        tier.set_select_width(4, 32)            # 4 * 72 = 288 > 200


def test_roundtrip_store_evict_fetch_exact():
    wl = replace(get_workload("c3s"), steps=3)
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    ref = {p: r.copy() for p, r in tier.mirror.items()}
    run.decode(wl, tier)                                   # thrashes: evicts and refetches
    assert tier.lru.counters["evictions"] > 0 and tier.bytes_fetched > 0
    _check_drop_clean(tier)
    for p, r in tier.mirror.items():
        assert np.array_equal(r, ref[p])


def test_lazy_rows_equal_materialized_rows():
    wl = get_workload("c4s")
    a = run.make_tier(wl, materialize=True)
    b = run.make_tier(wl, materialize=False)
    run.setup(wl, a)
    run.setup(wl, b)
    assert np.array_equal(a.slab, b.slab)
    for p in [0, 5, 100, 250, wl.num_logical_pages - 1]:
        assert np.array_equal(a.mirror_row(p), b.mirror_row(p))


def test_prefill_chain_small():
    wl = get_workload("c5s")
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    recs = run.prefill(wl, tier, attention_rows=[0, 1, 63, 64, 511])
    n0 = wl.contexts[0] // wl.page_size
    for rec in recs:
        sel = rec["sel"]
        # row 0 (position = cached length) sees pages 0..n0
        assert sel[0].max() <= n0
        assert np.all(rec["out_slots"][rec["needed"][0] >= 0] >= 0)
    assert tier.counters()["error_word"] == 0


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_host_tail_with_empty_pool_equals_dense(fmt):
    """Host tail read in place: with nothing resident every selected page comes
    from its mirror row, and with the budget covering the context the output
    is dense attention over the quantised keys and values."""
    base = get_workload("c1")
    wl = replace(base, kv_format=fmt, contexts=(256,), topk=16, num_slots=48, steps=1)
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    tier.reset_residency()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    tier.set_select_width(1, wl.topk, wl.max_sel_pages)
    rec = tier.decode_layer_host_tail(0, q[0, 0], np.array([0, 1]), bt, npg, ctx, wl.topk)
    assert not np.any(tier.lru.page_to_slot >= 0)          # nothing was made resident
    k = gen.kv_tokens(wl, gen.KIND_K, 0, 0, 0, 256)
    v = gen.kv_tokens(wl, gen.KIND_V, 0, 0, 0, 256)
    if fmt == "fp8":
        kc, ks = quantize_tokens(k)
        vc, vs = quantize_tokens(v)
        k = e4m3_decode(kc).astype(np.float64) * ks[:, None, None]
        v = e4m3_decode(vc).astype(np.float64) * vs[:, None, None]
    ref = dense_reference(q[0, 0, 0].astype(np.float64), k.transpose(1, 0, 2).astype(np.float64),
                          v.transpose(1, 0, 2).astype(np.float64))
    assert np.allclose(rec["out"][0], ref, rtol=1e-12, atol=1e-12)


def test_host_tail_leaves_residency_and_matches_fetch_path():
    """The in-place read gives the fetch path's output exactly (mirror rows
    hold the pool's bytes) and moves no residency state."""
    wl = get_workload("c3s")
    a = run.make_tier(wl, materialize=True)
    b = run.make_tier(wl, materialize=True)
    run.setup(wl, a)
    run.setup(wl, b)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.array([0, 1])
    for t in (a, b):
        t.set_select_width(1, wl.topk, wl.max_sel_pages)
    state = (b.lru.page_to_slot.copy(), b.lru.stamp.copy(), b.lru.clock, dict(b.lru.counters))
    for layer in range(wl.num_layers):
        ra = a.decode_layer(layer, q[0, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
        rb = b.decode_layer_host_tail(layer, q[0, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
        assert np.array_equal(ra["sel"], rb["sel"]) and np.array_equal(ra["needed"], rb["needed"])
        assert np.array_equal(ra["out"], rb["out"])
    assert a.lru.counters["misses"] > 0                     # the fetch path did move pages
    assert np.array_equal(b.lru.page_to_slot, state[0]) and np.array_equal(b.lru.stamp, state[1])
    assert b.lru.clock == state[2] and dict(b.lru.counters) == state[3]


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_decode_attends_over_grown_context(fmt):
    """Decode with one appended token per step: with the budget covering the
    context, every layer's output is dense attention over all tokens written
    so far, the new one included (stored before the layer's selection)."""
    base = get_workload("c1")
    wl = replace(base, kv_format=fmt, contexts=(200,), topk=16, num_slots=48, steps=3, append=True,
                 num_layers=2)
    assert wl.pages_of(0) == 13
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)
    tr = run.decode(wl, tier, attention=True)
    q = gen.decode_queries(wl)
    for s in range(wl.steps):
        n = 200 + s + 1
        for layer in range(wl.num_layers):
            k = gen.kv_tokens(wl, gen.KIND_K, layer, 0, 0, n)
            v = gen.kv_tokens(wl, gen.KIND_V, layer, 0, 0, n)
            if fmt == "fp8":
                kc, ks = quantize_tokens(k)
                vc, vs = quantize_tokens(v)
                k = e4m3_decode(kc).astype(np.float64) * ks[:, None, None]
                v = e4m3_decode(vc).astype(np.float64) * vs[:, None, None]
            out = tr[s][layer]["out"][0]
            for h in (0, 5):
                ref = dense_reference(q[s, layer, 0, h:h + 1].astype(np.float64),
                                      k.transpose(1, 0, 2).astype(np.float64),
                                      v.transpose(1, 0, 2).astype(np.float64))
                assert np.allclose(out[h], ref[0], rtol=1e-12, atol=1e-12), (s, layer, h)
    _check_drop_clean(tier)


def test_append_under_thrash_keeps_pool_rows_clean():
    """Appending on the thrashing small workload: every layer's write-ensure
    brings the page back if an earlier layer evicted it, so after each step
    (every layer has written its block of a freshly allocated page) resident
    pool rows equal their mirror rows, and the mirror holds every appended
    token."""
    wl = get_workload("c3sa")
    tier = run.make_tier(wl, materialize=True)
    run.setup(wl, tier)

    def at_layer(s, layer, rec):
        if layer == wl.num_layers - 1:
            _check_drop_clean(tier)

    run.decode(wl, tier, on_layer=at_layer)
    assert tier.lru.counters["evictions"] > 0
    bt, _ = gen.block_tables(wl)
    from oracle.store import read_kv
    last = wl.contexts[0] + wl.steps - 1
    page = int(bt[0][last // wl.page_size])
    k, _ = read_kv(tier.mirror_row(page), tier.lay, wl.num_layers - 1)
    kc, ks = quantize_tokens(gen.kv_tokens(wl, gen.KIND_K, wl.num_layers - 1, 0, last, 1))
    ref = e4m3_decode(kc).astype(np.float64) * ks[:, None, None]
    assert np.array_equal(k[:, last % wl.page_size], ref[0])


def test_prefetch_with_perfect_prediction_moves_every_miss_to_the_preload():
    """Preload of the exact list the layer is about to need: the preload
    fetches precisely the plain path's misses (same slots, same order), the
    layer itself then misses nothing, slot maps and attention are those of
    the plain path; with an empty prediction the layer is the plain one."""
    wl = get_workload("c3s")
    a = run.make_tier(wl, materialize=True)
    b = run.make_tier(wl, materialize=True)
    run.setup(wl, a)
    run.setup(wl, b)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.array([0, 1])
    for t in (a, b):
        t.set_select_width(1, wl.topk, wl.max_sel_pages)
    ca, cb = a.lru.counters["ensure_calls"], b.lru.counters["ensure_calls"]
    moved = 0
    for s in range(3):
        for layer in range(wl.num_layers):
            ra = a.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            pred = ra["needed"] if s > 0 else np.full_like(ra["needed"], -1)
            rb = b.decode_layer_prefetch(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, pred, bias=bias)
            if s > 0:
                assert np.array_equal(rb["pre_misses"], ra["misses"])
                assert len(rb["misses"]) == 0
                moved += len(ra["misses"])
            else:
                assert len(rb["pre_misses"]) == 0 and np.array_equal(rb["misses"], ra["misses"])
            assert np.array_equal(ra["sel"], rb["sel"]) and np.array_equal(ra["out_slots"], rb["out_slots"])
            assert np.array_equal(ra["out"], rb["out"])
            assert np.array_equal(a.lru.page_to_slot, b.lru.page_to_slot)
    assert moved > 0
    assert b.lru.counters["ensure_calls"] - cb == 2 * (a.lru.counters["ensure_calls"] - ca)


def test_prefix_save_restore_under_new_ids_decodes_like_the_original():
    """A request's prefix saved, then rehydrated under another request's
    logical ids (whose resident slots get unbound): decoding it through a
    block table pointing at the new ids gives exactly the original's
    selections and attention, with the moved pages fetched lazily."""
    wl = replace(get_workload("c4s"), contexts=(4096, 4096, 2048, 8192), steps=3)
    bt, npg = gen.block_tables(wl)
    a = run.make_tier(wl, materialize=True)
    b = run.make_tier(wl, materialize=True)
    run.setup(wl, a)
    run.setup(wl, b)
    ctx = gen.context_lengths(wl)
    q = gen.decode_queries(wl)
    rs = np.arange(wl.batch + 1)
    for t in (a, b):
        t.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    for layer in range(wl.num_layers):           # step 0 on both: some of request 0's pages get resident
        for t in (a, b):
            t.decode_layer(layer, q[0, layer], rs, bt, npg, ctx, wl.topk)
    src, dst = bt[1, :npg[1]], bt[0, :npg[0]]
    resident_before = int(np.sum(b.lru.page_to_slot[dst] >= 0))
    assert resident_before > 0
    b.prefix_restore(dst, b.prefix_save(src))
    assert not np.any(b.lru.page_to_slot[dst] >= 0)
    bt2 = bt.copy()
    bt2[1, :npg[1]] = dst                      # request 1 now lives on request 0's old ids
    m0 = b.lru.counters["misses"]
    for s in range(1, wl.steps):
        for layer in range(wl.num_layers):
            ra = a.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk)
            rb = b.decode_layer(layer, q[s, layer], rs, bt2, npg, ctx, wl.topk)
            assert np.array_equal(ra["sel"][1], rb["sel"][1])
            assert np.array_equal(ra["out"][1], rb["out"][1])
    assert b.lru.counters["misses"] > m0
