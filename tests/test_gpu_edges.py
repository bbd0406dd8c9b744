"""GPU parity on the edges of the decode path, against the oracle.

* contexts shorter than the top-k (a one-token request, contexts ending
  mid-page): selections padded with -1, masked tails;
* top-k above 64 pages (the block top-k and unsplit attention paths);
* bf16 KV with 16-token pages and a ragged batch of three;
* a compaction width below the top-k (FreeToken PR #499, "Design": pages
  past the cap are counted as drops, not silently lost);
* the device error word (FreeToken PR #499, "Design": fixed-shape calls
  report anomalies instead of faulting): an ensure needing more distinct
  pages than slots changes nothing; page ids out of range are skipped;
  fetch entries outside the pool or the page space are skipped; a store to a
  page with no slot writes the mirror and the slab only;
* random ensure traces (duplicates, padding, ids out of range, no-fetch
  flags, capacity overruns) through both ensure paths: widths up to 512 on
  pools up to 2,048 slots (state reads up front, first occurrences from an
  LDS hash table) and wider calls or larger pools (global first-occurrence
  marks);
* requests sharing physical pages (a shared prefix) from an empty pool: a
  page both select is one fetch, read by both rows in the step that fetches
  it;
* a decode layer whose ensure takes the global path (a pool above 2,048
  slots), from an empty pool.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import run
from oracle.lru import ERR_CAPACITY, ERR_PAGE_RANGE, LRUState
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu

TKV_ERR_PAGE_RANGE, TKV_ERR_CAPACITY, TKV_ERR_NOT_RESIDENT, TKV_ERR_BAD_MISS = 1, 2, 4, 8

EDGE = {
    "short": replace(get_workload("c4s"), name="edge_short_contexts", contexts=(1, 100, 130, 1000),
                     num_slots=128, num_layers=2, steps=4, topk=8, query="iid", setup_chunk=1024),
    "wide": replace(get_workload("c2s"), name="edge_topk_128", contexts=(16384,), topk=128, num_slots=512,
                    num_layers=2, steps=3, query="iid", setup_chunk=4096),
    "bf16": replace(get_workload("c1"), name="edge_bf16_batch", contexts=(700, 4096, 33), num_slots=160,
                    steps=4),
}


def _pair(wl):
    from workload.gpu_run import GpuWorkload
    g = GpuWorkload(wl)
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    return g, o


def _chain(wl, g, o, C=None):
    g.upload_queries()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, C or 0)
    for s in range(wl.steps):
        say(f"[edges] {wl.name} step {s}")
        g.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{wl.name} step {s} layer {layer}")
        compare_state(g, o, f"{wl.name} step {s}", check_rows=(s == wl.steps - 1))


@pytest.mark.parametrize("key", sorted(EDGE))
def test_decode_edges_bit_exact(key):
    wl = EDGE[key]
    say(f"[edges] {key}: {wl.name}")
    g, o = _pair(wl)
    compare_state(g, o, f"{wl.name} after setup")
    _chain(wl, g, o)
    if key == "short":
        sel = g.sel.cpu().numpy()
        assert (sel[:, 0, 1:] == -1).all(), "the one-page request pads its selection with -1"
    assert g.tier.read_counters()["error_word"] == 0


def test_decode_drops_when_the_cap_is_below_topk():
    wl = replace(get_workload("c3s"), name="edge_cap_5", num_layers=2, steps=3, query="iid")
    say("[edges] compaction width 5 < top-8")
    g, o = _pair(wl)
    C = 5
    B, L = wl.batch, wl.num_layers
    g.C = g.tier.set_select_width(B, wl.topk, C)
    g.needed = torch.full((L, B, C), -1, dtype=torch.int32, device="cuda")
    g.out_slots = torch.full((L, B * C), -1, dtype=torch.int32, device="cuda")
    g.miss = torch.zeros((L, B * C, 2), dtype=torch.int32, device="cuda")
    _chain(wl, g, o, C=C)
    c = g.tier.read_counters()
    assert c["drops"] == (wl.topk - C) * B * L * wl.steps, c["drops"]


def _small_tier(num_slots, max_width, layers=2):
    from tiered_kv_cache_indexer_amd import TieredKV
    return TieredKV(num_layers=layers, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                    kv_format="fp8", num_logical_pages=64, num_slots=num_slots, max_batch=1,
                    max_topk=8, max_pages_per_req=64, max_width=max_width)


def _ensure_both(t, lru, needed, no_fetch=None):
    W = len(needed)
    nd = torch.tensor(needed, dtype=torch.int32, device="cuda")
    out = torch.full((W,), -7, dtype=torch.int32, device="cuda")
    miss = torch.zeros((W, 2), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    nf = None if no_fetch is None else torch.tensor(no_fetch, dtype=torch.uint8, device="cuda")
    t.lru_ensure(nd, out, miss, cnt, no_fetch=nf)
    torch.cuda.synchronize()
    o_out, o_miss = lru.ensure(np.array(needed, dtype=np.int64), no_fetch)
    m = int(cnt.item())
    assert np.array_equal(out.cpu().numpy(), o_out), "out_slots"
    assert m == len(o_miss) and np.array_equal(miss[:m].cpu().numpy(), np.asarray(o_miss).reshape(-1, 2)), "misses"
    st = t.read_state()
    assert np.array_equal(st["page_to_slot"], lru.page_to_slot)
    assert np.array_equal(st["slot_to_page"], lru.slot_to_page)
    assert np.array_equal(st["stamp"], lru.stamp) and st["clock"] == lru.clock


def test_ensure_capacity_and_page_range_errors_match_oracle():
    say("[edges] ensure error words")
    S, N = 6, 64
    t = _small_tier(S, 16)
    lru = LRUState(N, S)
    _ensure_both(t, lru, [3, 4, 5])
    # seven distinct pages for six slots: nothing changes, every slot -1, error bit
    _ensure_both(t, lru, [10, 11, 12, 13, 14, 15, 16, 10])
    assert t.read_counters()["error_word"] == TKV_ERR_CAPACITY and lru.error_word == ERR_CAPACITY
    # ids out of range are skipped and flagged; the rest is served
    _ensure_both(t, lru, [4, N, -5, 20, -1, 21, 4])
    assert t.read_counters()["error_word"] == TKV_ERR_CAPACITY | TKV_ERR_PAGE_RANGE
    assert lru.error_word == ERR_CAPACITY | ERR_PAGE_RANGE
    _ensure_both(t, lru, [30, 31, 3, 20])


@pytest.mark.parametrize("S,N,widths", [(48, 160, (1, 130)), (200, 400, (300, 512)), (48, 160, (513, 700)),
                                         (2300, 2600, (40, 300))])
def test_ensure_random_traces_match_oracle(S, N, widths):
    from tiered_kv_cache_indexer_amd import TieredKV
    say(f"[edges] random ensure trace: {S} slots, {N} pages, widths {widths}")
    t = TieredKV(num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16, kv_format="bf16",
                 num_logical_pages=N, num_slots=S, max_batch=1, max_topk=8, max_pages_per_req=64,
                 max_width=widths[1])
    lru = LRUState(N, S)
    rng = np.random.default_rng([S, N, widths[1]])
    for call in range(40):
        W = int(rng.integers(widths[0], widths[1] + 1))
        # mostly a working set that fits the pool, sometimes one that does not
        ws = int(rng.integers(1, S + 1)) if call % 7 else int(rng.integers(S + 1, N + 1))
        base = rng.choice(N, size=min(ws, N), replace=False)
        needed = rng.choice(base, size=W).astype(np.int64)          # duplicates
        needed[rng.random(W) < 0.1] = -1                             # padding
        if call % 5 == 3:
            needed[int(rng.integers(W))] = N + int(rng.integers(3))  # out of range
        no_fetch = (rng.random(W) < 0.3).astype(np.uint8) if call % 2 else None
        _ensure_both(t, lru, needed.tolist(), no_fetch)
        assert t.read_counters()["error_word"] == lru.error_word, f"error word at call {call}"


def test_misaligned_rows_are_refused_before_any_launch():
    """bf16 rows are read in 16-byte vectors: a query or key buffer that is not
    16-byte aligned is an argument error, reported before anything runs."""
    from tiered_kv_cache_indexer_amd import TkvError
    say("[edges] misaligned q / k")
    t = _small_tier(16, 16)
    t.set_select_width(1, 4, 0)
    Hq, Hkv, d = 32, 4, 128
    qbuf = torch.zeros(1 + Hq * d, dtype=torch.bfloat16, device="cuda")
    q = qbuf[1:].view(1, Hq, d)                       # 2 bytes past an aligned address
    rs = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    bt = torch.arange(64, dtype=torch.int32, device="cuda").view(1, 64)
    npg = torch.tensor([8], dtype=torch.int32, device="cuda")
    sel = torch.full((1, 4), -1, dtype=torch.int32, device="cuda")
    needed = torch.full((1, t.C), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(TkvError, match="16-byte"):
        t.select_pages(0, q, rs, bt, npg, 4, sel, needed)
    kbuf = torch.zeros(1 + Hkv * d, dtype=torch.bfloat16, device="cuda")
    k = kbuf[1:].view(1, Hkv, d)
    v = torch.zeros(1, Hkv, d, dtype=torch.bfloat16, device="cuda")
    one = torch.tensor([0], dtype=torch.int32, device="cuda")
    with pytest.raises(TkvError, match="16-byte"):
        t.store_kv_mirror(0, k, v, one, one, torch.tensor([1], dtype=torch.int32, device="cuda"), one, 1, bt)
    torch.cuda.synchronize()
    assert t.read_counters()["error_word"] == 0


def test_fetch_skips_entries_outside_the_pool_or_page_space():
    say("[edges] fetch with bad miss entries")
    S, N = 6, 64
    t = _small_tier(S, 16)
    rb = t.row_bytes
    # give every mirror row distinct bytes through the write path's layout-free
    # view: the mirror is the library's pinned memory, written here directly
    import ctypes
    ptr = t.lib.tkv_mirror_host_ptr(t.ctx)
    mir = np.ctypeslib.as_array((ctypes.c_uint8 * (N * rb)).from_address(ptr)).reshape(N, rb)
    rng = np.random.default_rng(5)
    mir[:] = rng.integers(0, 256, size=mir.shape, dtype=np.uint8)
    before = t.pool_rows().clone()
    miss = torch.tensor([[2, 9], [S, 1], [1, N], [-1, 3], [4, 17]], dtype=torch.int32, device="cuda")
    cnt = torch.tensor([5], dtype=torch.int32, device="cuda")
    t.fetch_pages(miss, cnt)
    torch.cuda.synchronize()
    pool = t.pool_rows().cpu().numpy()
    assert np.array_equal(pool[2], mir[9]) and np.array_equal(pool[4], mir[17])
    for s in (0, 1, 3, 5):
        assert np.array_equal(pool[s], before[s].cpu().numpy()), f"slot {s} was written"
    assert t.read_counters()["error_word"] == TKV_ERR_BAD_MISS


def test_store_to_a_page_without_slot():
    """A full-page store to a page that is not resident: mirror row and slab
    take the new bytes (as the oracle's store does), the pool does not, and
    the error word says so."""
    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c3s"), name="edge_store_nonresident", num_layers=2, steps=1)
    say("[edges] store to a page without a slot")
    g, o = _pair(wl)
    bt, _ = gen.block_tables(wl)
    st = g.tier.read_state()
    page0 = int(bt[0][0])
    assert st["page_to_slot"][page0] < 0 and o.lru.page_to_slot[page0] < 0
    layer, n = 1, wl.page_size
    k = gen.kv_tokens(wl, gen.KIND_K, 0, 0, 64 * wl.page_size, n)     # other on-grid values
    v = gen.kv_tokens(wl, gen.KIND_V, 0, 0, 70 * wl.page_size, n)
    kt = torch.from_numpy(gen.to_bf16_bits(k).view(np.int16)).cuda().view(torch.bfloat16)
    vt = torch.from_numpy(gen.to_bf16_bits(v).view(np.int16)).cuda().view(torch.bfloat16)
    one = lambda x: torch.tensor([x], dtype=torch.int32, device="cuda")
    g.tier.store_kv_mirror(layer, kt, vt, one(0), one(0), one(n), one(0), n, g.bt)
    o.store(layer, [(0, 0, n)], k, v, bt)
    compare_state(g, o, "after the store", check_rows=True)
    assert g.tier.read_counters()["error_word"] == TKV_ERR_NOT_RESIDENT


def test_runs_longer_than_max_run_len_are_flagged():
    """A run whose device-side length spans more pages than the call's
    max_run_len reaches is reported, not silently cut: the write-ensure's
    samples miss a page and the store's grid does not reach the last one;
    both set the run-length bit (and the store to the page the ensure missed
    sets the not-resident bit)."""
    TKV_ERR_RUN_LEN = 16
    say("[edges] run longer than max_run_len")
    t = _small_tier(16, 16)
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    bt = torch.arange(64, dtype=torch.int32, device="cuda").view(1, 64)
    n = 3 * 64                                           # three pages on the device ...
    t.ensure_write_pages(i32([0]), i32([0]), i32([n]), 64, bt, i32([0]))   # ... max_run_len one page
    torch.cuda.synchronize()
    assert t.read_counters()["error_word"] == TKV_ERR_RUN_LEN
    st = t.read_state()
    assert st["page_to_slot"][0] >= 0 and st["page_to_slot"][2] >= 0 and st["page_to_slot"][1] < 0
    t.reset_residency()
    t.ensure_write_pages(i32([0]), i32([0]), i32([n]), n, bt, i32([0]))    # right length: all three
    torch.cuda.synchronize()
    assert t.read_counters()["error_word"] == 0
    k = torch.zeros(n, 4, 128, dtype=torch.bfloat16, device="cuda")
    t.store_kv_mirror(0, k, k, i32([0]), i32([0]), i32([n]), i32([0]), 64, bt)   # grid reaches 2 pages
    torch.cuda.synchronize()
    assert t.read_counters()["error_word"] == TKV_ERR_RUN_LEN


def test_binding_takes_the_compaction_width_from_the_library():
    """The buffers the binding sizes (needed [B][C], out_slots/miss [B*C])
    use the width the library set, read back through tkv_select_width, for
    the default (2*block_topk + 8, FreeToken PR #499 "Design") and an
    explicit max_sel_pages; a refused width leaves the old one."""
    from tiered_kv_cache_indexer_amd import TkvError
    t = _small_tier(64, 64)
    assert t.lib.tkv_select_width(t.ctx) == 0
    assert t.set_select_width(1, 8, 0) == 24 == t.lib.tkv_select_width(t.ctx) == t.C
    assert t.set_select_width(1, 8, 5) == 5 == t.lib.tkv_select_width(t.ctx) == t.C
    with pytest.raises(TkvError):
        t.set_select_width(1, 8, 65)                    # more than the 64 slots
    assert t.lib.tkv_select_width(t.ctx) == 5


def test_corrupted_mirror_byte_is_caught_after_refetch():
    """Failure forcing (FreeToken PR #525, commit summary: a mirror that held
    the wrong bytes corrupted fp8 pages with no error): one byte of a
    non-resident page's mirror row is flipped from the host, the page is
    fetched, and the pool-row byte compare against the oracle must report
    that slot -- at exactly that byte.  With the byte restored and the row
    fetched again, the compare passes."""
    import ctypes
    wl = replace(get_workload("c3s"), name="edge_mirror_corruption", num_layers=2, steps=1)
    say("[edges] corrupted mirror byte")
    g, o = _pair(wl)
    t = g.tier
    compare_state(g, o, "before the corruption")
    st = t.read_state()
    bt, _ = gen.block_tables(wl)
    page = next(int(p) for p in bt[0] if p >= 0 and st["page_to_slot"][p] < 0)
    off = t.layer_bytes + 1000                                   # layer 1, inside the K codes
    ptr = t.lib.tkv_mirror_host_ptr(t.ctx)
    mir = np.ctypeslib.as_array((ctypes.c_uint8 * (o.N * t.row_bytes)).from_address(ptr)).reshape(o.N, t.row_bytes)
    good = int(mir[page, off])
    mir[page, off] = good ^ 0x5A
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    miss = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    t.lru_ensure(i32([page]), out, miss, cnt)
    t.fetch_pages(miss, cnt)
    out_o, miss_o = o.ensure([page])
    o.fetch(miss_o)
    torch.cuda.synchronize()
    slot = int(out.item())
    assert slot == int(out_o[0]) >= 0
    row_g = t.pool_rows()[slot].cpu().numpy()
    diff = np.nonzero(row_g != o.pool_row(slot))[0]
    assert list(diff) == [off], diff                             # the compare sees exactly the flipped byte
    with pytest.raises(AssertionError, match=f"mirror row {page}"):
        compare_state(g, o, "after the corruption")
    mir[page, off] = good                                        # restore, fetch the row again into its slot
    t.fetch_pages(i32([[slot, page]]), i32([1]))
    o.fetch(np.array([[slot, page]]))
    compare_state(g, o, "after the restore")


def test_shared_prefix_pages_fetched_once_and_read_by_both_requests():
    """Two requests whose block tables share physical pages (request 1's first
    logical pages are request 0's pages: a shared prefix).  After a residency
    reset every selected page misses: a page both requests select is fetched
    once (its second needed entry is a duplicate, which takes the first
    occurrence's slot and fetch flag) and both rows read it in the step that
    fetches it -- through decode_layer, whose fetch rides in the attention
    launch (the missed pages' block of the layer read from the mirror and
    written back by every row that selected them), and through the split
    decode.  Against the oracle with the same block table."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c4s")
    say(f"[edges] shared prefix pages on {wl.name}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    bt, npg = gen.block_tables(wl)
    shared = int(npg[0])
    bt2 = bt.copy()
    bt2[1, :shared] = bt[0, :shared]
    g.bt = torch.from_numpy(np.ascontiguousarray(bt2, dtype=np.int32)).cuda()
    q = gen.decode_queries(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    side = torch.cuda.Stream()
    dups = 0
    for s in range(wl.steps):
        g.tier.reset_residency()
        o.reset_residency()
        if s % 2 == 0:
            g.decode_step(s)
        else:
            g.decode_step_split(s, side)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt2, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"shared prefix step {s} layer {layer}")
            need = rec["needed"]
            dups += len((set(need[0].tolist()) & set(need[1].tolist())) - {-1})
        compare_state(g, o, f"shared prefix step {s}")
    assert dups > 0, "no page was selected by both requests"


def test_decode_through_the_global_ensure_path_from_an_empty_pool():
    """A pool of 2,300 slots (above the LDS ensure's 2,048) sends the decode
    layer's ensure down the global first-occurrence path, which also writes
    the per-entry fetch flags the folded fetch reads: from an empty pool every
    selected page misses and is read from its mirror row by the attention
    that fetches it.  Against the oracle, state and pool rows included."""
    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c2s"), name="edge_global_ensure", num_slots=2300, steps=3)
    say(f"[edges] global ensure path on {wl.name}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    bt, npg = gen.block_tables(wl)
    q = gen.decode_queries(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    for s in range(wl.steps):
        if s == 0:
            g.tier.reset_residency()
            o.reset_residency()
        g.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"global ensure step {s} layer {layer}")
            if s == 0 and layer == 0:                 # (later layers hit the rows layer 0 fetched)
                assert len(rec["misses"]) == wl.topk, len(rec["misses"])
        compare_state(g, o, f"global ensure step {s}")
