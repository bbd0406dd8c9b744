"""GPU parity of the prefill chunk (store with write-through, per-query causal
top-k from the matrix-core indexer, union compaction, ensure, fetch, causal
sparse attention) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import assert_close, bf16_to_f64, compare_state, say

pytestmark = pytest.mark.gpu


def _capture(store):
    def on_layer(layer, bufs):
        store.append({k: bufs[k].clone() for k in ("sel", "needed", "out_slots", "miss", "miss_count", "out")})
    return on_layer


@pytest.mark.parametrize("kernel,ranges,split", [(0, 0, False), (0, 16, False), (1, 0, False), (0, 0, True)],
                         ids=["auto", "auto-16-page-ranges", "vector", "auto-split-store"])
def test_prefill_small_bit_exact(kernel, ranges, split):
    """The chunk against the oracle; `split`: the stores' mirror writes of
    whole pages on a second stream (tkv_store_kv_mirror_split), everything
    else ordered after them by the library."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5s")
    say(f"[prefill] {wl.name} attention kernel {kernel}, range pages {ranges}, split store {split}")
    g = GpuWorkload(wl)
    g.tier.set_attn_kernel(kernel)
    g.tier.set_attn_range(ranges)
    g.setup()
    got = []
    g.prefill(on_layer=_capture(got), copy_stream=torch.cuda.Stream() if split else None)
    torch.cuda.synchronize()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    recs = run.prefill(wl, o)
    for layer, (gg, rec) in enumerate(zip(got, recs)):
        where = f"c5s layer {layer}"
        assert np.array_equal(gg["sel"].cpu().numpy(), rec["sel"]), f"{where}: sel"
        assert np.array_equal(gg["needed"].cpu().numpy(), rec["needed"]), f"{where}: needed"
        assert np.array_equal(gg["out_slots"].cpu().numpy(), rec["out_slots"]), f"{where}: out_slots"
        m = int(gg["miss_count"].item())
        assert np.array_equal(gg["miss"].cpu().numpy()[:m], rec["misses"]), f"{where}: misses"
        out = bf16_to_f64(gg["out"])
        ref = np.stack([rec["out"][r] for r in range(wl.prefill_tokens)])
        assert_close(out, ref, f"{where}: attention")
    compare_state(g, o, "c5s after the chunk")


def test_matrix_core_scores_equal_scan_scores():
    """The prefill path (MFMA indexer) and the decode scan give the same
    selections for the same causal rows."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5s")
    say("[prefill] MFMA vs scan selections")
    g = GpuWorkload(wl)
    g.setup()
    bufs = g.prefill()
    t = g.tier
    layer = wl.num_layers - 1
    n = wl.prefill_tokens
    sel_mfma = bufs["sel"].clone()
    one = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    sel1 = torch.empty((1, wl.topk), dtype=torch.int32, device="cuda")
    need1 = torch.empty((1, g.C if g.C else wl.max_sel_pages), dtype=torch.int32, device="cuda")
    for r in [0, 1, 63, 64, 200, n - 1]:
        t.select_pages(layer, bufs["q"][r:r + 1], one, g.bt, g.n_pages, wl.topk, sel1, need1,
                       row_pos=bufs["row_pos"][r:r + 1])
        torch.cuda.synchronize()
        assert torch.equal(sel1[0], sel_mfma[r]), r


def test_multi_row_requests_union_and_drops():
    """Several requests with several causal rows each in one select call (the
    scan path): per-row selections, the per-request unions (ascending, first C
    kept) and the drop counter equal the oracle's.  Row counts straddle the
    64-row groups of the union bitmaps.  Then the unions' ensure and fetch and
    every row's attention."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c4s")
    counts = [70, 1, 130, 65]
    rows = sum(counts)
    say(f"[prefill] multi-row select on {wl.name}, rows {counts}")
    g = GpuWorkload(wl, max_rows=rows)
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    t = g.tier
    C = g.C                                   # 2*topk + 8: most unions overflow it
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    layer = wl.num_layers - 1
    q = gen.prefill_queries(wl, layer, 0, rows)
    ctx = gen.context_lengths(wl)
    rng = np.random.default_rng(5)
    row_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_pos = np.concatenate([np.sort(rng.integers(0, int(ctx[b]), counts[b])) for b in range(wl.batch)])
    row_pos = row_pos.astype(np.int32)
    bt, npg = gen.block_tables(wl)
    bias = gen.page_bias(wl)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    qd = dev(gen.to_bf16_bits(q).view(np.int16)).view(torch.bfloat16)
    sel = torch.full((rows, wl.topk), -7, dtype=torch.int32, device="cuda")
    needed = torch.full((wl.batch, C), -7, dtype=torch.int32, device="cuda")
    drops0 = t.read_counters()["drops"]
    for rep in range(2):      # the bitmaps are cleared after use: a second call gives the same
        t.select_pages(layer, qd, dev(row_start), g.bt, g.n_pages, wl.topk, sel, needed,
                       page_bias=g.bias, row_pos=dev(row_pos))
        torch.cuda.synchronize()
        ref_sel, ref_needed = o.select(layer, q, row_start, row_pos, bt, npg, wl.topk, bias=bias)
        assert np.array_equal(sel.cpu().numpy(), ref_sel), f"call {rep}: sel"
        assert np.array_equal(needed.cpu().numpy(), ref_needed), f"call {rep}: needed"
    drops = t.read_counters()["drops"] - drops0
    assert drops == o.drops > 0
    # the unions made resident, then every row's attention through the rows
    # kernel (266 rows: the last row group of its workgroups is ragged);
    # pages dropped from a union are not resident and are skipped
    W = wl.batch * C
    out_slots = torch.full((W,), -7, dtype=torch.int32, device="cuda")
    miss = torch.zeros((W, 2), dtype=torch.int32, device="cuda")
    miss_count = torch.zeros((1,), dtype=torch.int32, device="cuda")
    t.lru_ensure(needed.view(-1), out_slots, miss, miss_count)
    t.fetch_pages(miss, miss_count)
    out = torch.zeros((rows, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    t.sparse_paged_attn(layer, qd, dev(row_start), g.ctx_len, sel, g.bt, out, row_pos=dev(row_pos))
    torch.cuda.synchronize()
    ref_slots, ref_misses = o.ensure(ref_needed)
    o.fetch(ref_misses)
    assert np.array_equal(out_slots.cpu().numpy(), ref_slots), "out_slots"
    m = int(miss_count.item())
    assert np.array_equal(miss.cpu().numpy()[:m], ref_misses), "misses"
    ref = o.attention(layer, q, row_start, row_pos, ctx, ref_sel, bt)
    assert_close(bf16_to_f64(out), ref, "multi-row attention")


@pytest.mark.parametrize("pages", [7, 16, 64])
def test_range_passes_equal_single_pass(pages):
    """The multi-pass prefill attention (one launch per range of local page
    ids, softmax state carried in fp32 records) gives the single pass's bits,
    including rows whose pages skip ranges and ragged last ranges."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5s")
    say(f"[prefill] range passes of {pages} pages vs one pass")
    g = GpuWorkload(wl)
    g.setup()
    bufs = g.prefill()
    torch.cuda.synchronize()
    t = g.tier
    layer = wl.num_layers - 1
    outs = []
    for rp in (0, pages):
        t.set_attn_range(rp)
        out = torch.full_like(bufs["out"], 7.0)
        t.sparse_paged_attn(layer, bufs["q"], bufs["row_start"], bufs["ctx_len"], bufs["sel"], g.bt, out,
                            row_pos=bufs["row_pos"])
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], bufs["out"])


def test_split_store_page_evicted_and_fetched_before_its_mirror_copy():
    """A page a split store began is evicted and fetched again before any
    attention call enqueued the store's deferred mirror copy: the ensure
    completes the page's mirror row from the staging copy, so the fetched
    pool row holds the stored bytes (checked before anything waits for the
    copy), and after the copy the whole state equals the oracle's."""
    from dataclasses import replace

    from workload import gpu_gen
    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c5s"), name="c5_small_prefill_tiny_pool", num_slots=24, setup_chunk=1024)
    say(f"[prefill] {wl.name}: split store, evict, refetch before the mirror copy")
    g = GpuWorkload(wl)
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    t = g.tier
    PS = wl.page_size
    start, n = wl.contexts[0], wl.prefill_tokens
    bt, _ = gen.block_tables(wl)
    i32 = lambda xs: torch.tensor(list(xs), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    t.ensure_write_pages(i32([0]), i32([start]), i32([n]), n, g.bt, i32([start]))
    o.ensure_write_pages([(0, start, n)], bt, [start])
    layer = 1
    k = gpu_gen.tokens(wl, gen.KIND_K, layer, 0, start, n)
    v = gpu_gen.tokens(wl, gen.KIND_V, layer, 0, start, n)
    t.store_kv_mirror(layer, k, v, i32([0]), i32([start]), i32([n]), i32([0]), n, g.bt, copy_stream=side)
    run.store_run(o, layer, 0, start, n, gen.kv_tokens(wl, gen.KIND_K, layer, 0, start, n),
                  gen.kv_tokens(wl, gen.KIND_V, layer, 0, start, n), bt)
    chunk = [int(p) for p in bt[0, start // PS:(start + n) // PS]]
    others = [int(p) for p in bt[0, :start // PS]][:wl.num_slots]
    W = wl.num_slots
    out_slots = torch.full((W,), -1, dtype=torch.int32, device="cuda")
    miss = torch.zeros((W, 2), dtype=torch.int32, device="cuda")
    miss_count = torch.zeros(1, dtype=torch.int32, device="cuda")
    for needed in (others, chunk):          # every slot rebound, then the chunk's pages missed again
        t.lru_ensure(i32(needed), out_slots[:len(needed)], miss, miss_count)
        t.fetch_pages(miss, miss_count, width=len(needed))
        _, misses = o.ensure(np.array(needed, dtype=np.int64))
        o.fetch(misses)
        torch.cuda.synchronize()
        m = int(miss_count.item())
        assert np.array_equal(miss[:m].cpu().numpy(), misses), f"misses of {needed}"
    assert {int(p) for p in misses[:, 1]} == set(chunk)
    pool = t.pool_rows()
    for p in chunk:
        s = int(o.lru.page_to_slot[p])
        assert s >= 0, f"page {p} not resident in the oracle"
        assert np.array_equal(pool[s].cpu().numpy(), o.pool_row(s)), f"pool row of page {p} (slot {s})"
    compare_state(g, o, "after the mirror copy")


def test_split_store_pending_rows_reach_host_tail_and_flush():
    """A split store's deferred mirror copy reached before any attention over
    the pool: host-tail attention over pages the pool no longer holds (it
    enqueues the copy and waits for it, then reads the stored rows from the
    mirror), and tkv_mirror_flush (after which the mirror, read directly,
    holds the stored rows)."""
    from dataclasses import replace

    from workload import gpu_gen
    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c5s"), name="c5_small_prefill_tiny_pool", num_slots=24, setup_chunk=1024)
    say(f"[prefill] {wl.name}: split store, then host-tail attention and a flush before the mirror copy")
    g = GpuWorkload(wl)
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    t = g.tier
    PS = wl.page_size
    start, n = wl.contexts[0], wl.prefill_tokens
    bt, _ = gen.block_tables(wl)
    i32 = lambda xs: torch.tensor(list(xs), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    chunk = [int(p) for p in bt[0, start // PS:(start + n) // PS]]
    others = [int(p) for p in bt[0, :start // PS]][:wl.num_slots]

    def split_store(layer, old):
        t.ensure_write_pages(i32([0]), i32([start]), i32([n]), n, g.bt, i32([old]))
        o.ensure_write_pages([(0, start, n)], bt, [old])
        k = gpu_gen.tokens(wl, gen.KIND_K, layer, 0, start, n)
        v = gpu_gen.tokens(wl, gen.KIND_V, layer, 0, start, n)
        t.store_kv_mirror(layer, k, v, i32([0]), i32([start]), i32([n]), i32([0]), n, g.bt, copy_stream=side)
        run.store_run(o, layer, 0, start, n, gen.kv_tokens(wl, gen.KIND_K, layer, 0, start, n),
                      gen.kv_tokens(wl, gen.KIND_V, layer, 0, start, n), bt)

    layer = 1
    split_store(layer, start)
    out_slots = torch.full((len(others),), -1, dtype=torch.int32, device="cuda")
    miss = torch.zeros((len(others), 2), dtype=torch.int32, device="cuda")
    miss_count = torch.zeros(1, dtype=torch.int32, device="cuda")
    t.lru_ensure(i32(others), out_slots, miss, miss_count)        # the chunk's pages leave the pool
    t.fetch_pages(miss, miss_count)
    _, misses = o.ensure(np.array(others, dtype=np.int64))
    o.fetch(misses)
    assert not any(o.lru.page_to_slot[p] >= 0 for p in chunk)
    # rows at the chunk's last position, each selecting the chunk's pages
    rows = 8
    q = gen.prefill_queries(wl, layer, 0, n)[:rows]
    qd = torch.from_numpy(gen.to_bf16_bits(q).view(np.int16)).cuda().view(torch.bfloat16)
    sel = np.full((rows, wl.topk), -1, dtype=np.int32)
    sel[:, :len(chunk)] = np.arange(start // PS, start // PS + len(chunk))
    pos = np.full(rows, start + n - 1)
    out = torch.zeros((rows, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    t.sparse_paged_attn(layer, qd, i32([0, rows]), i32([start + n]), torch.from_numpy(sel).cuda(), g.bt, out,
                        row_pos=i32(pos), host_tail=True)
    torch.cuda.synchronize()
    ref = o.attention(layer, q, np.array([0, rows]), pos, np.array([start + n]), sel, bt, host_tail=True)
    assert_close(bf16_to_f64(out), ref, "host-tail attention over the split-stored pages")
    # the chunk's pages back (their rows fetched), another split store, then a flush
    split_store(0, start + n)
    t.mirror_flush()
    torch.cuda.synchronize()
    mir = t.mirror()
    for p in chunk:
        assert np.array_equal(mir[p], o.mirror_row(p)), f"mirror row {p} after the flush"
    compare_state(g, o, "after the flush")
