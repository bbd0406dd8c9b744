"""GPU parity on general bf16 inputs (keys, values and queries N(0,1) rounded
to bf16, not on the workloads' grids), stage by stage, against the oracle.

* store: fp8 codes and scales of every token, mirror and pool rows, and the
  slab (its key sums are fp64 on both sides and certified exact) bit-exact;
* decode selection: the scores' fp64 sums are certified exact (53 bits), so
  selections, slot maps, misses and LRU state are bit-exact;
* prefill selection (the dense bf16 product with fp32 accumulation, as the
  chunk config describes it): off the grids fp32 sums round, so the rows are
  checked against the oracle's exact keys within the accumulation bound --
  every selected page within the bound of the k-th key, every other page too;
* attention, fed the oracle's own selection, on the matrix-core and vector
  kernels, within 2e-2 abs + 1e-2 rel -- including query rows whose values
  span 2^-14 .. 2^2 (the matrix-core kernel's two-part fp8 query keeps about
  8 significant bits relative to the row's largest value).
"""
import numpy as np
import pytest
import torch

from oracle import run
from oracle.select import group_query, keys_from_scores, page_scores
from workload import gen, get_workload

from tests.gpu_compare import assert_close, bf16_to_f64, compare_layer, compare_state, say

pytestmark = pytest.mark.gpu

KERNELS = {"auto": 0, "vector": 1, "matrix": 2}


def _pair(key, kernel="auto"):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[offgrid] {key} ({kernel} attention): {wl.name}")
    g = GpuWorkload(wl)
    g.tier.set_attn_kernel(KERNELS[kernel])
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    return wl, g, o


def _bf16_dev(x):
    return torch.from_numpy(gen.to_bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)


def _wide(q, rng):
    """Each element scaled by 2^-j, j uniform in 0..14 (exact in bf16)."""
    j = rng.integers(0, 15, size=q.shape)
    return (q * np.ldexp(1.0, -j)).astype(np.float32)


@pytest.mark.parametrize("key,kernel", [("c2s_bf16", "auto"), ("c3s_bf16", "auto"), ("c3s_bf16", "vector")])
def test_offgrid_decode_chain_bit_exact(key, kernel):
    """The whole decode chain on general bf16 inputs: store bytes and slab
    after setup, selections, compaction, slot maps, misses, LRU state and
    counters bit-exact every layer of every step; attention in tolerance."""
    wl, g, o = _pair(key, kernel)
    compare_state(g, o, f"{key} after setup")
    g.upload_queries()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    for s in range(wl.steps):
        say(f"[offgrid] {key} step {s}")
        g.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{key} step {s} layer {layer}")
        compare_state(g, o, f"{key} step {s}", check_rows=(s == wl.steps - 1))
    say(f"[offgrid] {key}: score bits needed <= {o.max_score_bits:.1f} (fp64 sums exact below 53)")
    assert 24 <= o.max_score_bits < 53           # off the fp32 exactness range, inside fp64's
    assert o.counters()["error_word"] == 0


@pytest.mark.parametrize("kernel", ["auto", "vector"])
def test_offgrid_decode_attention_wide_range_queries(kernel):
    """Decode rows whose values span 2^-14 .. 2^2: the selection (fp64 sums)
    is still bit-exact and attention over the oracle's selection stays in
    tolerance on both kernels."""
    wl, g, o = _pair("c2s_bf16", kernel)
    rng = np.random.default_rng(77)
    q = _wide(gen.decode_queries(wl)[:3], rng)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    t = g.tier
    assert wl.num_logical_pages <= wl.num_slots             # every page resident: no ensure needed
    rs_d = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    sel = torch.empty((wl.batch, wl.topk), dtype=torch.int32, device="cuda")
    need = torch.empty((wl.batch, g.C), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    for s in range(q.shape[0]):
        for layer in range(wl.num_layers):
            where = f"wide q step {s} layer {layer}"
            qd = _bf16_dev(q[s, layer])
            sel_o, need_o = o.select(layer, q[s, layer], rs, None, bt, npg, wl.topk)
            t.select_pages(layer, qd, rs_d, g.bt, g.n_pages, wl.topk, sel, need)
            torch.cuda.synchronize()
            assert np.array_equal(sel.cpu().numpy(), sel_o), f"{where}: sel"
            assert np.array_equal(need.cpu().numpy(), need_o), f"{where}: needed"
            sel.copy_(torch.from_numpy(sel_o).cuda())
            t.sparse_paged_attn(layer, qd, rs_d, g.ctx_len, sel, g.bt, out)
            torch.cuda.synchronize()
            ref = o.attention(layer, q[s, layer], rs, None, ctx, sel_o, bt)
            assert_close(bf16_to_f64(out), ref, f"{where}: attention ({kernel})")


def _selection_within_bound(sel_row, keys, visible, k, delta):
    """GPU row: a valid selection (ascending, distinct, visible, min(k,
    visible) pages), every selected key >= kth - delta and every other key
    <= kth + delta, where kth is the oracle's k-th largest exact key."""
    chosen = sel_row[sel_row >= 0]
    assert np.all(sel_row[len(chosen):] == -1) and np.all(np.diff(chosen) > 0)
    assert len(chosen) == min(k, visible) and (len(chosen) == 0 or chosen[-1] < visible)
    if visible <= k:
        return True
    kth = np.sort(keys[:visible].astype(np.float64))[::-1][k - 1]
    rest = np.setdiff1d(np.arange(visible), chosen)
    return bool(np.all(keys[chosen] >= kth - delta) and np.all(keys[rest] <= kth + delta))


@pytest.mark.parametrize("kernel", ["auto", "vector"])
def test_offgrid_prefill_stagewise(kernel):
    """Prefill chunk on general bf16 inputs, stage by stage: the chunk's store
    (bytes and slab) bit-exact; the matrix-core indexer's selections within
    the fp32 accumulation bound of the oracle's exact keys; attention fed the
    oracle's selection (a quarter of the rows with values spanning 2^-14 ..
    2^2) in tolerance on every row of every layer."""
    wl, g, o = _pair("c5s_bf16", kernel)
    t = g.tier
    assert wl.num_logical_pages <= wl.num_slots              # every page resident after the write-ensure
    bt, npg = gen.block_tables(wl)
    start, n = wl.contexts[0], wl.prefill_tokens
    bufs = g.prefill_buffers()
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    t.ensure_write_pages(i32([0]), i32([start]), i32([n]), n, g.bt, i32([start]))
    o.ensure_write_pages([(0, start, n)], bt, [start])
    t.set_select_width(1, wl.topk, wl.max_sel_pages)
    o.set_select_width(1, wl.topk, wl.max_sel_pages)
    o.check_scores = False                                   # chunk rows off the grid: compared by bound
    ctx = np.array([start + n])
    row_pos = np.arange(start, start + n)
    rs = np.array([0, n])
    rng = np.random.default_rng(5)
    exact_rows = 0
    for layer in range(wl.num_layers):
        k = gen.kv_tokens(wl, gen.KIND_K, layer, 0, start, n)
        v = gen.kv_tokens(wl, gen.KIND_V, layer, 0, start, n)
        t.store_kv_mirror(layer, _bf16_dev(k), _bf16_dev(v), i32([0]), i32([start]), i32([n]), i32([0]), n, g.bt)
        run.store_run(o, layer, 0, start, n, k, v, bt)
        compare_state(g, o, f"c5s_bf16 layer {layer} after the chunk's store", check_rows=(layer == wl.num_layers - 1))
        q = gen.prefill_queries(wl, layer, 0, n)
        t.select_pages(layer, _bf16_dev(q), bufs["row_start"], g.bt, g.n_pages, wl.topk, bufs["sel"],
                       bufs["needed"], row_pos=bufs["row_pos"])
        sel_o, _ = o.select(layer, q, rs, row_pos, bt, npg, wl.topk)
        sel_g = bufs["sel"].cpu().numpy()
        slab = o.slab[layer][bt[0, :npg[0]]]
        for r in range(n):
            visible = min(int(npg[0]), int(row_pos[r]) // wl.page_size + 1)
            qg = group_query(q[r], wl.num_kv_heads)
            keys = keys_from_scores(page_scores(qg, slab[:visible]), None)
            absq = np.abs(qg.astype(np.float64)).reshape(-1)
            A = float((np.abs(slab[:visible].astype(np.float64)).reshape(visible, -1) @ absq).max())
            delta = 512 * 2.0 ** -24 * A + 2.0 ** -23 * float(np.abs(keys).max(initial=0.0))
            assert _selection_within_bound(sel_g[r], keys, visible, wl.topk, delta), f"layer {layer} row {r}"
            exact_rows += int(np.array_equal(sel_g[r], sel_o[r]))
        qw = q.copy()
        wide_rows = rng.choice(n, n // 4, replace=False)
        qw[wide_rows] = _wide(q[wide_rows], rng)
        bufs["sel"].copy_(torch.from_numpy(sel_o).cuda())
        t.sparse_paged_attn(layer, _bf16_dev(qw), bufs["row_start"], bufs["ctx_len"], bufs["sel"], g.bt,
                            bufs["out"], row_pos=bufs["row_pos"])
        torch.cuda.synchronize()
        ref = o.attention(layer, qw, rs, row_pos, ctx, sel_o, bt)
        assert_close(bf16_to_f64(bufs["out"]), ref, f"c5s_bf16 layer {layer}: attention ({kernel})")
    say(f"[offgrid] prefill rows with the oracle's exact selection: {exact_rows} of {n * wl.num_layers}")
