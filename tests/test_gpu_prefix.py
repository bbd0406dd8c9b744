"""GPU parity of cold-prefix records and rehydration into the mirror
(FreeToken PR #525, "What the patch does", items 2-4).  A request's prefix
is saved, restored under another request's logical ids (resident ones get
unbound), and decoded through a block table pointing at the new ids:
records, mirror rows, slab, LRU state and every later layer equal the
oracle's; the moved request's selections and attention bits equal those of
an untouched run."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu


def test_prefix_save_restore_decode():
    from oracle.codecs import bf16_bits_from_f32
    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c4s"), contexts=(4096, 4000, 2048, 8192), steps=3)
    say("[prefix] save/restore on a batch-4 workload")
    g, ref = GpuWorkload(wl), GpuWorkload(wl)
    for x in (g, ref):
        x.setup()
        x.upload_queries()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    g.decode_step(0)
    ref.decode_step(0)
    for layer in range(wl.num_layers):
        o.decode_layer(layer, q[0, layer], rs, bt, npg, ctx, wl.topk)
    src, dst = bt[1, :npg[1]], bt[0, :npg[1]]
    assert np.any(o.lru.page_to_slot[dst] >= 0)
    recs = g.tier.prefix_save(src)
    orecs = o.prefix_save(src)
    L, E = wl.num_layers, wl.num_kv_heads * wl.head_dim
    rb = g.tier.row_bytes
    assert recs.shape == (len(src), rb + L * E * 10)
    for i, r in enumerate(orecs):
        assert np.array_equal(recs[i, :rb], r["row"]), f"record {i}: row"
        vals = recs[i, rb:rb + L * E * 2].view(np.uint16).reshape(L, -1)
        assert np.array_equal(vals, bf16_bits_from_f32(r["slab"]).reshape(L, -1)), f"record {i}: slab"
        sums = recs[i, rb + L * E * 2:].view(np.float64).reshape(L, -1)
        for layer, v in r["sums"].items():
            assert np.array_equal(sums[layer], v[0].reshape(-1)), f"record {i}: sums"
    assert any(r["sums"] for r in orecs)            # the partly written last page
    g.tier.prefix_restore(dst, recs)
    o.prefix_restore(dst, orecs)
    compare_state(g, o, "after restore")
    bt2 = bt.copy()
    bt2[1, :npg[1]] = dst
    g.bt = torch.from_numpy(bt2).cuda()
    for s in range(1, wl.steps):
        g.decode_step(s)
        ref.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt2, npg, ctx, wl.topk)
            compare_layer(g, rec, layer, f"step {s} layer {layer}")
            assert torch.equal(g.sel[layer][1], ref.sel[layer][1])
            assert torch.equal(g.out[layer][1], ref.out[layer][1])
        compare_state(g, o, f"step {s}")
    assert g.tier.read_counters()["error_word"] == 0


def test_prefix_restore_rejects_bad_ids():
    from tiered_kv_cache_indexer_amd import TkvError
    from workload.gpu_run import GpuWorkload
    g = GpuWorkload(get_workload("c1"))
    recs = g.tier.prefix_save([0, 1])
    with pytest.raises(TkvError, match="duplicates"):
        g.tier.prefix_restore([3, 3], recs)
    with pytest.raises(TkvError, match="out of"):
        g.tier.prefix_restore([3, 10 ** 6], recs)
