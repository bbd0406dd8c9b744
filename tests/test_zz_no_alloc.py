"""tkv_prefix_restore_noalloc against tkv_prefix_restore: two tiers brought
to the same state, one restoring through each entry point, compared byte for
byte (mirror rows, slab values and fp64 key sums via saved records, LRU
state, counters) after two calls in a row -- the first spanning several
passes of the fixed staging array, the second smaller, so whatever the first
left in the array must not leak into the second."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from workload import gen, get_workload

from tests.gpu_compare import say

pytestmark = pytest.mark.gpu


def _tier_pair(wl):
    from workload.gpu_run import GpuWorkload
    pair = []
    for _ in range(2):
        g = GpuWorkload(wl)
        g.setup()
        g.upload_queries()
        g.decode_step(0)
        pair.append(g)
    torch.cuda.synchronize()
    return pair


def _same(a, b, dst, where):
    ta, tb = a.tier, b.tier
    torch.cuda.synchronize()
    assert np.array_equal(ta.mirror(), tb.mirror()), f"{where}: mirror"
    assert np.array_equal(ta.prefix_save(dst), tb.prefix_save(dst)), f"{where}: records (row, slab, sums)"
    assert torch.equal(ta.slab_view(), tb.slab_view()), f"{where}: slab"
    sa, sb = ta.read_state(), tb.read_state()
    for k in ("page_to_slot", "slot_to_page", "stamp"):
        assert np.array_equal(sa[k], sb[k]), f"{where}: {k}"
    assert sa["clock"] == sb["clock"]
    assert ta.read_counters() == tb.read_counters(), f"{where}: counters"


# 12 layers x 4 KV heads x d 128: 34 pages of slab entries per staging pass;
# 193 pages, the last one partly written (its key sums travel in the records)
WL = replace(get_workload("c2s"), name="noalloc_12_layers", num_layers=12, contexts=(12320,), num_slots=200,
             steps=2)


def test_noalloc_restore_matches_restore():
    wl = WL
    say(f"[noalloc] {wl.name}: two tiers, restore vs restore_noalloc")
    a, b = _tier_pair(wl)
    bt, npg = gen.block_tables(wl)
    assert npg[0] == 193 and wl.contexts[0] % wl.page_size                 # a partly written last page
    calls = [(bt[0, 113:193], bt[0, 0:80]),                                   # 80 pages: three staging passes
             (bt[0, 150:170], bt[0, 90:110])]                                 # then 20: one pass
    for i, (src, dst) in enumerate(calls):
        say(f"[noalloc] call {i}: {len(src)} records")
        recs = a.tier.prefix_save(src)
        assert np.array_equal(recs, b.tier.prefix_save(src))
        a.tier.prefix_restore(dst, recs)
        b.tier.prefix_restore(dst, recs, noalloc=True)
        _same(a, b, dst, f"after call {i}")
    # the restored pages decode the same way through both tiers
    for g in (a, b):
        g.decode_step(1)
    torch.cuda.synchronize()
    assert torch.equal(a.sel, b.sel) and torch.equal(a.needed, b.needed) and torch.equal(a.out, b.out)
    _same(a, b, bt[0, 0:80], "after a decode step")


def test_noalloc_restore_rejects_duplicates_and_bad_ids():
    from tiered_kv_cache_indexer_amd import TkvError
    wl = WL
    a, _ = _tier_pair(wl)
    bt, _ = gen.block_tables(wl)
    recs = a.tier.prefix_save(bt[0, 40:43])
    with pytest.raises(TkvError, match="duplicates"):
        a.tier.prefix_restore(np.array([bt[0, 0], bt[0, 1], bt[0, 0]]), recs, noalloc=True)
    with pytest.raises(TkvError, match="out of"):
        a.tier.prefix_restore(np.array([0, 1, wl.num_logical_pages]), recs, noalloc=True)
