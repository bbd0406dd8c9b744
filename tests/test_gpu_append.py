"""GPU parity of decode with one appended token per request per step
(FreeToken PR #499, Design: the write-ensure precedes store_kv, which writes
through to the mirror).  Per layer: batched write-ensure, store, fused
decode layer over the grown context.  Selections, compaction, slot maps,
miss lists, LRU state, counters, slab, mirror and pool rows bit-exact;
attention within tolerance."""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", ["c3sa", "c4sa"])
def test_append_chain(key):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[append] {key}: {wl.name}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    kv = g.append_kv()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    compare_state(g, o, f"{key} after setup")
    q = gen.decode_queries(wl)
    bt, _ = gen.block_tables(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    for s in range(wl.steps):
        say(f"[append] {key} step {s}")
        g.decode_step_append(s, kv)
        torch.cuda.synchronize()
        ctx, npg = gen.append_lengths(wl, s)
        for layer in range(wl.num_layers):
            run.append_token(wl, o, s, layer, bt)
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{key} step {s} layer {layer}")
        compare_state(g, o, f"{key} step {s}")
    c = g.tier.read_counters()
    assert c["error_word"] == 0 and c["fresh_allocs"] > 0
