"""GPU parity of the decode layer with a top-k preload (vLLM RFC #33980,
"Topk KV preload"): layer l first preloads the page list layer l+1 needed
last time, the copy running on a second stream under layer l's selection.
Everything is compared with the oracle's ensure+fetch of the same list
followed by its decode layer: selections, compaction, slot maps, miss
lists, LRU state, counters, slab, mirror and pool rows bit-exact, attention
within tolerance."""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", ["c3s", "c4s"])
def test_prefetch_chain(key):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[prefetch] {key}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    C = o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    last = [np.full((wl.batch, C), -1, dtype=np.int32) for _ in range(wl.num_layers)]
    side = torch.cuda.Stream()
    L = wl.num_layers
    for s in range(wl.steps):
        say(f"[prefetch] {key} step {s}")
        g.decode_step_prefetch(s, side)
        torch.cuda.synchronize()
        for layer in range(L):
            rec = o.decode_layer_prefetch(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, last[(layer + 1) % L],
                                          bias=bias)
            last[layer] = rec["needed"]
            compare_layer(g, rec, layer, f"{key} step {s} layer {layer}")
        compare_state(g, o, f"{key} step {s}")
    assert g.tier.read_counters()["error_word"] == 0
