"""GPU parity of the decode layer with its fused row copy issued in two
parts (FreeToken PR #499, "Design": one copy per miss carries the page for
every layer): the decoded layer's slice first, the rest of the rows on a
copy stream beside the attention and the next layer's selection.  The
oracle is the plain decode layer: selections, compaction, slot maps, miss
lists, LRU state, counters, slab, mirror and pool rows bit-exact, attention
within tolerance."""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu


def _oracle(wl):
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    return o


@pytest.mark.parametrize("key", ["c2s", "c3s", "c4s", "c3sc", "c4sc"])
def test_split_chain(key):
    """c3sc and c4sc have pools of three times the batch width, so each call's
    copies chain on the previous call's; the others take the full wait."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[split] {key}")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = _oracle(wl)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    side = torch.cuda.Stream()
    for s in range(wl.steps):
        say(f"[split] {key} step {s}")
        g.decode_step_split(s, side)
        torch.cuda.current_stream().synchronize()      # the step joined the copy stream
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{key} step {s} layer {layer}")
        compare_state(g, o, f"{key} step {s}", check_rows=True)
    assert g.tier.read_counters()["error_word"] == 0


def test_split_chain_from_an_empty_pool():
    """A 12-layer chain (top-24, a pool of three call widths) whose pool is
    emptied after setup: the first call misses every page it selects (24
    misses of 11 parts of 64 KiB each, enough for the rest copy's
    claimed-pieces path), later calls fewer (its dealt-items path); every
    layer against the oracle, pool and mirror rows included."""
    from dataclasses import replace

    from workload.gpu_run import GpuWorkload
    wl = replace(get_workload("c3sc"), name="c3_small_thrash_chain_12_layers", num_layers=12, steps=2, topk=24,
                 num_slots=168)
    say(f"[split] {wl.name} from an empty pool")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = _oracle(wl)
    g.tier.reset_residency()
    o.reset_residency()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    side = torch.cuda.Stream()
    misses = []
    for s in range(wl.steps):
        g.decode_step_split(s, side)
        torch.cuda.current_stream().synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{wl.name} step {s} layer {layer}")
            misses.append(len(rec["misses"]))
        compare_state(g, o, f"{wl.name} step {s}", check_rows=True)
    assert misses[0] == wl.topk and max(misses) * 11 >= 12 * 16   # claimed pieces (12 items per workgroup)
    assert min(misses) * 11 < 12 * 16                                # dealt items
    assert g.tier.read_counters()["error_word"] == 0


def test_split_then_plain_calls_wait_for_the_rest_copy():
    """Split calls for all but the last layer, no join by the caller; the last
    layer through the plain decode_layer, which orders its copy after the
    pending rest copy.  After the main stream alone is synchronised the pool
    rows must be complete."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3sc")
    say("[split] split then plain, c3sc")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = _oracle(wl)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    side = torch.cuda.Stream()
    L = wl.num_layers
    for s in range(2):
        for layer in range(L):
            args = (layer, g.q[s, layer], g.bt, g.n_pages, g.ctx_len, wl.topk, g.sel[layer], g.needed[layer],
                    g.out_slots[layer], g.miss[layer], g.miss_count[layer], g.out[layer])
            if layer < L - 1:
                g.tier.decode_layer_split(*args, side, page_bias=g.bias)
            else:
                g.tier.decode_layer(*args, page_bias=g.bias)
        torch.cuda.current_stream().synchronize()
        for layer in range(L):
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"c3sc step {s} layer {layer}")
        compare_state(g, o, f"c3sc step {s}", check_rows=True)


def test_split_calls_out_of_layer_order():
    """Layers visited 0, 2, 1, 3, 4 each step: calls that do not follow the
    previous call's layer take the full wait; results follow the oracle run
    in the same order."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3sc")
    say("[split] out-of-order layers, c3sc")
    g = GpuWorkload(wl)
    g.setup()
    g.upload_queries()
    o = _oracle(wl)
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    side = torch.cuda.Stream()
    order = [0, 2, 1, 3, 4]
    assert sorted(order) == list(range(wl.num_layers))
    for s in range(4):
        for layer in order:
            g.tier.decode_layer_split(layer, g.q[s, layer], g.bt, g.n_pages, g.ctx_len, wl.topk, g.sel[layer],
                                      g.needed[layer], g.out_slots[layer], g.miss[layer], g.miss_count[layer],
                                      g.out[layer], side, page_bias=g.bias)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.current_stream().synchronize()
        for layer in order:
            rec = o.decode_layer(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"c3sc step {s} layer {layer}")
        compare_state(g, o, f"c3sc step {s}", check_rows=True)


OUTS = ("sel", "needed", "out_slots", "miss_count", "out")


def test_split_steps_capture_and_replay_like_eager():
    """Split steps captured in a HIP graph (the copy stream forks from the
    capture stream and is joined at the end of the step) replay exactly like
    the same steps run eagerly; eager work runs between the replays."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3sc")
    say("[split] graph capture, c3sc")
    eager, graphed = GpuWorkload(wl), GpuWorkload(wl)
    for g in (eager, graphed):
        g.setup()
        g.upload_queries()
    torch.cuda.synchronize()
    side_e, side_g = torch.cuda.Stream(), torch.cuda.Stream()
    graphs = []
    for s in range(wl.steps):
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            graphed.decode_step_split(s, side_g)
        graphs.append(cg)
    torch.cuda.synchronize()
    for s in range(wl.steps):
        eager.decode_step_split(s, side_e)
        graphs[s].replay()
        _ = graphed.tier.read_counters()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(getattr(eager, k), getattr(graphed, k)), f"step {s}: {k}"
    sa, sb = eager.tier.read_state(), graphed.tier.read_state()
    for k in ("page_to_slot", "slot_to_page", "stamp"):
        assert np.array_equal(sa[k], sb[k]), k
    ca, cb = eager.tier.read_counters(), graphed.tier.read_counters()
    assert ca == cb and ca["error_word"] == 0
    assert torch.equal(eager.tier.pool_rows(), graphed.tier.pool_rows())


def test_fetch_halves_match_fetch_pages():
    """select_pages -> lru_ensure -> fetch_pages_layer -> fetch_pages_rest ->
    sparse_paged_attn on one stream gives the fused decode_layer's results
    and pool bytes."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3sc")
    say("[split] fetch halves vs fetch_pages, c3sc")
    a, b = GpuWorkload(wl), GpuWorkload(wl)
    a.setup()
    b.setup()
    a.upload_queries()
    b.upload_queries()
    t = b.tier
    rs = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    for s in range(3):
        a.decode_step(s)
        for layer in range(wl.num_layers):
            q = b.q[s, layer]
            t.select_pages(layer, q, rs, b.bt, b.n_pages, wl.topk, b.sel[layer], b.needed[layer],
                           page_bias=b.bias)
            t.lru_ensure(b.needed[layer].view(-1), b.out_slots[layer], b.miss[layer], b.miss_count[layer])
            t.fetch_pages_layer(b.miss[layer], b.miss_count[layer], layer)
            t.fetch_pages_rest(b.miss[layer].shape[0], layer)
            t.sparse_paged_attn(layer, q, rs, b.ctx_len, b.sel[layer], b.bt, b.out[layer])
        torch.cuda.synchronize()
        for name in ("sel", "needed", "out_slots", "miss_count"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
        assert torch.equal(a.out, b.out)
        assert torch.equal(a.tier.pool_rows(), b.tier.pool_rows())
    assert a.tier.read_counters() == b.tier.read_counters()
