"""GPU parity of the host tail read in place (vLLM RFC #33980, discussion:
KV beyond the HBM tier is host memory the attention kernel loads over the
interconnect, without a staging copy).

Against the oracle: selections and compaction bit-exact, attention within
tolerance, and no residency state moves.  Against the fetch path of the same
library: identical attention bits (the mirror rows hold the pool's bytes and
both read them with the same kernel arithmetic).
"""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import assert_close, bf16_to_f64, say

pytestmark = pytest.mark.gpu

KERNELS = {"auto": 0, "vector": 1}


@pytest.mark.parametrize("key,kernel", [("c1", "auto"), ("c3s", "auto"), ("c4s", "auto"), ("c3s", "vector")])
def test_host_tail_decode_chain(key, kernel):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[host-tail] {key} ({kernel} attention)")
    g, f = GpuWorkload(wl), GpuWorkload(wl)          # host tail, fetch path
    for x in (g, f):
        x.tier.set_attn_kernel(KERNELS[kernel])
        x.setup()
        x.upload_queries()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    st0 = g.tier.read_state()
    c0 = g.tier.read_counters()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    rs = np.arange(wl.batch + 1)
    non_resident = 0
    for s in range(wl.steps):
        g.decode_step_host_tail(s)
        f.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            where = f"{key} step {s} layer {layer}"
            rec = o.decode_layer_host_tail(layer, q[s, layer], rs, bt, npg, ctx, wl.topk, bias=bias)
            assert np.array_equal(g.sel[layer].cpu().numpy(), rec["sel"]), f"{where}: sel"
            assert np.array_equal(g.needed[layer].cpu().numpy(), rec["needed"]), f"{where}: needed"
            assert_close(bf16_to_f64(g.out[layer]), rec["out"], f"{where}: attention")
            assert torch.equal(g.sel[layer], f.sel[layer]), f"{where}: sel vs fetch path"
            assert torch.equal(g.out[layer], f.out[layer]), f"{where}: attention bits vs fetch path"
            sel = rec["sel"]
            for b in range(wl.batch):
                for i in sel[b]:
                    if i >= 0 and o.lru.page_to_slot[bt[b][i]] < 0:
                        non_resident += 1
    assert non_resident > 0, "no page was read from the host"
    st1 = g.tier.read_state()
    for k in ("page_to_slot", "slot_to_page", "stamp", "clock"):
        assert np.array_equal(st0[k], st1[k]), k
    c1 = g.tier.read_counters()
    for k in ("ensure_calls", "hits", "misses", "evictions", "bytes_fetched", "error_word"):
        assert c0[k] == c1[k], k
    say(f"[host-tail] {key}: {non_resident} selected pages read from the host")


def test_host_tail_prefill_rows_with_empty_pool():
    """Wave-per-row attention over a prefill chunk with nothing resident: every
    page comes from the mirror, and the output bits equal those of the chunk's
    own attention over the pool."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c5s")
    say("[host-tail] c5s prefill rows, empty pool")
    g = GpuWorkload(wl)
    g.setup()
    bufs = g.prefill()
    torch.cuda.synchronize()
    ref = bufs["out"].clone()
    t = g.tier
    t.reset_residency()
    out = torch.zeros_like(ref)
    layer = wl.num_layers - 1
    t.sparse_paged_attn(layer, bufs["q"], bufs["row_start"], bufs["ctx_len"], bufs["sel"], g.bt, out,
                        row_pos=bufs["row_pos"], host_tail=True)
    torch.cuda.synchronize()
    assert not np.any(t.read_state()["page_to_slot"] >= 0)
    assert torch.equal(out, ref)
