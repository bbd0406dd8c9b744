"""GPU parity: the HIP tier through the C ABI against the oracle, on the same
seeded inputs.

Small workloads (every layer of every step, every byte): selections,
compaction, slot maps, miss lists, LRU state, counters, slab, mirror and pool
bytes bit-exact; attention within 2e-2 abs + 1e-2 rel.
"""
import numpy as np
import pytest
import torch

from oracle import run
from workload import gen, get_workload

from tests.gpu_compare import compare_layer, compare_state, say

pytestmark = pytest.mark.gpu


KERNELS = {"auto": 0, "vector": 1, "matrix": 2}


def _pair(key, kernel="auto"):
    from workload.gpu_run import GpuWorkload
    wl = get_workload(key)
    say(f"[parity] {key} ({kernel} attention): {wl.description or wl.name}")
    g = GpuWorkload(wl)
    g.tier.set_attn_kernel(KERNELS[kernel])
    g.setup()
    o = run.make_tier(wl, materialize=True)
    run.setup(wl, o)
    return wl, g, o


@pytest.mark.parametrize("key,kernel", [("c1", "auto"), ("c2s", "auto"), ("c3s", "auto"), ("c4s", "auto"),
                                        ("c3s", "vector"), ("c4s", "vector")])
def test_decode_chain_bit_exact(key, kernel):
    """Fixed-point results bit-exact, attention within tolerance; `auto` runs
    the matrix-core attention kernel on the fp8 configs, `vector` the other."""
    wl, g, o = _pair(key, kernel)
    compare_state(g, o, f"{key} after setup")
    g.upload_queries()
    q = gen.decode_queries(wl)
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    row_start = np.arange(wl.batch + 1)
    o.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    for s in range(wl.steps):
        say(f"[parity] {key} step {s}")
        g.decode_step(s)
        torch.cuda.synchronize()
        for layer in range(wl.num_layers):
            rec = o.decode_layer(layer, q[s, layer], row_start, bt, npg, ctx, wl.topk, bias=bias)
            compare_layer(g, rec, layer, f"{key} step {s} layer {layer}")
        compare_state(g, o, f"{key} step {s}", check_rows=(s == wl.steps - 1))
    assert o.counters()["error_word"] == 0


def test_unfused_entry_points_match_fused_step():
    """select_pages -> lru_ensure -> fetch_pages -> sparse_paged_attn gives the
    fused decode_layer's results (and both follow the oracle)."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3s")
    say("[parity] unfused vs fused on c3s")
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
            t.fetch_pages(b.miss[layer], b.miss_count[layer])
            t.sparse_paged_attn(layer, q, rs, b.ctx_len, b.sel[layer], b.bt, b.out[layer])
        torch.cuda.synchronize()
        for name in ("sel", "needed", "out_slots", "miss_count"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
        assert torch.equal(a.out, b.out)
    sa, sb = a.tier.read_state(), b.tier.read_state()
    for k in ("page_to_slot", "slot_to_page", "stamp"):
        assert np.array_equal(sa[k], sb[k])


def test_matrix_attention_refused_where_it_does_not_apply():
    from tiered_kv_cache_indexer_amd import TkvError
    from workload.gpu_run import GpuWorkload
    g = GpuWorkload(get_workload("c1"))          # bf16, 16-token pages
    with pytest.raises(TkvError, match="matrix-core"):
        g.tier.set_attn_kernel(2)
    g.tier.set_attn_kernel(1)
    g.tier.set_attn_kernel(0)


def test_codecs_match_oracle():
    from oracle.codecs import e4m3_decode, e4m3_encode
    from workload.gpu_run import GpuWorkload
    say("[parity] e4m3 codecs")
    g = GpuWorkload(get_workload("c1"))
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    dec = g.tier.e4m3_decode(codes).cpu().numpy()
    ref = e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = ~np.isnan(ref)
    assert np.array_equal(dec[fin], ref[fin]) and np.all(np.isnan(dec[~fin]))
    assert np.array_equal(np.signbit(dec[fin]), np.signbit(ref[fin]))
    # encoder: every fp32 bit pattern with exponent in the e4m3 range, strided,
    # plus all midpoints and their neighbours, plus specials
    rng = np.random.default_rng(0)
    pats = np.arange(0, 2 ** 32, 4099, dtype=np.uint64).astype(np.uint32)
    vals = pats.view(np.float32)
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    mids = (e4m3_decode(np.arange(0x7E, dtype=np.uint8)).astype(np.float64) +
            e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8)).astype(np.float64)) / 2
    m32 = mids.astype(np.float32)
    extra = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                            -m32, rng.standard_normal(100000).astype(np.float32) * 100,
                            np.array([0.0, -0.0, 448.0, 464.0, -464.0, 1e-45, np.inf, -np.inf],
                                     dtype=np.float32)])
    allv = np.concatenate([vals, extra]).astype(np.float32)
    allv = allv[~np.isnan(allv)]
    got = g.tier.e4m3_encode(torch.from_numpy(allv).cuda()).cpu().numpy()
    exp = e4m3_encode(allv)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {allv[bad[:5]]} -> {got[bad[:5]]} vs {exp[bad[:5]]}"


def test_gpu_generator_matches_numpy():
    from workload import gpu_gen
    say("[parity] Philox generator")
    for key, kind, layer, req, start, count in [("c2", 0, 3, 0, 0, 200), ("c2", 1, 11, 0, 4000, 300),
                                                ("c4", 0, 5, 2, 12345, 77), ("c1", 1, 0, 0, 17, 40),
                                                ("c5", 2, 7, 0, 100, 130), ("c2s_bf16", 0, 1, 0, 0, 200),
                                                ("c3s_bf16", 1, 2, 0, 640, 65), ("c5s_bf16", 2, 1, 0, 64, 130)]:
        wl = get_workload(key)
        got = gpu_gen.tokens(wl, kind, layer, req, start, count).float().cpu().numpy()
        if kind == gen.KIND_Q:
            ref = gen.prefill_queries(wl, layer, start, count)
        else:
            ref = gen.kv_tokens(wl, kind, layer, req, start, count)
        assert np.array_equal(got, ref), (key, kind, layer, req, start, count)
