"""Drive the oracle tier over a synthetic workload.

Setup: each request's context is written through the tier's own write path
in ``setup_chunk``-token runs, request by request: one ensure_write_pages
per run, then store for every layer.  Decode steps then start from whatever
the LRU holds.  A prefill workload then writes its chunk (one write-ensure,
then per layer: store, select with causal rows, ensure, fetch, attention).
"""
from __future__ import annotations

import numpy as np

from workload import gen
from workload.configs import Workload

from .engine import OracleTier
from .store import write_tokens


def make_tier(wl: Workload, materialize: bool) -> OracleTier:
    tier = OracleTier(num_layers=wl.num_layers, num_q_heads=wl.num_q_heads,
                      num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
                      page_size=wl.page_size, fp8=(wl.kv_format == "fp8"),
                      num_logical_pages=wl.num_logical_pages, num_slots=wl.num_slots,
                      materialize=materialize)
    bt, npg = gen.block_tables(wl)
    owner = {}
    for b in range(wl.batch):
        for lp in range(npg[b]):
            owner[int(bt[b, lp])] = (b, lp)
    cache = {}

    def row_builder(page: int) -> np.ndarray:
        if page in cache:
            return cache[page]
        row = np.zeros(tier.lay.row_bytes, dtype=np.uint8)
        n = int(tier.written[page])
        if n > 0:
            b, lp = owner[page]
            for layer in range(wl.num_layers):
                k = gen.kv_page(wl, gen.KIND_K, layer, b, lp)[:n]
                v = gen.kv_page(wl, gen.KIND_V, layer, b, lp)[:n]
                write_tokens(row, tier.lay, layer, 0, k, v)
        if len(cache) > 4096:
            cache.clear()
        cache[page] = row
        return row

    tier.row_builder = row_builder
    return tier


def setup(wl: Workload, tier: OracleTier) -> None:
    bt, _ = gen.block_tables(wl)
    for b, ctx in enumerate(wl.contexts):
        written = 0
        for start in range(0, ctx, wl.setup_chunk):
            length = min(wl.setup_chunk, ctx - start)
            old_len = [0] * wl.batch
            old_len[b] = written
            tier.ensure_write_pages([(b, start, length)], bt, old_len)
            for layer in range(wl.num_layers):
                k = gen.kv_tokens(wl, gen.KIND_K, layer, b, start, length)
                v = (gen.kv_tokens(wl, gen.KIND_V, layer, b, start, length)
                     if tier.materialize else None)
                store_run(tier, layer, b, start, length, k, v, bt)
            written += length


def store_run(tier, layer, b, start, length, k, v, bt):
    if v is None:
        v = np.zeros_like(k)
    tier.store(layer, [(b, start, length)], k, v, bt)


def append_token(wl: Workload, tier: OracleTier, s: int, layer: int, bt):
    """Write step s's appended token of every request for one layer: the
    write-ensure of its page, then the store (write-through, slab update).

    Reading taken: the write-ensure runs for each layer right before that
    layer's store (a batched call over the requests), so the target page is
    resident when it is written even if earlier layers' ensures evicted it;
    the request's old length counts the new token as present once layer 0
    has written it, so a page that holds earlier layers' bytes is fetched,
    never allocated blank."""
    ctx = gen.context_lengths(wl)
    runs = [(b, int(ctx[b]) + s, 1) for b in range(wl.batch)]
    old = [int(ctx[b]) + s + (1 if layer > 0 else 0) for b in range(wl.batch)]
    tier.ensure_write_pages(runs, bt, old)
    k = np.concatenate([gen.kv_tokens(wl, gen.KIND_K, layer, b, int(ctx[b]) + s, 1) for b in range(wl.batch)])
    v = np.concatenate([gen.kv_tokens(wl, gen.KIND_V, layer, b, int(ctx[b]) + s, 1) for b in range(wl.batch)])
    tier.store(layer, runs, k, v, bt)


def decode(wl: Workload, tier: OracleTier, steps=None, attention=False, on_layer=None):
    """Run decode steps; returns a list over steps of lists over layers of the
    per-layer record (sel, needed, out_slots, misses[, out]).  Appending
    workloads write each step's new token before every layer's selection and
    attend over the grown context."""
    bt, npg = gen.block_tables(wl)
    ctx = gen.context_lengths(wl)
    bias = gen.page_bias(wl)
    q = gen.decode_queries(wl)
    row_start = np.arange(wl.batch + 1)
    tier.set_select_width(wl.batch, wl.topk, wl.max_sel_pages)
    trace = []
    nsteps = wl.steps if steps is None else steps
    for s in range(nsteps):
        per_layer = []
        if wl.append:
            ctx, npg = gen.append_lengths(wl, s)
        for layer in range(wl.num_layers):
            if wl.append:
                append_token(wl, tier, s, layer, bt)
            rec = tier.decode_layer(layer, q[s, layer], row_start, bt, npg, ctx, wl.topk,
                                    bias=bias, with_attention=attention)
            if on_layer is not None:
                on_layer(s, layer, rec)
            per_layer.append(rec)
        trace.append(per_layer)
    return trace


def prefill(wl: Workload, tier: OracleTier, attention_rows=None, on_layer=None):
    """The prefill chunk of request 0.  attention_rows: None = all rows,
    otherwise a list of chunk-relative row indices to attend."""
    assert wl.prefill_tokens > 0 and wl.batch == 1
    bt, npg = gen.block_tables(wl)
    start, n = wl.contexts[0], wl.prefill_tokens
    tier.ensure_write_pages([(0, start, n)], bt, [start])
    tier.set_select_width(1, wl.topk, wl.max_sel_pages)
    ctx = np.array([start + n], dtype=np.int32)
    row_pos = np.arange(start, start + n, dtype=np.int64)
    row_start = np.array([0, n])
    recs = []
    for layer in range(wl.num_layers):
        k = gen.kv_tokens(wl, gen.KIND_K, layer, 0, start, n)
        v = gen.kv_tokens(wl, gen.KIND_V, layer, 0, start, n)
        store_run(tier, layer, 0, start, n, k, v, bt)
        q = gen.prefill_queries(wl, layer, 0, n)
        sel, needed = tier.select(layer, q, row_start, row_pos, bt, npg, wl.topk)
        out_slots, misses = tier.ensure(needed)
        tier.fetch(misses)
        rows = range(n) if attention_rows is None else attention_rows
        out = {r: tier.attention_row(layer, q[r], 0, sel[r], bt, ctx, row_pos[r]) for r in rows}
        rec = dict(sel=sel, needed=needed, out_slots=out_slots, misses=misses, out=out)
        if on_layer is not None:
            on_layer(layer, rec)
        recs.append(rec)
    return recs
