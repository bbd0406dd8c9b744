"""Feed a synthetic workload to the HIP tier (setup, decode steps, prefill).

The same procedure as ``oracle/run.py`` on the oracle side: each request's
context is written through the tier's write path in ``setup_chunk``-token
runs (one ensure_write_pages per run, then store_kv_mirror for every layer),
then decode steps call decode_layer for every layer in order.  Keys, values
and prefill queries are generated on the GPU (``gpu_gen``); decode queries,
block tables and the page bias come from ``gen`` and are uploaded once.
"""
from __future__ import annotations

import numpy as np
import torch

from tiered_kv_cache_indexer_amd import TieredKV

from . import gen, gpu_gen
from .configs import Workload


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype=dtype, device="cuda")


class GpuWorkload:
    def __init__(self, wl: Workload, max_rows: int | None = None):
        self.wl = wl
        B = wl.batch
        C = wl.max_sel_pages
        bt, npg = gen.block_tables(wl)
        self.bt_np, self.npg_np = bt, npg
        self.bt = _dev(bt, torch.int32)
        self.n_pages = _dev(npg, torch.int32)
        self.ctx_len = _dev(gen.context_lengths(wl), torch.int32)
        bias = gen.page_bias(wl)
        self.bias = None if bias is None else _dev(bias, torch.float32)
        spr = wl.setup_chunk // wl.page_size + 2
        width = max(B * C, spr, (wl.prefill_tokens // wl.page_size + 2) if wl.prefill_tokens else 1)
        self.tier = TieredKV(
            num_layers=wl.num_layers, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
            head_dim=wl.head_dim, page_size=wl.page_size, kv_format=wl.kv_format,
            num_logical_pages=wl.num_logical_pages, num_slots=wl.num_slots, max_batch=B,
            max_rows=max(B, wl.prefill_tokens, max_rows or 0), max_topk=wl.topk, max_pages_per_req=wl.max_pages,
            max_width=width)
        self.C = self.tier.set_select_width(B, wl.topk, wl.max_sel_pages)
        L = wl.num_layers
        self.sel = torch.full((L, B, wl.topk), -1, dtype=torch.int32, device="cuda")
        self.needed = torch.full((L, B, self.C), -1, dtype=torch.int32, device="cuda")
        self.out_slots = torch.full((L, B * self.C), -1, dtype=torch.int32, device="cuda")
        self.miss = torch.zeros((L, B * self.C, 2), dtype=torch.int32, device="cuda")
        self.miss_count = torch.zeros((L, 1), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((L, B, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        self.q = None
        self.row_start = torch.arange(B + 1, dtype=torch.int32, device="cuda")

    # -------------------------------------------------------------- setup --
    def setup(self):
        wl, t = self.wl, self.tier
        chunk = wl.setup_chunk
        k = torch.empty((chunk, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        for b, ctx in enumerate(wl.contexts):
            written = 0
            for start in range(0, ctx, chunk):
                n = min(chunk, ctx - start)
                self._write_run(b, start, n, written, k, v)
                written += n

    def _write_run(self, b, start, n, old, k, v, layers=None):
        wl, t = self.wl, self.tier
        run_req = torch.tensor([b], dtype=torch.int32, device="cuda")
        run_start = torch.tensor([start], dtype=torch.int32, device="cuda")
        run_len = torch.tensor([n], dtype=torch.int32, device="cuda")
        run_off = torch.zeros(1, dtype=torch.int32, device="cuda")
        old_len = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
        old_len[b] = old
        t.ensure_write_pages(run_req, run_start, run_len, n, self.bt, old_len)
        for layer in (range(wl.num_layers) if layers is None else layers):
            gpu_gen.tokens(wl, gen.KIND_K, layer, b, start, n, out=k[:n])
            gpu_gen.tokens(wl, gen.KIND_V, layer, b, start, n, out=v[:n])
            t.store_kv_mirror(layer, k[:n], v[:n], run_req, run_start, run_len, run_off, n, self.bt)

    # ------------------------------------------------------------- decode --
    def upload_queries(self):
        q = gen.decode_queries(self.wl)                     # [steps][L][B][Hq][d] fp32 on grid
        self.q = _dev(gen.to_bf16_bits(q).view(np.int16), torch.int16).view(torch.bfloat16)
        return self.q

    def decode_step(self, s, q=None, stream=None):
        wl = self.wl
        q = self.q if q is None else q
        for layer in range(wl.num_layers):
            self.tier.decode_layer(layer, q[s, layer], self.bt, self.n_pages, self.ctx_len, wl.topk,
                                   self.sel[layer], self.needed[layer], self.out_slots[layer],
                                   self.miss[layer], self.miss_count[layer], self.out[layer],
                                   page_bias=self.bias, stream=stream)

    def decode_step_split(self, s, copy_stream, q=None, stream=None, join=True):
        """One decode step through decode_layer_split: each layer's missed rows
        copy their other layers on `copy_stream`, beside that layer's attention
        and the next layer's selection.  With `join`, `stream` waits for the
        copy stream at the end of the step (pool complete in stream order)."""
        wl = self.wl
        q = self.q if q is None else q
        for layer in range(wl.num_layers):
            self.tier.decode_layer_split(layer, q[s, layer], self.bt, self.n_pages, self.ctx_len, wl.topk,
                                         self.sel[layer], self.needed[layer], self.out_slots[layer],
                                         self.miss[layer], self.miss_count[layer], self.out[layer],
                                         copy_stream, page_bias=self.bias, stream=stream)
        if join:
            (stream or torch.cuda.current_stream()).wait_stream(copy_stream)

    def decode_step_prefetch(self, s, copy_stream, q=None, stream=None):
        """One decode step where layer l first preloads the page list layer
        l+1 needed last time (the next step's layer 0 for the last layer),
        its copy on `copy_stream` overlapping layer l's selection."""
        wl = self.wl
        q = self.q if q is None else q
        L = wl.num_layers
        for layer in range(L):
            self.tier.decode_layer_prefetch(layer, q[s, layer], self.bt, self.n_pages, self.ctx_len, wl.topk,
                                            self.sel[layer], self.needed[layer], self.out_slots[layer],
                                            self.miss[layer], self.miss_count[layer], self.out[layer],
                                            self.needed[(layer + 1) % L].view(-1), page_bias=self.bias,
                                            stream=stream, copy_stream=copy_stream)

    # ------------------------------------------------------------- append --
    def append_kv(self, steps=None):
        """Keys and values of the appended tokens, generated on the GPU:
        bf16 [2][steps][L][B][Hkv][d] (token of step s at position ctx + s)."""
        wl = self.wl
        steps = wl.steps if steps is None else steps
        kv = torch.empty((2, steps, wl.num_layers, wl.batch, wl.num_kv_heads, wl.head_dim),
                         dtype=torch.bfloat16, device="cuda")
        for s in range(steps):
            for layer in range(wl.num_layers):
                for b in range(wl.batch):
                    for i, kind in enumerate((gen.KIND_K, gen.KIND_V)):
                        gpu_gen.tokens(wl, kind, layer, b, wl.contexts[b] + s, 1, out=kv[i, s, layer, b:b + 1])
        return kv

    def decode_step_append(self, s, kv, q=None, stream=None):
        """One decode step that appends one token per request: per layer, a
        batched write-ensure of the new tokens' pages, their store (write-
        through), then the fused decode layer over the grown context.  The
        old length counts the new token once layer 0 has written it."""
        wl, t = self.wl, self.tier
        q = self.q if q is None else q
        if not hasattr(self, "_run_req"):
            B = wl.batch
            self._run_req = torch.arange(B, dtype=torch.int32, device="cuda")
            self._run_one = torch.ones(B, dtype=torch.int32, device="cuda")
        start = self.ctx_len + s
        ctx_s = start + 1
        npg_s = torch.div(ctx_s + (wl.page_size - 1), wl.page_size, rounding_mode="floor").to(torch.int32)
        for layer in range(wl.num_layers):
            t.ensure_write_pages(self._run_req, start, self._run_one, 1, self.bt, start if layer == 0 else ctx_s,
                                 stream=stream)
            t.store_kv_mirror(layer, kv[0, s, layer], kv[1, s, layer], self._run_req, start, self._run_one,
                              self._run_req, 1, self.bt, stream=stream)
            t.decode_layer(layer, q[s, layer], self.bt, npg_s, ctx_s, wl.topk, self.sel[layer],
                           self.needed[layer], self.out_slots[layer], self.miss[layer], self.miss_count[layer],
                           self.out[layer], page_bias=self.bias, stream=stream)

    def decode_step_host_tail(self, s, q=None, stream=None):
        """One decode step with the host tail read in place: per layer,
        select_pages then the attention that reads non-resident pages from
        their mirror rows.  No ensure, no fetch: the pool does not change."""
        wl, t = self.wl, self.tier
        q = self.q if q is None else q
        for layer in range(wl.num_layers):
            t.select_pages(layer, q[s, layer], self.row_start, self.bt, self.n_pages, wl.topk, self.sel[layer],
                           self.needed[layer], page_bias=self.bias, stream=stream)
            t.sparse_paged_attn(layer, q[s, layer], self.row_start, self.ctx_len, self.sel[layer], self.bt,
                                self.out[layer], stream=stream, host_tail=True)

    # ------------------------------------------------------------ prefill --
    def prefill_buffers(self):
        wl = self.wl
        n = wl.prefill_tokens
        C = wl.max_sel_pages
        return dict(
            sel=torch.full((n, wl.topk), -1, dtype=torch.int32, device="cuda"),
            needed=torch.full((1, C), -1, dtype=torch.int32, device="cuda"),
            out_slots=torch.full((C,), -1, dtype=torch.int32, device="cuda"),
            miss=torch.zeros((C, 2), dtype=torch.int32, device="cuda"),
            miss_count=torch.zeros(1, dtype=torch.int32, device="cuda"),
            out=torch.zeros((n, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda"),
            q=torch.empty((n, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda"),
            k=torch.empty((n, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda"),
            v=torch.empty((n, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda"),
            row_start=torch.tensor([0, n], dtype=torch.int32, device="cuda"),
            row_pos=torch.arange(wl.contexts[0], wl.contexts[0] + n, dtype=torch.int32, device="cuda"),
            ctx_len=torch.tensor([wl.contexts[0] + n], dtype=torch.int32, device="cuda"),
        )

    def prefill(self, bufs=None, on_layer=None, copy_stream=None):
        """The prefill chunk of request 0: one write-ensure, then per layer
        store -> select (causal rows) -> ensure -> fetch -> attention.  With
        `copy_stream`, the stores are split: whole pages' mirror writes run on
        that stream beside the layer's attention."""
        wl, t = self.wl, self.tier
        bufs = bufs or self.prefill_buffers()
        start, n = wl.contexts[0], wl.prefill_tokens
        run_req = torch.tensor([0], dtype=torch.int32, device="cuda")
        run_start = torch.tensor([start], dtype=torch.int32, device="cuda")
        run_len = torch.tensor([n], dtype=torch.int32, device="cuda")
        run_off = torch.zeros(1, dtype=torch.int32, device="cuda")
        old_len = torch.tensor([start], dtype=torch.int32, device="cuda")
        t.ensure_write_pages(run_req, run_start, run_len, n, self.bt, old_len)
        t.set_select_width(1, wl.topk, wl.max_sel_pages)
        for layer in range(wl.num_layers):
            gpu_gen.tokens(wl, gen.KIND_K, layer, 0, start, n, out=bufs["k"])
            gpu_gen.tokens(wl, gen.KIND_V, layer, 0, start, n, out=bufs["v"])
            t.store_kv_mirror(layer, bufs["k"], bufs["v"], run_req, run_start, run_len, run_off, n, self.bt,
                              copy_stream=copy_stream)
            gpu_gen.tokens(wl, gen.KIND_Q, layer, 0, 0, n, out=bufs["q"])
            t.select_pages(layer, bufs["q"], bufs["row_start"], self.bt, self.n_pages, wl.topk,
                           bufs["sel"], bufs["needed"], row_pos=bufs["row_pos"])
            t.lru_ensure(bufs["needed"].view(-1), bufs["out_slots"], bufs["miss"], bufs["miss_count"])
            t.fetch_pages(bufs["miss"], bufs["miss_count"])
            t.sparse_paged_attn(layer, bufs["q"], bufs["row_start"], bufs["ctx_len"], bufs["sel"], self.bt,
                                bufs["out"], row_pos=bufs["row_pos"])
            if on_layer is not None:
                on_layer(layer, bufs)
        return bufs
