"""PyTorch-facing binding: device buffers come from torch, every call goes to
the C ABI with the same name (select_pages, lru_ensure, fetch_pages,
sparse_paged_attn, decode_layer, ensure_write_pages, store_kv_mirror)."""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from ._lib import (KV_BF16, KV_FP8, KV_NVFP4, Config, Counters, DeviceBuffers, Sizes, check,
                   load)

_FORMATS = {"bf16": KV_BF16, "fp8": KV_FP8, "nvfp4": KV_NVFP4}


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class TieredKV:
    """One tier: pinned host mirror (owned by the library) + device pool, slab,
    residency state and workspace (allocated here with torch)."""

    def __init__(self, *, num_layers, num_q_heads, num_kv_heads, head_dim, page_size, kv_format,
                 num_logical_pages, num_slots, max_batch=1, max_rows=None, max_topk=64,
                 max_pages_per_req=None, max_width=None, device="cuda"):
        self.lib = load()
        if not torch.cuda.is_available():
            raise RuntimeError("TieredKV needs a GPU (gfx950); none is visible")
        fmt = _FORMATS.get(kv_format, kv_format)
        max_rows = max_rows or max_batch
        max_pages_per_req = max_pages_per_req or num_logical_pages
        max_width = max_width or max(num_slots, 1)
        self.cfg = Config(num_layers, num_q_heads, num_kv_heads, head_dim, page_size, fmt,
                          num_logical_pages, num_slots, max_batch, max_rows, max_topk,
                          max_pages_per_req, min(max_width, 65535))
        self.sizes = Sizes()
        check(self.lib.tkv_required_bytes(C.byref(self.cfg), C.byref(self.sizes)))
        ctx = C.c_void_p()
        check(self.lib.tkv_create(C.byref(self.cfg), C.byref(ctx)))
        self.ctx = ctx
        self.device = torch.device(device)
        s = self.sizes

        def buf(n):
            t = torch.empty(max(int(n), 256), dtype=torch.uint8, device=self.device)
            assert t.data_ptr() % 256 == 0
            return t

        self.pool = buf(s.pool_bytes)
        self.slab = buf(s.slab_bytes)
        self.state = buf(s.state_bytes)
        self.workspace = buf(s.workspace_bytes)
        self._bufs = DeviceBuffers(self.pool.data_ptr(), self.slab.data_ptr(), self.state.data_ptr(),
                                   self.workspace.data_ptr())
        check(self.lib.tkv_attach_device(self.ctx, C.byref(self._bufs), _stream(None)))
        self.row_bytes = int(s.row_bytes)
        self.layer_bytes = int(s.layer_bytes)
        self.C = None

    # ------------------------------------------------------------ lifetime --
    def close(self):
        if getattr(self, "ctx", None):
            torch.cuda.synchronize()
            self.lib.tkv_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ config ----
    def set_select_width(self, max_bs, block_topk, max_sel_pages=0):
        check(self.lib.tkv_set_select_width(self.ctx, max_bs, block_topk, max_sel_pages))
        self.C = int(self.lib.tkv_select_width(self.ctx))   # the width the library set
        return self.C

    def reset_residency(self, stream=None):
        check(self.lib.tkv_reset_residency(self.ctx, _stream(stream)))

    # ------------------------------------------------------------ calls -----
    def select_pages(self, layer, q, row_start, block_table, n_pages, topk, sel_local, needed,
                     row_pos=None, page_bias=None, stream=None):
        rows = q.shape[0]
        B = n_pages.shape[0]
        check(self.lib.tkv_select_pages(
            self.ctx, layer, _ptr(q, torch.bfloat16, "q"), rows, _ptr(row_start, torch.int32, "row_start"),
            _ptr(row_pos, torch.int32, "row_pos"), _ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1], _ptr(n_pages, torch.int32, "n_pages"), B,
            _ptr(page_bias, torch.float32, "page_bias"), topk, _ptr(sel_local, torch.int32, "sel_local"),
            _ptr(needed, torch.int32, "needed"), _stream(stream)))

    def lru_ensure(self, needed, out_slots, miss, miss_count, no_fetch=None, stream=None):
        check(self.lib.tkv_lru_ensure(
            self.ctx, _ptr(needed, torch.int32, "needed"), needed.numel(),
            _ptr(no_fetch, torch.uint8, "no_fetch"), _ptr(out_slots, torch.int32, "out_slots"),
            _ptr(miss, torch.int32, "miss"), _ptr(miss_count, torch.int32, "miss_count"), _stream(stream)))

    def fetch_pages(self, miss, miss_count, width=None, stream=None):
        width = width or miss.shape[0]
        check(self.lib.tkv_fetch_pages(self.ctx, _ptr(miss, torch.int32, "miss"),
                                       _ptr(miss_count, torch.int32, "miss_count"), width, _stream(stream)))

    def fetch_pages_layer(self, miss, miss_count, layer, width=None, stream=None):
        width = width or miss.shape[0]
        check(self.lib.tkv_fetch_pages_layer(self.ctx, _ptr(miss, torch.int32, "miss"),
                                             _ptr(miss_count, torch.int32, "miss_count"), width, layer,
                                             _stream(stream)))

    def fetch_pages_rest(self, width, layer, stream=None):
        check(self.lib.tkv_fetch_pages_rest(self.ctx, width, layer, _stream(stream)))

    def sparse_paged_attn(self, layer, q, row_start, ctx_len, sel_local, block_table, out,
                          row_pos=None, stream=None, host_tail=False):
        fn = self.lib.tkv_sparse_paged_attn_host_tail if host_tail else self.lib.tkv_sparse_paged_attn
        check(fn(
            self.ctx, layer, _ptr(q, torch.bfloat16, "q"), q.shape[0],
            _ptr(row_start, torch.int32, "row_start"), _ptr(row_pos, torch.int32, "row_pos"),
            _ptr(ctx_len, torch.int32, "ctx_len"), ctx_len.shape[0],
            _ptr(sel_local, torch.int32, "sel_local"), _ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1], sel_local.shape[1], _ptr(out, torch.bfloat16, "out"), _stream(stream)))

    def decode_layer(self, layer, q, block_table, n_pages, ctx_len, topk, sel_local, needed, out_slots,
                     miss, miss_count, out, page_bias=None, stream=None):
        check(self.lib.tkv_decode_layer(
            self.ctx, layer, _ptr(q, torch.bfloat16, "q"), q.shape[0],
            _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
            _ptr(n_pages, torch.int32, "n_pages"), _ptr(ctx_len, torch.int32, "ctx_len"),
            _ptr(page_bias, torch.float32, "page_bias"), topk, _ptr(sel_local, torch.int32, "sel_local"),
            _ptr(needed, torch.int32, "needed"), _ptr(out_slots, torch.int32, "out_slots"),
            _ptr(miss, torch.int32, "miss"), _ptr(miss_count, torch.int32, "miss_count"),
            _ptr(out, torch.bfloat16, "out"), _stream(stream)))

    def decode_layer_split(self, layer, q, block_table, n_pages, ctx_len, topk, sel_local, needed, out_slots,
                           miss, miss_count, out, copy_stream, page_bias=None, stream=None):
        """decode_layer with the missed rows' other layers copied on copy_stream;
        the caller waits for copy_stream before reading the pool itself."""
        check(self.lib.tkv_decode_layer_split(
            self.ctx, layer, _ptr(q, torch.bfloat16, "q"), q.shape[0],
            _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
            _ptr(n_pages, torch.int32, "n_pages"), _ptr(ctx_len, torch.int32, "ctx_len"),
            _ptr(page_bias, torch.float32, "page_bias"), topk, _ptr(sel_local, torch.int32, "sel_local"),
            _ptr(needed, torch.int32, "needed"), _ptr(out_slots, torch.int32, "out_slots"),
            _ptr(miss, torch.int32, "miss"), _ptr(miss_count, torch.int32, "miss_count"),
            _ptr(out, torch.bfloat16, "out"), _stream(stream), _stream(copy_stream)))

    def decode_layer_prefetch(self, layer, q, block_table, n_pages, ctx_len, topk, sel_local, needed, out_slots,
                              miss, miss_count, out, pred, page_bias=None, stream=None, copy_stream=None):
        check(self.lib.tkv_decode_layer_prefetch(
            self.ctx, layer, _ptr(q, torch.bfloat16, "q"), q.shape[0],
            _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
            _ptr(n_pages, torch.int32, "n_pages"), _ptr(ctx_len, torch.int32, "ctx_len"),
            _ptr(page_bias, torch.float32, "page_bias"), topk, _ptr(sel_local, torch.int32, "sel_local"),
            _ptr(needed, torch.int32, "needed"), _ptr(out_slots, torch.int32, "out_slots"),
            _ptr(miss, torch.int32, "miss"), _ptr(miss_count, torch.int32, "miss_count"),
            _ptr(out, torch.bfloat16, "out"), _ptr(pred, torch.int32, "pred"), pred.numel(), _stream(stream),
            _stream(copy_stream) if copy_stream is not None else None))

    def ensure_write_pages(self, run_req, run_start, run_len, max_run_len, block_table, old_len,
                           stream=None):
        check(self.lib.tkv_ensure_write_pages(
            self.ctx, run_req.numel(), _ptr(run_req, torch.int32, "run_req"),
            _ptr(run_start, torch.int32, "run_start"), _ptr(run_len, torch.int32, "run_len"),
            max_run_len, _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
            _ptr(old_len, torch.int32, "old_len"), _stream(stream)))

    def store_kv_mirror(self, layer, k, v, run_req, run_start, run_len, run_tok_off, max_run_len,
                        block_table, stream=None, copy_stream=None):
        """With `copy_stream`: tkv_store_kv_mirror_split (the mirror writes of
        whole pages on that stream, enqueued beside the next attention call)."""
        args = (self.ctx, layer, _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"), run_req.numel(),
                _ptr(run_req, torch.int32, "run_req"), _ptr(run_start, torch.int32, "run_start"),
                _ptr(run_len, torch.int32, "run_len"), _ptr(run_tok_off, torch.int32, "run_tok_off"),
                max_run_len, _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], _stream(stream))
        if copy_stream is None:
            check(self.lib.tkv_store_kv_mirror(*args))
        else:
            check(self.lib.tkv_store_kv_mirror_split(*args, _stream(copy_stream)))

    # ------------------------------------------------------------ readout ---
    def read_counters(self, stream=None) -> dict:
        c = Counters()
        check(self.lib.tkv_read_counters(self.ctx, C.byref(c), _stream(stream)))
        return c.as_dict()

    def read_state(self, stream=None):
        N, S = self.cfg.num_logical_pages, self.cfg.num_slots
        p2s = np.empty(N, dtype=np.int32)
        s2p = np.empty(S, dtype=np.int32)
        stamp = np.empty(S, dtype=np.int64)
        clock = C.c_int64()
        check(self.lib.tkv_debug_read_state(self.ctx, p2s.ctypes.data, s2p.ctypes.data, stamp.ctypes.data,
                                            C.byref(clock), _stream(stream)))
        return dict(page_to_slot=p2s, slot_to_page=s2p, stamp=stamp, clock=clock.value)

    def mirror_flush(self, stream=None):
        """Enqueue a split store's deferred mirror copy and order `stream` after it."""
        check(self.lib.tkv_mirror_flush(self.ctx, _stream(stream)))

    def mirror(self) -> np.ndarray:
        """Read-only view [num_logical_pages][row_bytes] of the pinned mirror."""
        ptr = self.lib.tkv_mirror_host_ptr(self.ctx)
        n = int(self.sizes.mirror_bytes)
        arr = np.ctypeslib.as_array((C.c_uint8 * n).from_address(ptr))
        arr = arr.reshape(self.cfg.num_logical_pages, self.row_bytes)
        arr.flags.writeable = False
        return arr

    def pool_rows(self) -> torch.Tensor:
        return self.pool[: self.cfg.num_slots * self.row_bytes].view(self.cfg.num_slots, self.row_bytes)

    def slab_view(self) -> torch.Tensor:
        L, N = self.cfg.num_layers, self.cfg.num_logical_pages
        H, D = self.cfg.num_kv_heads, self.cfg.head_dim
        return self.slab[: L * N * H * D * 2].view(torch.bfloat16).view(L, N, H, D)

    # ------------------------------------------------------------ codecs ----
    def e4m3_encode(self, x: torch.Tensor) -> torch.Tensor:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        check(self.lib.tkv_debug_e4m3_encode(_ptr(x, torch.float32, "x"), out.data_ptr(), x.numel(),
                                             _stream(None)))
        return out

    # ------------------------------------------------------ prefix tier ---
    def prefix_record_bytes(self) -> int:
        return int(self.lib.tkv_prefix_record_bytes(self.ctx))

    def prefix_save(self, pages, stream=None) -> np.ndarray:
        """Records of the given logical pages: uint8 [n][prefix_record_bytes]."""
        pages = np.ascontiguousarray(pages, dtype=np.int32)
        out = np.empty((len(pages), self.prefix_record_bytes()), dtype=np.uint8)
        check(self.lib.tkv_prefix_save(self.ctx, pages.ctypes.data, len(pages), out.ctypes.data, _stream(stream)))
        return out

    def prefix_restore(self, pages, records: np.ndarray, stream=None, noalloc=False) -> None:
        """Rehydration of records into `pages`; with `noalloc` through
        tkv_prefix_restore_noalloc (no memory allocated during the call)."""
        pages = np.ascontiguousarray(pages, dtype=np.int32)
        records = np.ascontiguousarray(records, dtype=np.uint8)
        if records.shape != (len(pages), self.prefix_record_bytes()):
            raise ValueError(f"records shape {records.shape} != ({len(pages)}, {self.prefix_record_bytes()})")
        fn = self.lib.tkv_prefix_restore_noalloc if noalloc else self.lib.tkv_prefix_restore
        check(fn(self.ctx, pages.ctypes.data, len(pages), records.ctypes.data, _stream(stream)))

    ATTN_AUTO, ATTN_VECTOR, ATTN_MATRIX = 0, 1, 2

    def set_attn_kernel(self, kernel: int) -> None:
        """Attention kernel of later calls (tkv_debug_set_attn_kernel)."""
        check(self.lib.tkv_debug_set_attn_kernel(self.ctx, int(kernel)))

    def set_attn_range(self, pages: int) -> None:
        """Pages per range of the multi-pass prefill attention (0 = one pass)."""
        check(self.lib.tkv_debug_set_attn_range(self.ctx, int(pages)))

    def e4m3_decode(self, codes: torch.Tensor) -> torch.Tensor:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
        check(self.lib.tkv_debug_e4m3_decode(_ptr(codes, torch.uint8, "codes"), out.data_ptr(),
                                             codes.numel(), _stream(None)))
        return out
