"""Seeded input generators (NumPy side).

Bulk tensors (keys, values, prefill queries) are addressed by block: one
block is ``block_tokens`` consecutive tokens of one request in one layer,
laid out ``[token][head][dim]``.  Block ``(kind, seed, layer, req, block)``
is drawn from NumPy's Philox4x64-10 bit generator with

    key = (seed << 16 | kind,  layer << 48 | req << 32 | block)

taking ``random_raw`` 64-bit words and splitting each into four 16-bit
uniforms, lowest half first.  A uniform ``u`` maps through a 65,536-entry
table to an integer ``m`` and the value is ``m * 2**-e``:

* keys/values: ``m = clip(rint(16 * Phi^-1((u + .5) / 65536)), -64, 64)``,
  ``e = 4`` -- N(0,1) on the 2^-4 grid clipped to +-4;
* queries: ``m = clip(rint(32 * Phi^-1((u + .5) / 65536)), -128, 128)``,
  ``e = 5`` -- N(0,1) on the 2^-5 grid clipped to +-4.

Every such value is exactly representable in bfloat16.  The grids make the
indexer's fp32 dot products exact in any summation order, which is what lets
the GPU's page selection be compared bit for bit with the oracle's.

A workload with ``values == "bf16"`` draws the same uniforms but maps them to
``bf16(Phi^-1((u + .5) / 65536))`` (round to nearest even): general bf16
N(0,1) values, no grid; its decode queries are the same processes rounded to
bf16 instead of to the query grid.

Decode queries are small and drawn on the host from ``default_rng``: either
i.i.d. N(0,1) per step, or the AR(1) process ``q_t = (0.9 q_{t-1} + 0.1 n_t)
/ sqrt(0.82)`` (variance preserving) kept in fp64 and emitted on the query
grid; ``ar_literal`` drops the ``1/sqrt(0.82)``.
"""
from __future__ import annotations

import math
from functools import lru_cache
from statistics import NormalDist

import numpy as np

from .configs import Workload

KIND_K, KIND_V, KIND_Q = 0, 1, 2
KV_EXP, Q_EXP = 4, 5


@lru_cache(maxsize=None)
def _inv_normal_grid(scale: int, lim: int) -> np.ndarray:
    nd = NormalDist()
    u = [(i + 0.5) / 65536.0 for i in range(65536)]
    vals = np.array([nd.inv_cdf(x) for x in u], dtype=np.float64)
    m = np.clip(np.rint(scale * vals), -lim, lim).astype(np.int16)
    m.setflags(write=False)
    return m


def kv_table() -> np.ndarray:
    """int16[65536]: grid integer for keys/values (value = m / 16)."""
    return _inv_normal_grid(16, 64)


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of finite fp32 values, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@lru_cache(maxsize=None)
def bf16_table() -> np.ndarray:
    """uint16[65536]: bf16 bit patterns of Phi^-1((u + .5) / 65536)."""
    nd = NormalDist()
    vals = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float64)
    t = _bf16_rne_bits(vals.astype(np.float32))
    t.setflags(write=False)
    return t


def q_table() -> np.ndarray:
    """int16[65536]: grid integer for prefill queries (value = m / 32)."""
    return _inv_normal_grid(32, 128)


def philox_key(kind: int, seed: int, layer: int, req: int, block: int) -> np.ndarray:
    k0 = (seed << 16) | kind
    k1 = (layer << 48) | (req << 32) | block
    return np.array([k0, k1], dtype=np.uint64)


def block_uniforms(kind: int, seed: int, layer: int, req: int, block: int, n: int) -> np.ndarray:
    """The n 16-bit uniforms of one block."""
    assert n % 4 == 0
    bg = np.random.Philox(key=philox_key(kind, seed, layer, req, block))
    return bg.random_raw(n // 4).astype("<u8").view("<u2")


def block_ints(kind: int, seed: int, layer: int, req: int, block: int,
               block_tokens: int, heads: int, dim: int) -> np.ndarray:
    """Grid integers of one block, int16 [block_tokens][heads][dim]."""
    u = block_uniforms(kind, seed, layer, req, block, block_tokens * heads * dim)
    tab = q_table() if kind == KIND_Q else kv_table()
    return np.take(tab, u).reshape(block_tokens, heads, dim)


def block_values(kind, seed, layer, req, block, block_tokens, heads, dim, values="grid") -> np.ndarray:
    """float32 values of one block: grid integers times a power of two, or
    (values == "bf16") the bf16 table's values; exact in bf16 either way."""
    if values == "bf16":
        u = block_uniforms(kind, seed, layer, req, block, block_tokens * heads * dim)
        bits = np.take(bf16_table(), u).astype(np.uint32) << 16
        return bits.view(np.float32).reshape(block_tokens, heads, dim)
    e = Q_EXP if kind == KIND_Q else KV_EXP
    m = block_ints(kind, seed, layer, req, block, block_tokens, heads, dim)
    return m.astype(np.float32) * np.float32(2.0 ** -e)


def kv_page(wl: Workload, kind: int, layer: int, req: int, page: int) -> np.ndarray:
    """Keys (kind 0) or values (kind 1) of one page: float32 [page_size][Hkv][d]."""
    return block_values(kind, wl.seed, layer, req, page, wl.page_size,
                        wl.num_kv_heads, wl.head_dim, wl.values)


def kv_tokens(wl: Workload, kind: int, layer: int, req: int, start: int, count: int) -> np.ndarray:
    """Keys or values of tokens [start, start+count) of a request: float32 [count][Hkv][d]."""
    ps = wl.page_size
    p0, p1 = start // ps, (start + count - 1) // ps
    pages = [kv_page(wl, kind, layer, req, p) for p in range(p0, p1 + 1)]
    allv = np.concatenate(pages, axis=0)
    off = start - p0 * ps
    return allv[off:off + count]


def prefill_queries(wl: Workload, layer: int, start: int, count: int) -> np.ndarray:
    """Queries of prefill tokens [start, start+count) (positions relative to the
    chunk start) of request 0: float32 [count][Hq][d].  Blocks of 64 tokens."""
    bt = 64
    b0, b1 = start // bt, (start + count - 1) // bt
    blocks = [block_values(KIND_Q, wl.seed, layer, 0, b, bt, wl.num_q_heads, wl.head_dim, wl.values)
              for b in range(b0, b1 + 1)]
    allv = np.concatenate(blocks, axis=0)
    off = start - b0 * bt
    return allv[off:off + count]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of values that are exactly representable (asserted)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    bits = x32.view(np.uint32)
    assert not np.any(bits & 0xFFFF), "value not exactly representable in bfloat16"
    return (bits >> 16).astype(np.uint16)


def _on_q_grid(x: np.ndarray) -> np.ndarray:
    return (np.clip(np.rint(x * 32.0), -128, 128) / 32.0).astype(np.float32)


def decode_queries(wl: Workload) -> np.ndarray:
    """float32 [steps][L][B][Hq][d] on the query grid (or rounded to bf16)."""
    if wl.values == "bf16":
        def emit(x):
            return (_bf16_rne_bits(np.asarray(x, dtype=np.float32)).astype(np.uint32) << 16).view(np.float32)
    else:
        emit = _on_q_grid
    rng = np.random.default_rng(wl.seed)
    shape = (wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim)
    out = np.empty((wl.steps,) + shape, dtype=np.float32)
    if wl.query == "iid":
        for t in range(wl.steps):
            out[t] = emit(rng.standard_normal(shape))
        return out
    norm = 1.0 / math.sqrt(0.82) if wl.query == "ar" else 1.0
    state = rng.standard_normal(shape)
    out[0] = emit(state)
    for t in range(1, wl.steps):
        state = (0.9 * state + 0.1 * rng.standard_normal(shape)) * norm
        out[t] = emit(state)
    return out


def block_tables(wl: Workload):
    """(block_table int32 [B][max_pages] padded with -1, n_pages int32 [B]).

    Logical ids are the identity, request by request, unless the workload
    permutes them (a seeded permutation of all logical ids split by request
    in order)."""
    n = wl.num_logical_pages
    ids = np.arange(n, dtype=np.int64)
    if wl.permute_pages:
        ids = np.random.default_rng([wl.seed, 11]).permutation(n)
    bt = np.full((wl.batch, wl.max_pages), -1, dtype=np.int32)
    npg = np.zeros(wl.batch, dtype=np.int32)
    off = 0
    for b in range(wl.batch):
        k = wl.pages_of(b)
        bt[b, :k] = ids[off:off + k]
        npg[b] = k
        off += k
    return bt, npg


def page_bias(wl: Workload):
    """float32 [num_logical_pages] log-Zipf prior, or None.

    Page rank r = 1 + a seeded permutation; bias = fp32(-s * ln r)."""
    if wl.bias == "none":
        return None
    n = wl.num_logical_pages
    r = 1 + np.random.default_rng([wl.seed, 7]).permutation(n)
    return (-wl.zipf_s * np.log(r.astype(np.float64))).astype(np.float32)


def context_lengths(wl: Workload) -> np.ndarray:
    """Decode context length per request (int32 [B])."""
    return np.array(wl.contexts, dtype=np.int32)


def append_lengths(wl: Workload, s: int):
    """Appending workloads: per request, the context length once step s's token
    is written and the pages it spans (int32 [B] each)."""
    ctx = context_lengths(wl) + np.int32(s + 1)
    return ctx, ((ctx + wl.page_size - 1) // wl.page_size).astype(np.int32)
