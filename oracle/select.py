"""Indexer top-k page selection and compact_selected_pages.

FreeToken PR #499, "Why this works for sparse attention": every attend step
first runs the indexer -- a top-k block selection over a compressed slab that
stays on the GPU -- and only then reads the selected pages.  "Design" adds
compact_selected_pages with a cap of max_sel_pages = 2*block_topk + 8 and a
counter of what the cap drops.

Readings where the page is silent (each listed in the design notes):

* one selection per request row per layer, over all query heads: the
  per-KV-group query is ``qg[g] = bf16(sum of the group's query heads)`` and
  the page score is ``S = sum_g qg[g] . slab[page][g]`` (no 1/sqrt(d): it
  does not change the ranking);
* key = fp32(fp32(S) + bias[page]) (bias is 0 unless a workload supplies it);
* top-k by key descending, equal keys -> lower local page index first;
  emitted in ascending local page order, padded with -1 when fewer than k
  pages are visible;
* prefill rows see page i iff page_size * i <= their position;
* the cap keeps the lowest local page ids and counts the rest as drops.

Scores are summed in fp64, where every product of two bfloat16 values and
every partial sum of a few hundred of them is exact for the input grids the
workloads use; ``score_certificate`` reports the quantity that makes the fp32
sum exact in ANY order (all products on the 2^-15 grid and sum |products| <
2^9), which the GPU needs for bit-exact selections.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round


def group_query(q: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """q float32 [Hq][d] -> qg float32 [Hkv][d] (bf16 values): exact group sum,
    then fp32, then bf16."""
    Hq, d = q.shape
    G = Hq // num_kv_heads
    s = q.astype(np.float64).reshape(num_kv_heads, G, d).sum(axis=1)
    return bf16_round(s.astype(np.float32))


def page_scores(qg: np.ndarray, slab_pages: np.ndarray) -> np.ndarray:
    """qg [Hkv][d], slab_pages [P][Hkv][d] -> exact fp64 scores [P]."""
    return np.einsum("gd,pgd->p", qg.astype(np.float64), slab_pages.astype(np.float64))


def score_certificate(qg: np.ndarray, slab_pages: np.ndarray) -> float:
    """max over pages of sum |qg * slab| (exactness needs < 2^9 on the grids)."""
    a = np.einsum("gd,pgd->p", np.abs(qg.astype(np.float64)), np.abs(slab_pages.astype(np.float64)))
    return float(a.max()) if a.size else 0.0


def keys_from_scores(scores: np.ndarray, bias_pages) -> np.ndarray:
    k = scores.astype(np.float32)
    if bias_pages is not None:
        k = (k + np.asarray(bias_pages, dtype=np.float32)).astype(np.float32)
    return k


def topk_pages(keys: np.ndarray, visible: int, k: int) -> np.ndarray:
    """Top-k local page ids among pages [0, visible) by key desc, ties to the
    lower id; returned ascending, padded with -1 to length k."""
    idx = np.arange(visible)
    order = np.lexsort((idx, -keys[:visible].astype(np.float64)))
    chosen = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def select_row(q_row: np.ndarray, slab_layer: np.ndarray, block_row: np.ndarray,
               n_pages: int, k: int, num_kv_heads: int, bias=None, row_pos=None,
               page_size: int = 64):
    """One query row: returns (sel_local int32 [k], certificate).

    slab_layer float32 [N][Hkv][d] indexed by logical page id; block_row maps
    local -> logical page id."""
    visible = n_pages if row_pos is None else min(n_pages, row_pos // page_size + 1)
    qg = group_query(q_row, num_kv_heads)
    logical = block_row[:visible].astype(np.int64)
    slab_pages = slab_layer[logical]
    scores = page_scores(qg, slab_pages)
    bias_pages = None if bias is None else bias[logical]
    keys = keys_from_scores(scores, bias_pages)
    return topk_pages(keys, visible, k), score_certificate(qg, slab_pages)


def select_rows(q_rows: np.ndarray, slab_layer: np.ndarray, block_row: np.ndarray, n_pages: int,
                k: int, num_kv_heads: int, bias=None, row_pos=None, page_size: int = 64):
    """Many rows of one request: the same definition as ``select_row``, with
    the scores of all rows against all pages as one fp64 matrix product.
    Returns (sel_local int32 [rows][k], certificate)."""
    rows = q_rows.shape[0]
    qg = np.stack([group_query(q_rows[r], num_kv_heads) for r in range(rows)])   # [rows][Hkv][d]
    logical = block_row[:n_pages].astype(np.int64)
    slab_pages = slab_layer[logical].astype(np.float64).reshape(n_pages, -1)
    qmat = qg.astype(np.float64).reshape(rows, -1)
    scores = qmat @ slab_pages.T                                                   # exact on the grids
    cert = float((np.abs(qmat) @ np.abs(slab_pages).T).max()) if n_pages else 0.0
    bias_pages = None if bias is None else bias[logical]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        visible = n_pages if row_pos is None else min(n_pages, int(row_pos[r]) // page_size + 1)
        keys = keys_from_scores(scores[r, :visible], None if bias_pages is None else bias_pages[:visible])
        out[r] = topk_pages(keys, visible, k)
    return out, cert


def compact_request(sel_rows: np.ndarray, block_row: np.ndarray, cap: int):
    """Union of one request's selections -> (needed logical ids int32 [cap],
    drops).  Ascending local ids, unique, first `cap` kept, -1 padded."""
    vals = sel_rows.reshape(-1)
    u = np.unique(vals[vals >= 0])
    kept = u[:cap]
    needed = np.full(cap, -1, dtype=np.int32)
    needed[:len(kept)] = block_row[kept]
    return needed, max(0, len(u) - cap)
