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

The score is the exact dot product rounded once to fp32.  The oracle sums
it in fp64 and proves the sum exact with a certificate: every product of two
bfloat16 values is a multiple of 2^e, e = (lowest set bit of the query
element) + (lowest set bit of the slab element), so with e_min the smallest
such exponent of a page and A = sum |qg * slab|, every partial sum -- in ANY
order -- is a multiple of 2^e_min no larger than A, hence exact in a float
with b significand bits whenever A < 2^(b + e_min).  ``score_bits`` is
log2(A) - e_min per (row, page): below 53 the fp64 sum (and any fp64
accumulation) is exact; below 24 any fp32 accumulation is too, whatever its
order (a matrix-core product included).  On the workloads' input grids (keys
on 2^-4, queries on 2^-5, so products on 2^-15) A < 2^9 gives < 24 bits.
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


class ScoreCertificateError(ArithmeticError):
    """The inputs do not let the score sums be proven exact at the required
    accumulator width."""


NO_BITS = 10 ** 6   # lowest-set-bit exponent of an all-zero vector (never the minimum)


def lowest_bit_exponent(x: np.ndarray, axis=-1) -> np.ndarray:
    """Per vector along ``axis``: the smallest e such that some element has
    its lowest set bit at 2^e (every element is then a multiple of 2^e).
    Elements are fp32 values (bf16 values included); zeros are ignored; an
    all-zero vector gives NO_BITS."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    expf = (u >> 23) & 0xFF
    man = (u & 0x7FFFFF) | np.where(expf > 0, np.uint32(0x800000), np.uint32(0))   # implicit bit
    low = man & (np.uint32(0) - man)                        # the lowest set bit, a power of two (or 0)
    tz = np.frexp(low.astype(np.float64))[1] - 1            # its position
    base = np.where(expf > 0, expf.astype(np.int64) - 150, -149)   # exponent of the mantissa's last bit
    e = np.where(man != 0, base + tz, NO_BITS)
    return e.min(axis=axis)


def score_bits(qg: np.ndarray, slab_pages: np.ndarray) -> np.ndarray:
    """Significand bits an accumulator needs for the scores of qg [Hkv][d]
    against slab_pages [P][Hkv][d] to be exact in any order: log2(A) - e_min
    per page (0 for a page whose products are all zero)."""
    P = slab_pages.shape[0]
    qf = qg.reshape(-1)
    sf = slab_pages.reshape(P, -1)
    A = np.abs(sf).astype(np.float64) @ np.abs(qf).astype(np.float64)
    e_min = lowest_bit_exponent(qf) + lowest_bit_exponent(sf, axis=1)
    with np.errstate(divide="ignore"):
        bits = np.where(A > 0, np.log2(A * (1 + 2.0 ** -30)) - e_min, 0.0)
    return bits


def score_certificate(qg: np.ndarray, slab_pages: np.ndarray) -> float:
    """max over pages of sum |qg * slab| (on the workloads' grids: < 2^9)."""
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
               page_size: int = 64, with_keys: bool = False):
    """One query row: returns (sel_local int32 [k], certificate) where the
    certificate is (max sum |qg*slab|, max score bits) over the visible pages;
    with ``with_keys`` also the fp32 keys of the visible pages.

    slab_layer float32 [N][Hkv][d] indexed by logical page id; block_row maps
    local -> logical page id."""
    visible = n_pages if row_pos is None else min(n_pages, row_pos // page_size + 1)
    qg = group_query(q_row, num_kv_heads)
    logical = block_row[:visible].astype(np.int64)
    slab_pages = slab_layer[logical]
    scores = page_scores(qg, slab_pages)
    bias_pages = None if bias is None else bias[logical]
    keys = keys_from_scores(scores, bias_pages)
    bits = score_bits(qg, slab_pages)
    cert = (score_certificate(qg, slab_pages), float(bits.max()) if bits.size else 0.0)
    sel = topk_pages(keys, visible, k)
    return (sel, cert, keys) if with_keys else (sel, cert)


def select_rows(q_rows: np.ndarray, slab_layer: np.ndarray, block_row: np.ndarray, n_pages: int,
                k: int, num_kv_heads: int, bias=None, row_pos=None, page_size: int = 64):
    """Many rows of one request: the same definition as ``select_row``, with
    the scores of all rows against all pages as one fp64 matrix product.
    Returns (sel_local int32 [rows][k], certificate) with the certificate as
    in ``select_row``, over every row's visible pages."""
    rows = q_rows.shape[0]
    qg = np.stack([group_query(q_rows[r], num_kv_heads) for r in range(rows)])   # [rows][Hkv][d]
    logical = block_row[:n_pages].astype(np.int64)
    slab32 = slab_layer[logical].reshape(n_pages, -1)
    slab_pages = slab32.astype(np.float64)
    qmat = qg.astype(np.float64).reshape(rows, -1)
    scores = qmat @ slab_pages.T                                   # exact while the certificate holds
    A = np.abs(qmat) @ np.abs(slab_pages).T
    e_min = (lowest_bit_exponent(qg.reshape(rows, -1), axis=1)[:, None]
             + lowest_bit_exponent(slab32, axis=1)[None, :])
    with np.errstate(divide="ignore"):
        bits = np.where(A > 0, np.log2(A * (1 + 2.0 ** -30)) - e_min, 0.0)
    if row_pos is not None:   # only the pages a row sees count
        vis = np.minimum(n_pages, np.asarray(row_pos, dtype=np.int64) // page_size + 1)
        seen = np.arange(n_pages)[None, :] < vis[:, None]
        A = np.where(seen, A, 0.0)
        bits = np.where(seen, bits, 0.0)
    cert = (float(A.max()) if A.size else 0.0, float(bits.max()) if bits.size else 0.0)
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
