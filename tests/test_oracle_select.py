"""Pins for the oracle's indexer top-k and compact_selected_pages."""
import json
import os

import numpy as np
import pytest

from oracle.engine import CapacityError, OracleTier
from oracle.select import (compact_request, group_query, page_scores, select_row,
                           topk_pages)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _slab(P, H=4, d=128, seed=0):
    rng = np.random.default_rng(seed)
    return (np.rint(rng.standard_normal((P, H, d)) * 128) / 1024).astype(np.float32)


def _q(Hq=32, d=128, seed=1):
    rng = np.random.default_rng(seed)
    return (np.clip(np.rint(rng.standard_normal((Hq, d)) * 32), -128, 128) / 32).astype(np.float32)


def test_group_query_one_head_is_that_head():
    q = np.zeros((32, 128), dtype=np.float32)
    q[9] = _q()[0]
    qg = group_query(q, 4)
    assert np.array_equal(qg[1], q[9]) and not np.any(qg[[0, 2, 3]])


def test_scores_one_hot_query_reads_one_coordinate():
    slab = _slab(50)
    qg = np.zeros((4, 128), dtype=np.float32)
    qg[2, 77] = 1.0
    assert np.array_equal(page_scores(qg, slab), slab[:, 2, 77].astype(np.float64))


def test_scores_match_float128_like_exact_sum():
    """On the grids, the fp64 score equals the exact rational dot product
    (checked with Python integers)."""
    slab = _slab(20, seed=3)
    qg = group_query(_q(seed=4), 4)
    got = page_scores(qg, slab)
    qi = (qg.astype(np.float64) * 32).astype(np.int64)          # q grid 2^-5
    si = (slab.astype(np.float64) * 1024).astype(np.int64)      # slab grid 2^-10
    for p in range(20):
        exact = sum(int(a) * int(b) for a, b in zip(qi.ravel(), si[p].ravel()))
        assert got[p] == exact / 2.0 ** 15


def test_topk_matches_full_argsort():
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(1, 90))
        k = int(rng.integers(1, 40))
        keys = rng.integers(-5, 5, n).astype(np.float32)   # many exact ties
        got = topk_pages(keys, n, k)
        order = sorted(range(n), key=lambda i: (-float(keys[i]), i))[:k]
        exp = sorted(order) + [-1] * (k - min(k, n))
        assert got.tolist() == exp


def test_budget_at_least_context_selects_everything():
    slab = _slab(30)
    bt = np.arange(30, dtype=np.int32)
    sel, _ = select_row(_q(), slab, bt, 30, 40, 4)
    assert sel.tolist() == list(range(30)) + [-1] * 10


def test_causal_visibility_in_prefill_rows():
    slab = _slab(30)
    bt = np.arange(30, dtype=np.int32)
    # a query at position 64*5 + 3 sees pages 0..5 only
    sel, _ = select_row(_q(), slab, bt, 30, 10, 4, row_pos=64 * 5 + 3, page_size=64)
    assert sel.tolist() == list(range(6)) + [-1] * 4


def test_bias_shifts_selection():
    slab = np.zeros((10, 4, 128), dtype=np.float32)
    bias = np.arange(10, dtype=np.float32)
    sel, _ = select_row(_q(), slab, np.arange(10, dtype=np.int32), 10, 3, 4, bias=bias)
    assert sel.tolist() == [7, 8, 9]


def test_compact_forced_drops_are_counted():
    sel = np.array([[1, 4, 6, 9, 12, 20, 33, 41]], dtype=np.int32)
    bt = np.arange(100, 150, dtype=np.int32)
    needed, drops = compact_request(sel, bt, 5)
    assert needed.tolist() == [101, 104, 106, 109, 112] and drops == 3


def test_compact_union_of_rows_sorted_unique():
    sel = np.array([[3, 5, 7, -1], [1, 5, 9, 11]], dtype=np.int32)
    bt = np.arange(20, dtype=np.int32)[::-1].copy()
    needed, drops = compact_request(sel, bt, 8)
    assert needed.tolist() == [18, 16, 14, 12, 10, 8, -1, -1] and drops == 0


def test_pages_printed_figures():
    """Figures the pages print, recomputed from the definitions."""
    g = json.load(open(GOLDEN))
    tier = OracleTier(num_layers=12, num_q_heads=32, num_kv_heads=4, head_dim=128,
                      page_size=64, fp8=True, num_logical_pages=10, num_slots=100000,
                      materialize=False)
    # cap formula: 2*block_topk + 8 at the largest per-request width the page quotes
    assert tier.set_select_width(1, g["block_topk_for_520"]) == g["max_sel_pages_upper"]
    # logical capacity = (GPU pages + host pages) * page_size
    assert (g["gpu_pages"] + g["host_pages"]) * g["page_size"] == g["logical_capacity_tokens"]
    # fp8 pages roughly halve the fetch bytes of bf16 ones
    fp8 = OracleTier(num_layers=1, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                     fp8=True, num_logical_pages=1, num_slots=1).lay.row_bytes
    bf16 = OracleTier(num_layers=1, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                      fp8=False, num_logical_pages=1, num_slots=1).lay.row_bytes
    assert abs(fp8 / bf16 - 0.5) < 0.01


def test_select_width_must_fit_pool():
    tier = OracleTier(num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16,
                      fp8=False, num_logical_pages=256, num_slots=64)
    assert tier.set_select_width(1, 16) == 40
    with pytest.raises(CapacityError):
        tier.set_select_width(2, 16)


def test_batched_rows_equal_single_rows():
    """select_rows (one matrix product for all rows) == select_row row by row,
    including causal rows and the page bias."""
    from oracle.select import select_rows
    rng = np.random.default_rng(12)
    slab = _slab(90, seed=5)
    bt = rng.permutation(90).astype(np.int32)
    q = np.stack([_q(seed=s) for s in range(20)])
    bias = (-np.log(1 + rng.permutation(90))).astype(np.float32)
    pos = rng.integers(0, 90 * 64, 20)
    got, _ = select_rows(q, slab, bt, 90, 7, 4, bias=bias, row_pos=pos)
    for r in range(20):
        exp, _ = select_row(q[r], slab, bt, 90, 7, 4, bias=bias, row_pos=int(pos[r]))
        assert np.array_equal(got[r], exp)
