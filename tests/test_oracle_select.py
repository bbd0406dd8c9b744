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


# ------------------------------------------------------- group sum rounding --
def _group_rounds_once(fn):
    """Hand case: heads 1, 2^-8, 2^-8 (others 0).  Exact sum 1 + 2^-7 is a
    bf16 value, so one rounding keeps it; rounding after each head gives
    1 + 2^-8 -> 1 (a tie, to even) and then 1 again."""
    q = np.zeros((8, 4), dtype=np.float32)
    q[0, :] = 1.0
    q[1, :] = 2.0 ** -8
    q[2, :] = 2.0 ** -8
    qg = fn(q, 1)
    return bool(np.all(qg == np.float32(1.0 + 2.0 ** -7)))


def _group_query_per_head_rounding(q, num_kv_heads):
    """A plausible wrong group sum: bf16 rounding after every head."""
    from oracle.codecs import bf16_round
    Hq, d = q.shape
    G = Hq // num_kv_heads
    acc = np.zeros((num_kv_heads, d), dtype=np.float32)
    for h in range(G):
        acc = bf16_round((acc + q.reshape(num_kv_heads, G, d)[:, h]).astype(np.float32))
    return acc


def test_group_query_rounds_the_exact_sum_once():
    assert _group_rounds_once(group_query)
    assert not _group_rounds_once(_group_query_per_head_rounding)


def test_group_rounding_decides_a_selection():
    """The same hand case through select_row (one KV group of 8 heads):
    qg[0] = 1 + 2^-7 (exact sum) and qg[1] = 1.  Page 1's slab row is
    (+1, -1, 0, ...), so it scores qg[0] - qg[1] = 2^-7; page 0's is
    (0, 2^-8, 0, ...), scoring 2^-8.  Top-1 is page 1.  With per-head
    rounding qg[0] would be 1, page 1 would score 0 and page 0 would win."""
    q = np.zeros((8, 128), dtype=np.float32)
    q[0, 0] = 1.0
    q[1, 0] = 2.0 ** -8
    q[2, 0] = 2.0 ** -8
    q[3, 1] = 1.0
    slab = np.zeros((2, 1, 128), dtype=np.float32)
    slab[0, 0, 1] = 2.0 ** -8
    slab[1, 0, 0] = 1.0
    slab[1, 0, 1] = -1.0
    bt = np.arange(2, dtype=np.int32)
    sel, _ = select_row(q, slab, bt, 2, 1, 1)
    assert list(sel) == [1]
    bad = page_scores(_group_query_per_head_rounding(q, 1), slab)
    assert bad[0] == 2.0 ** -8 and bad[1] == 0.0


# ----------------------------------------------------------- certificate --
def test_certificate_bits_on_the_grids_match_the_sum_bound():
    """On the workload grids (products on 2^-15) the bits needed are
    log2(sum |qg*slab|) + 15 or fewer (the data may sit on a coarser grid)."""
    from oracle.select import score_bits, score_certificate
    slab = _slab(40, seed=5)
    qg = group_query(_q(seed=6), 4)
    bits = score_bits(qg, slab)
    A = score_certificate(qg, slab)
    assert bits.max() <= np.log2(A) + 15 + 1e-6
    assert bits.max() < 24


def test_certificate_is_exactness_for_a_brute_force_sum():
    """Where the certificate says < 24 bits, fp32 sums in random orders all
    equal fp32 of the exact (integer) sum; an input needing more bits has an
    order whose fp32 sum differs."""
    from oracle.select import score_bits
    rng = np.random.default_rng(12)
    qg = np.zeros((1, 128), dtype=np.float32)
    qg[0] = _q(Hq=1, seed=13)[0]
    slab = _slab(1, H=1, seed=14)
    assert score_bits(qg, slab)[0] < 24
    prods = (qg[0] * slab[0, 0]).astype(np.float32)
    ref = np.float32(sum(int(v * 2 ** 15) for v in prods.astype(np.float64)) / 2.0 ** 15)
    for _ in range(50):
        acc = np.float32(0)
        for v in prods[rng.permutation(128)]:
            acc = np.float32(acc + v)
        assert acc == ref
    # 2^20 and 2^-10 side by side need 31 bits: some order loses the small terms
    wide = np.zeros((1, 1, 4), dtype=np.float32)
    wide[0, 0] = [2.0 ** 20, 2.0 ** -10, 2.0 ** -10, -(2.0 ** 20)]
    one = np.ones((1, 4), dtype=np.float32)
    assert score_bits(one, wide)[0] >= 24
    a = np.float32(0)
    for v in wide[0, 0]:
        a = np.float32(a + v)
    assert a != np.float32(2.0 ** -9)


def test_select_asserts_the_certificate_for_chunk_rows():
    """Off-grid queries and slab (general bf16 values) need more than fp32's
    24 bits for exact chunk scores: select with causal rows raises; decode
    rows (fp64, 53 bits) pass on the same data."""
    from oracle.codecs import bf16_round
    from oracle.select import ScoreCertificateError
    rng = np.random.default_rng(21)
    t = OracleTier(num_layers=1, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64, fp8=True,
                   num_logical_pages=16, num_slots=16)
    t.set_select_width(1, 4)
    t.slab[0] = bf16_round((rng.standard_normal((16, 4, 128)) / 8).astype(np.float32))
    q = bf16_round(rng.standard_normal((1, 32, 128)).astype(np.float32))
    bt = np.arange(16, dtype=np.int32)[None, :]
    rs = np.array([0, 1])
    t.select(0, q, rs, None, bt, np.array([16]), 4)          # decode: fine
    assert 24 <= t.max_score_bits < 53
    with pytest.raises(ScoreCertificateError):
        t.select(0, q, rs, np.array([64 * 16 - 1]), bt, np.array([16]), 4)
    t.check_scores = False
    t.select(0, q, rs, np.array([64 * 16 - 1]), bt, np.array([16]), 4)


def test_select_certificate_holds_on_the_workload_grids():
    from workload import get_workload
    from oracle.run import make_tier, setup
    wl = get_workload("c2s")
    t = make_tier(wl, materialize=False)
    setup(wl, t)
    from workload import gen
    bt, npg = gen.block_tables(wl)
    q = gen.decode_queries(wl)[0, 0]
    t.set_select_width(wl.batch, wl.topk)
    t.select(0, q, np.arange(wl.batch + 1), None, bt, npg, wl.topk)
    assert t.max_score_bits < 24 and t.max_certificate < 2 ** 9


def test_lowest_bit_exponent_brute_force():
    """Per element, the exponent of the lowest set bit of an fp32 value,
    from its exact integer ratio (normals, subnormals, signs; zeros ignored)."""
    from oracle.select import NO_BITS, lowest_bit_exponent
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 2.0 ** -149, 3 * 2.0 ** -140, -1.5, 6.0])])

    def lsb(v):
        num, den = float(v).as_integer_ratio()
        num = abs(num)
        return (num & -num).bit_length() - 1 - (den.bit_length() - 1)

    for v in x:
        exp = lsb(v) if v != 0 else NO_BITS
        assert lowest_bit_exponent(np.array([v], dtype=np.float32)) == exp, v
    m = x.reshape(-1)[: (x.size // 7) * 7].reshape(-1, 7)
    got = lowest_bit_exponent(m, axis=1)
    for r in range(m.shape[0]):
        nz = [lsb(v) for v in m[r] if v != 0]
        assert got[r] == (min(nz) if nz else NO_BITS)
