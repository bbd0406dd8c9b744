"""Pins for the oracle's LRU residency (ensure).

* an independent simulator (per-slot last-use times, victims by repeated
  linear-scan argmin instead of a sort) on every trace of up to three calls
  over four pages, and on long random traces;
* with one page per call the hit/miss sequence equals the textbook LRU of
  capacity S (collections.OrderedDict), and misses never grow with S (LRU's
  inclusion property);
* state invariants after every call.
"""
import itertools
from collections import OrderedDict

import numpy as np
import pytest

from oracle.lru import ERR_CAPACITY, ERR_PAGE_RANGE, LRUState


class ScanLRU:
    """Same policy, different construction."""

    def __init__(self, N, S):
        self.res = {}                    # page -> slot
        self.slot_page = [None] * S
        self.last = [0] * S
        self.t = 0
        self.S = S

    def ensure(self, needed, no_fetch=None):
        distinct = []
        for j, p in enumerate(needed):
            if p >= 0 and p not in [d[0] for d in distinct]:
                distinct.append((p, j))
        if len(distinct) > self.S:
            return None
        self.t += 1
        used = [False] * self.S
        miss = []
        for p, j in distinct:
            if p in self.res:
                s = self.res[p]
                used[s] = True
                self.last[s] = self.t
            else:
                miss.append((p, j))
        fetched = []
        for p, j in miss:
            best = None
            for s in range(self.S):
                if used[s]:
                    continue
                if best is None or self.last[s] < self.last[best]:
                    best = s
            used[best] = True
            if self.slot_page[best] is not None:
                del self.res[self.slot_page[best]]
            self.slot_page[best] = p
            self.res[p] = best
            self.last[best] = self.t
            if not (no_fetch is not None and no_fetch[j]):
                fetched.append((best, p))
        out = [self.res.get(p, -1) if p >= 0 else -1 for p in needed]
        return out, fetched


def _check_invariants(lru: LRUState, needed, out):
    p2s, s2p = lru.page_to_slot, lru.slot_to_page
    for p in range(lru.N):
        if p2s[p] >= 0:
            assert s2p[p2s[p]] == p
    for s in range(lru.S):
        if s2p[s] >= 0:
            assert p2s[s2p[s]] == s
        else:
            assert lru.stamp[s] == 0
    for j, p in enumerate(needed):
        if p >= 0:
            assert out[j] == p2s[p] >= 0 and lru.stamp[out[j]] == lru.clock


def _run_both(N, S, trace, nofetch_trace=None):
    a, b = LRUState(N, S), ScanLRU(N, S)
    for i, call in enumerate(trace):
        nf = None if nofetch_trace is None else nofetch_trace[i]
        res_b = b.ensure(list(call), nf)
        before = (a.clock, a.page_to_slot.copy())
        out, miss = a.ensure(np.array(call), nf)
        if res_b is None:
            assert a.error_word & ERR_CAPACITY
            assert a.clock == before[0] and np.array_equal(a.page_to_slot, before[1])
            assert np.all(out == -1) and len(miss) == 0
            a.error_word = 0
            continue
        assert out.tolist() == res_b[0]
        assert [tuple(m) for m in miss.tolist()] == res_b[1]
        _check_invariants(a, call, out)
        c = a.counters
        assert c["hits"] + c["misses"] + c["fresh_allocs"] >= 0


def test_exhaustive_tiny_traces():
    pages = range(4)
    calls = [c for n in (1, 2, 3) for c in itertools.product(pages, repeat=n)]
    count = 0
    for S in (1, 2, 3):
        for L in (1, 2):
            for trace in itertools.product(calls, repeat=L):
                _run_both(4, S, trace)
                count += 1
    # three-call traces over 1-2 pages per call
    short = [c for n in (1, 2) for c in itertools.product(pages, repeat=n)]
    for S in (1, 2, 3):
        for trace in itertools.product(short, repeat=3):
            _run_both(4, S, trace)
            count += 1
    assert count > 20000


def test_random_long_traces_with_no_fetch_and_padding():
    rng = np.random.default_rng(3)
    for _ in range(300):
        N = int(rng.integers(2, 12))
        S = int(rng.integers(1, 8))
        trace, nft = [], []
        for _ in range(int(rng.integers(1, 25))):
            w = int(rng.integers(1, 6))
            call = rng.integers(-1, N, w).tolist()
            trace.append(call)
            nft.append(rng.integers(0, 2, w).astype(bool).tolist())
        _run_both(N, S, trace, nft)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
def test_single_page_calls_equal_textbook_lru(S):
    rng = np.random.default_rng(S)
    trace = rng.integers(0, 12, 400).tolist()
    lru = LRUState(12, S)
    od = OrderedDict()
    for p in trace:
        h0 = lru.counters["hits"]
        lru.ensure(np.array([p]))
        hit = lru.counters["hits"] > h0
        tb_hit = p in od
        if tb_hit:
            od.move_to_end(p)
        else:
            if len(od) == S:
                od.popitem(last=False)
            od[p] = True
        assert hit == tb_hit


def test_inclusion_property_misses_monotone_in_pool_size():
    rng = np.random.default_rng(11)
    trace = (rng.zipf(1.3, 2000) % 40).tolist()
    prev = None
    for S in range(1, 41):
        lru = LRUState(40, S)
        for p in trace:
            lru.ensure(np.array([p]))
        m = lru.counters["misses"]
        assert prev is None or m <= prev
        prev = m


def test_out_of_range_ids_flagged_and_ignored():
    lru = LRUState(5, 3)
    out, miss = lru.ensure(np.array([1, 7, -3, -1, 2]))
    assert lru.error_word & ERR_PAGE_RANGE
    assert out[1] == -1 and out[2] == -1 and out[3] == -1 and out[0] >= 0 and out[4] >= 0


def test_free_slots_first_lowest_index_then_least_recent():
    lru = LRUState(10, 3)
    _, m = lru.ensure(np.array([5, 6]))
    assert m.tolist() == [[0, 5], [1, 6]]
    _, m = lru.ensure(np.array([7]))
    assert m.tolist() == [[2, 7]]
    lru.ensure(np.array([5]))                 # 5 (slot 0) refreshed
    _, m = lru.ensure(np.array([8, 9]))       # victims: slot 1 (page 6, stamp 1), slot 2 (page 7, stamp 2)
    assert m.tolist() == [[1, 8], [2, 9]] and lru.counters["evictions"] == 2


# ------------------------------------------------------------------ unbind --
def _unbind_trace(state_cls):
    """Hand trace, 2 slots, pages 0..3 (one clock tick per call):
      ensure [0] -> clock 1: page 0 takes slot 0 (free slots, lowest first)
      ensure [1] -> clock 2: page 1 takes slot 1
      unbind 1   -> slot 1 empty, keeps stamp 2 (its place in the order)
      ensure [2] -> clock 3: candidates by (stamp, slot): slot 0 (1), slot 1 (2):
                    page 2 takes slot 0 and evicts page 0
      ensure [3] -> clock 4: slot 1 (2) before slot 0 (3): page 3 takes the
                    empty slot 1, nothing evicted
    Returns whether the final state is exactly that."""
    st = state_cls(4, 2)
    st.ensure([0])
    st.ensure([1])
    st.unbind(1)
    st.ensure([2])
    st.ensure([3])
    return (list(st.page_to_slot) == [-1, -1, 0, 1] and list(st.slot_to_page) == [2, 3]
            and list(st.stamp) == [3, 4] and st.counters["evictions"] == 1 and st.counters["misses"] == 4)


class _StampResetLRU(LRUState):
    """A plausible wrong unbind: the emptied slot goes back to stamp 0
    (first in line, like a never-used slot)."""

    def unbind(self, page):
        s = int(self.page_to_slot[page])
        super().unbind(page)
        if s >= 0:
            self.stamp[s] = 0


def test_unbind_keeps_the_slots_recency():
    assert _unbind_trace(LRUState)
    assert not _unbind_trace(_StampResetLRU)
