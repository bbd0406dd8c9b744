"""Device-side LRU residency over a fixed pool of GPU slots (FreeToken PR #499,
"What": the GPU pool is an LRU cache of physical slots over the logical page
space; "Design": lru_ensure is fixed-shape and the mirror is write-through,
so eviction is a pure rebind with no write-back).

State: page_to_slot[N], slot_to_page[S] (-1 = empty), stamp[S] (0 = never
used), clock.  One ``ensure`` call over a list of needed logical pages:

1. reject the call (no state change) if it needs more distinct pages than
   there are slots -- PR #525's set_select_width makes that impossible by
   construction; ids outside [-1, N) are flagged and ignored; -1 is padding;
2. clock += 1;
3. distinct pages in first-occurrence order; a resident page is a hit and is
   restamped with the new clock;
4. the misses, in first-occurrence order, take the slots not hit by this
   call in ascending (stamp, slot) order -- free slots (stamp 0) first,
   lowest index first; the page a victim slot held loses its residency;
5. each miss is emitted as (slot, page) for the fetch unless its first
   occurrence is marked no_fetch (a page being written for the first time
   has nothing in the mirror yet);
6. out_slots[j] = slot of needed[j] (or -1).

All pages touched by one call are equally recent (one clock tick per call).
"""
from __future__ import annotations

import numpy as np

ERR_PAGE_RANGE = 1
ERR_CAPACITY = 2


class LRUState:
    def __init__(self, num_pages: int, num_slots: int):
        self.N, self.S = int(num_pages), int(num_slots)
        self.reset()

    def reset(self):
        self.page_to_slot = np.full(self.N, -1, dtype=np.int32)
        self.slot_to_page = np.full(self.S, -1, dtype=np.int32)
        self.stamp = np.zeros(self.S, dtype=np.int64)
        self.clock = 0
        self.counters = dict(ensure_calls=0, hits=0, misses=0, fresh_allocs=0, evictions=0)
        self.error_word = 0

    def unbind(self, page):
        """Forget a resident page: its slot becomes empty and keeps its stamp
        (its place in the recency order); later taking it as a victim evicts
        nothing."""
        s = int(self.page_to_slot[page])
        if s >= 0:
            self.page_to_slot[page] = -1
            self.slot_to_page[s] = -1

    def ensure(self, needed, no_fetch=None):
        """Returns (out_slots int32 [W], miss list int32 [m][2] as (slot, page))."""
        needed = np.asarray(needed, dtype=np.int64).reshape(-1)
        W = len(needed)
        nf = np.zeros(W, dtype=bool) if no_fetch is None else np.asarray(no_fetch, dtype=bool)
        first = {}                                  # page -> first index
        for j, p in enumerate(needed):
            if p == -1:
                continue
            if p < -1 or p >= self.N:
                self.error_word |= ERR_PAGE_RANGE
                continue
            if p not in first:
                first[int(p)] = j
        if len(first) > self.S:
            self.error_word |= ERR_CAPACITY
            return np.full(W, -1, dtype=np.int32), np.zeros((0, 2), dtype=np.int32)

        self.clock += 1
        clock = self.clock
        hit_slots = set()
        miss_pages = []
        for p, j in sorted(first.items(), key=lambda kv: kv[1]):
            s = int(self.page_to_slot[p])
            if s >= 0:
                self.stamp[s] = clock
                hit_slots.add(s)
                self.counters["hits"] += 1
            else:
                miss_pages.append((p, j))

        candidates = [s for s in range(self.S) if s not in hit_slots]
        candidates.sort(key=lambda s: (int(self.stamp[s]), s))
        victims = candidates[:len(miss_pages)]
        assert len(victims) == len(miss_pages)

        misses = []
        for (p, j), s in zip(miss_pages, victims):
            old = int(self.slot_to_page[s])
            if old >= 0:
                self.page_to_slot[old] = -1
                self.counters["evictions"] += 1
            self.page_to_slot[p] = s
            self.slot_to_page[s] = p
            self.stamp[s] = clock
            if nf[j]:
                self.counters["fresh_allocs"] += 1
            else:
                self.counters["misses"] += 1
                misses.append((s, p))
        self.counters["ensure_calls"] += 1

        out = np.full(W, -1, dtype=np.int32)
        for j, p in enumerate(needed):
            if 0 <= p < self.N:
                out[j] = self.page_to_slot[p]
        return out, np.array(misses, dtype=np.int32).reshape(-1, 2)
