"""The whole tier, step by step, in the order the pages give (FreeToken PR
#499, "Why this works for sparse attention" and "Design"):

    write path:  ensure_write_pages -> store (pool + write-through mirror + slab)
    decode path: select (indexer top-k) -> compact -> ensure -> fetch -> attention

Rows of a call are grouped by request: rows of request b are
``row_start[b] .. row_start[b+1]-1``.

Content modes.  With ``materialize=True`` the mirror and the pool are real
byte rows, written by the store and copied by the fetch.  With
``materialize=False`` (the full-size workloads) only the slab and the
per-page written-token counts are kept; the bytes of a page are rebuilt on
demand by ``row_builder(page)`` -- the same ``write_tokens`` arithmetic
applied to the page's tokens -- and a resident slot reads its page's mirror
row, which is what the write-through mirror guarantees (PR #499 "Design":
a slot never holds bytes the mirror lacks, so dropping it loses nothing).
"""
from __future__ import annotations

import numpy as np

from .attention import attend
from .layout import RowLayout
from .lru import LRUState
from .select import NO_BITS, ScoreCertificateError, compact_request, select_row, select_rows
from .store import read_kv, slab_entry, write_tokens

ERR_NOT_RESIDENT = 4      # store to a page that is not resident (pool not written)


class CapacityError(ValueError):
    pass


class SlabCertificateError(ArithmeticError):
    """A page's key sums cannot be proven exact in fp64."""


class OracleTier:
    def __init__(self, *, num_layers, num_q_heads, num_kv_heads, head_dim, page_size,
                 fp8, num_logical_pages, num_slots, materialize=True, row_builder=None):
        self.L, self.Hq, self.Hkv, self.d = num_layers, num_q_heads, num_kv_heads, head_dim
        self.ps, self.N, self.S = page_size, int(num_logical_pages), int(num_slots)
        self.lay = RowLayout(num_layers, num_kv_heads, page_size, head_dim, fp8)
        self.materialize = materialize
        self.row_builder = row_builder
        self.mirror = {}                      # page -> uint8 row
        self.pool = (np.zeros((self.S, self.lay.row_bytes), dtype=np.uint8)
                     if materialize else None)
        self._lazy_pool = {}                  # slot -> (page, row copied by the fetch)
        self.slab = np.zeros((self.L, self.N, self.Hkv, self.d), dtype=np.float32)
        # (layer, page) -> (fp64 key sum, fp64 sum of |key|, lowest-bit exponent)
        # of a partly written page; the last two certify the sum exact
        self._partial_sums = {}
        self.written = np.zeros(self.N, dtype=np.int64)   # tokens written per page (layer 0)
        self.lru = LRUState(self.N, self.S)
        self.drops = 0
        self.bytes_fetched = 0
        self.bytes_mirrored = 0
        self.max_sel_pages = None
        self.max_certificate = 0.0            # largest sum |qg * slab| seen by select
        self.max_score_bits = 0.0             # largest log2(A) - e_min seen by select
        # Exactness of the selection scores is asserted on every select: the
        # scores are fp32(exact dot product), and the certificate proves the
        # fp64 sums exact and that an accumulator of `score_bits` significand
        # bits reproduces them in any order -- 24 (fp32, the dense bf16
        # product of a prefill chunk) for rows with a causal position, 53
        # (fp64) for decode rows.  None switches the check off (inputs off the
        # workloads' grids, compared by a bound instead of bit for bit).
        self.check_scores = True

    # ------------------------------------------------------------ config --
    def set_select_width(self, max_bs, block_topk, max_sel_pages=0):
        """PR #525 commit summary (set_select_width takes the batch size): the
        width is chosen so that a full batch's compacted selection always has
        enough slots."""
        C = max_sel_pages if max_sel_pages > 0 else 2 * block_topk + 8
        if max_bs * C > self.S:
            raise CapacityError(f"max_bs*max_sel_pages={max_bs * C} > num_slots={self.S}")
        self.max_sel_pages = C
        return C

    def reset_residency(self):
        self.lru.reset()
        self._lazy_pool.clear()
        self.drops = self.bytes_fetched = self.bytes_mirrored = 0

    # ------------------------------------------------------------ rows ----
    def mirror_row(self, page: int) -> np.ndarray:
        if self.materialize:
            if page not in self.mirror:
                self.mirror[page] = np.zeros(self.lay.row_bytes, dtype=np.uint8)
            return self.mirror[page]
        return self.row_builder(page)

    def pool_row(self, slot: int) -> np.ndarray:
        if self.materialize:
            return self.pool[slot]
        page = int(self.lru.slot_to_page[slot])
        held = self._lazy_pool.get(slot)
        if held is not None and held[0] == page:
            return held[1]
        return self.row_builder(page)

    # ----------------------------------------------------- prefix tier ---
    def prefix_save(self, pages):
        """Copy-out of a cold prefix (FreeToken PR #525, "What the patch does",
        items 2 and 4): the pages' mirror rows and their indexer slab entries
        (bf16 values and the key sums of partly written pages), host side,
        since the mirror holds every written byte.  Returns a record list."""
        assert self.materialize, "prefix records need materialised rows"
        recs = []
        for p in pages:
            p = int(p)
            recs.append(dict(row=self.mirror_row(p).copy(), slab=self.slab[:, p].copy(),
                             sums={l: tuple(np.copy(x) for x in self._partial_sums[(l, p)])
                                   for l in range(self.L) if (l, p) in self._partial_sums},
                             written=int(self.written[p])))
        return recs

    def prefix_restore(self, pages, recs):
        """Rehydration (PR #525, item 3: with the offloader active the copy is
        host to host into its mirror and its lazy fetch covers residency):
        the records land in the mirror rows and slab entries of ``pages``
        (new logical ids), and any of these ids that is resident is unbound
        -- its slot holds the id's previous content -- keeping the slot's
        recency.  Nothing is fetched."""
        assert self.materialize and len(pages) == len(recs)
        assert len(set(int(p) for p in pages)) == len(pages)
        for p, r in zip(pages, recs):
            p = int(p)
            self.mirror[p] = r["row"].copy()
            self.slab[:, p] = r["slab"]
            for l in range(self.L):
                self._partial_sums.pop((l, p), None)
            for l, v in r["sums"].items():
                self._partial_sums[(l, p)] = tuple(np.copy(x) for x in v)
            self.written[p] = r["written"]
            self.lru.unbind(p)

    # ------------------------------------------------------------ write ---
    def ensure_write_pages(self, runs, block_table, old_len):
        """runs: list of (req, start, length).  Every page a run touches is made
        resident; a page whose first position is >= the request's old length
        has no content yet and is allocated without a fetch."""
        needed, nofetch = [], []
        for req, start, length in runs:
            if length <= 0:
                continue
            for lp in range(start // self.ps, (start + length - 1) // self.ps + 1):
                needed.append(int(block_table[req][lp]))
                nofetch.append(lp * self.ps >= old_len[req])
        out, misses = self.lru.ensure(np.array(needed, dtype=np.int64), np.array(nofetch, dtype=bool))
        self.fetch(misses)
        return out, misses

    def store(self, layer, runs, k, v, block_table):
        """k, v float32 [n_tok][Hkv][d], tokens of the runs concatenated in order.
        The pages must be resident (ensure_write_pages first); a page that is
        not is still written to the mirror and the slab, and flagged."""
        off = 0
        for req, start, length in runs:
            pos = start
            while pos < start + length:
                lp = pos // self.ps
                a = pos - lp * self.ps
                n = min(self.ps - a, start + length - pos)
                page = int(block_table[req][lp])
                kk = k[off:off + n]
                vv = v[off:off + n]
                slot = int(self.lru.page_to_slot[page])
                if slot < 0:
                    self.lru.error_word |= ERR_NOT_RESIDENT
                if self.materialize:
                    write_tokens(self.mirror_row(page), self.lay, layer, a, kk, vv)
                    if slot >= 0:
                        write_tokens(self.pool[slot], self.lay, layer, a, kk, vv)
                # slab: mean of all written keys of the page
                key = (layer, page)
                prev = self._partial_sums.pop(key, None) if a > 0 else None
                k64 = kk.astype(np.float64)
                s = k64.sum(axis=0)
                mags = np.abs(k64)
                sabs = mags.sum(axis=0)
                # every fp32 value of magnitude >= m is a multiple of 2^(floor(log2 m) - 23)
                mn = np.where(mags > 0, mags, np.inf).min(axis=0)
                lsb = np.where(np.isfinite(mn), np.frexp(np.where(np.isfinite(mn), mn, 1.0))[1] - 24, NO_BITS)
                if prev is not None:
                    s, sabs, lsb = s + prev[0], sabs + prev[1], np.minimum(lsb, prev[2])
                self._certify_slab(sabs, lsb, layer, page)
                cnt = a + n
                if cnt < self.ps:
                    self._partial_sums[key] = (s, sabs, lsb)
                self.slab[layer, page] = slab_entry_from_sum(s, cnt)
                if layer == 0:
                    self.written[page] = cnt
                tok_bytes = self.lay.layer_bytes // self.ps
                self.bytes_mirrored += (n + (self.ps - cnt if a == 0 else 0)) * tok_bytes
                pos += n
                off += n

    # ------------------------------------------------------------ decode --
    def select(self, layer, q, row_start, row_pos, block_table, n_pages, topk, bias=None):
        """q float32 [rows][Hq][d] -> (sel_local int32 [rows][topk], needed int32 [B][C])."""
        B = len(n_pages)
        rows = q.shape[0]
        sel = np.full((rows, topk), -1, dtype=np.int32)
        need = 24 if row_pos is not None else 53
        for b in range(B):
            r0, r1 = int(row_start[b]), int(row_start[b + 1])
            if r1 - r0 > 8:
                pos = None if row_pos is None else np.asarray(row_pos[r0:r1])
                sel[r0:r1], cert = select_rows(q[r0:r1], self.slab[layer], block_table[b], int(n_pages[b]),
                                               topk, self.Hkv, bias, pos, self.ps)
                self._certify(cert, need, layer, b)
                continue
            for r in range(r0, r1):
                pos = None if row_pos is None else int(row_pos[r])
                sel[r], cert = select_row(q[r], self.slab[layer], block_table[b], int(n_pages[b]),
                                          topk, self.Hkv, bias, pos, self.ps)
                self._certify(cert, need, layer, b)
        C = self.max_sel_pages
        needed = np.full((B, C), -1, dtype=np.int32)
        for b in range(B):
            needed[b], drops = compact_request(sel[row_start[b]:row_start[b + 1]], block_table[b], C)
            self.drops += drops
        return sel, needed

    def _certify_slab(self, sabs, lsb, layer, page):
        """Every key of the page (per feature) is a multiple of 2^lsb (a lower
        bound: floor(log2 of the smallest nonzero |key|) - 23) and the
        partial sums stay below sum |key|, so the fp64 sums -- in any order,
        the oracle's and an fp64 accumulator's alike -- are exact when
        sum |key| < 2^(53 + lsb)."""
        live = lsb < NO_BITS
        if np.any(live & (sabs >= np.ldexp(1.0, np.minimum(53 + lsb, 1000)))):
            raise SlabCertificateError(f"layer {layer}, page {page}: the key sums are not exact in fp64")

    def _certify(self, cert, need_bits, layer, b):
        A, bits = cert
        self.max_certificate = max(self.max_certificate, A)
        self.max_score_bits = max(self.max_score_bits, bits)
        if self.check_scores and bits >= need_bits:
            raise ScoreCertificateError(
                f"layer {layer}, request {b}: the score sums need {bits:.1f} significand bits "
                f"(sum |qg*slab| = {A:.6g}); exact selection needs < {need_bits}")

    def ensure(self, needed, no_fetch=None):
        return self.lru.ensure(np.asarray(needed).reshape(-1), no_fetch)

    def fetch(self, misses):
        """Copy the mirror row of each missed page into its slot, all layers and
        all banks at once."""
        for slot, page in np.asarray(misses).reshape(-1, 2):
            if self.materialize:
                self.pool[slot][:] = self.mirror_row(int(page))
            else:
                self._lazy_pool[int(slot)] = (int(page), self.mirror_row(int(page)).copy())
            self.bytes_fetched += self.lay.row_bytes

    def gather_kv(self, layer, b, sel_row, block_table, ctx_len, row_pos=None, host_tail=False):
        """Dequantised K, V [Hkv][T][d] of the selected pages' visible tokens.

        Resident pages are read from their pool slot.  A page that is not
        resident is skipped, or with ``host_tail`` read in place from its
        mirror row (vLLM RFC #33980, discussion: the tail of the KV space is
        host memory that the attention kernel loads over the interconnect,
        with no staging copy; only this layer's block of the row is used)."""
        ks, vs = [], []
        limit = int(ctx_len[b]) if row_pos is None else min(int(ctx_len[b]), int(row_pos) + 1)
        for i in sel_row:
            if i < 0:
                continue
            page = int(block_table[b][i])
            slot = int(self.lru.page_to_slot[page])
            if slot < 0 and not host_tail:
                continue
            n = min(self.ps, limit - int(i) * self.ps)
            if n <= 0:
                continue
            row = self.pool_row(slot) if slot >= 0 else self.mirror_row(page)
            k, v = read_kv(row, self.lay, layer)
            ks.append(k[:, :n])
            vs.append(v[:, :n])
        if not ks:
            z = np.zeros((self.Hkv, 0, self.d))
            return z, z
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)

    def attention_row(self, layer, q_row, b, sel_row, block_table, ctx_len, row_pos=None, host_tail=False):
        k, v = self.gather_kv(layer, b, sel_row, block_table, ctx_len, row_pos, host_tail)
        return attend(q_row.astype(np.float64), k, v)

    def attention(self, layer, q, row_start, row_pos, ctx_len, sel, block_table, host_tail=False):
        out = np.zeros(q.shape, dtype=np.float64)
        for b in range(len(row_start) - 1):
            for r in range(row_start[b], row_start[b + 1]):
                pos = None if row_pos is None else row_pos[r]
                out[r] = self.attention_row(layer, q[r], b, sel[r], block_table, ctx_len, pos, host_tail)
        return out

    def decode_layer(self, layer, q, row_start, block_table, n_pages, ctx_len, topk,
                     bias=None, row_pos=None, with_attention=True):
        sel, needed = self.select(layer, q, row_start, row_pos, block_table, n_pages, topk, bias)
        out_slots, misses = self.ensure(needed)
        self.fetch(misses)
        out = (self.attention(layer, q, row_start, row_pos, ctx_len, sel, block_table)
               if with_attention else None)
        return dict(sel=sel, needed=needed, out_slots=out_slots, misses=misses, out=out)

    def decode_layer_prefetch(self, layer, q, row_start, block_table, n_pages, ctx_len, topk, pred,
                              bias=None, row_pos=None, with_attention=True):
        """The decode layer preceded by a preload of a predicted page list
        (vLLM RFC #33980, "Topk KV preload": an earlier top-k index -- from
        the previous step or layer -- is loaded ahead, and only the pages it
        missed are loaded after the real selection).  Reading taken: the
        preload is an ensure of ``pred`` (logical ids, -1 ignored) with the
        fetch of its misses, ordered before this layer's selection; its copy
        may overlap the selection in time, which changes no result."""
        pred = np.asarray(pred, dtype=np.int64).reshape(-1)
        pre_slots, pre_misses = self.ensure(pred)
        self.fetch(pre_misses)
        rec = self.decode_layer(layer, q, row_start, block_table, n_pages, ctx_len, topk, bias=bias,
                                row_pos=row_pos, with_attention=with_attention)
        rec["pre_misses"] = pre_misses
        return rec

    def decode_layer_host_tail(self, layer, q, row_start, block_table, n_pages, ctx_len, topk,
                               bias=None, row_pos=None):
        """The decode layer with the host tail read in place: selection and
        compaction as usual, no ensure and no fetch (the residency state does
        not move), attention over pool slots and mirror rows."""
        sel, needed = self.select(layer, q, row_start, row_pos, block_table, n_pages, topk, bias)
        out = self.attention(layer, q, row_start, row_pos, ctx_len, sel, block_table, host_tail=True)
        return dict(sel=sel, needed=needed, out=out)

    def counters(self):
        c = dict(self.lru.counters)
        c.update(drops=self.drops, bytes_fetched=self.bytes_fetched,
                 bytes_mirrored=self.bytes_mirrored, error_word=self.lru.error_word)
        return c


def slab_entry_from_sum(s: np.ndarray, n: int) -> np.ndarray:
    """bf16(fp32(sum) / n) -- the mean of n written keys given their exact sum."""
    from .codecs import bf16_round
    return bf16_round(s.astype(np.float32) / np.float32(n))


__all__ = ["OracleTier", "CapacityError", "ScoreCertificateError", "SlabCertificateError", "slab_entry",
           "slab_entry_from_sum"]
