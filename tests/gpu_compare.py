"""Helpers that compare the HIP tier with the oracle tier (GPU tests only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle.codecs import bf16_bits_from_f32

ATOL, RTOL = 2e-2, 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(gpu - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside {ATOL}+{RTOL}|ref|, "
                           f"max err {err.max():.3g}")


def compare_state(g, o, where: str, check_rows=True, sample_pages=None):
    """LRU state, counters, slab, mirror rows and resident pool rows."""
    t = g.tier
    torch.cuda.synchronize()
    st = t.read_state()
    assert np.array_equal(st["page_to_slot"], o.lru.page_to_slot), f"{where}: page_to_slot"
    assert np.array_equal(st["slot_to_page"], o.lru.slot_to_page), f"{where}: slot_to_page"
    assert np.array_equal(st["stamp"], o.lru.stamp), f"{where}: stamp"
    assert st["clock"] == o.lru.clock, f"{where}: clock"
    cg = t.read_counters()
    co = o.counters()
    for k in ("ensure_calls", "hits", "misses", "fresh_allocs", "evictions", "drops", "bytes_fetched",
              "bytes_mirrored", "error_word"):
        assert cg[k] == co[k], f"{where}: counter {k}: gpu {cg[k]} oracle {co[k]}"
    assert cg["clock"] == o.lru.clock
    slab_g = t.slab_view().view(torch.int16).cpu().numpy().view(np.uint16)
    slab_o = bf16_bits_from_f32(o.slab)
    assert np.array_equal(slab_g, slab_o), f"{where}: slab"
    if not check_rows:
        return
    mir = t.mirror()
    pages = range(o.N) if sample_pages is None else sample_pages
    for p in pages:
        ref = o.mirror_row(p)
        assert np.array_equal(mir[p], ref), f"{where}: mirror row {p}"
    pool = t.pool_rows()
    for s in range(o.S):
        p = int(o.lru.slot_to_page[s])
        if p < 0:
            continue
        if sample_pages is not None and p not in sample_pages:
            continue
        row = pool[s].cpu().numpy()
        assert np.array_equal(row, o.pool_row(s)), f"{where}: pool slot {s} (page {p})"


def compare_layer(g, rec, layer, where: str, attention=True):
    wl = g.wl
    B, C = wl.batch, g.C
    sel = g.sel[layer].cpu().numpy()
    assert np.array_equal(sel, rec["sel"]), f"{where}: sel_local\n{sel}\n{rec['sel']}"
    needed = g.needed[layer].cpu().numpy()
    assert np.array_equal(needed, rec["needed"]), f"{where}: needed"
    out_slots = g.out_slots[layer].cpu().numpy()
    assert np.array_equal(out_slots, rec["out_slots"]), f"{where}: out_slots"
    m = int(g.miss_count[layer].item())
    miss = g.miss[layer].cpu().numpy()[:m]
    assert m == len(rec["misses"]) and np.array_equal(miss, rec["misses"]), f"{where}: miss list"
    if attention and rec.get("out") is not None:
        out = bf16_to_f64(g.out[layer])
        assert_close(out, rec["out"], f"{where}: attention")
