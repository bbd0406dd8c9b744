"""The C-ABI library loads and exports every entry point its header declares;
configuration checks that need no GPU (sizes, refused formats, bad shapes)."""
import ctypes as C
import os
import re

import pytest

from tiered_kv_cache_indexer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tkv.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|int64_t|void|const char\*|const void\*)\s+(tkv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_path():
    names = _declared()
    for n in ("tkv_select_pages", "tkv_lru_ensure", "tkv_fetch_pages", "tkv_sparse_paged_attn",
              "tkv_store_kv_mirror", "tkv_decode_layer", "tkv_ensure_write_pages"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_lib.SIGNATURES) == set(_declared())


def _cfg(**kw):
    base = dict(num_layers=12, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                kv_format=_lib.KV_FP8, num_logical_pages=3072, num_slots=256, max_batch=1,
                max_rows=1, max_topk=32, max_pages_per_req=3072, max_width=256)
    base.update(kw)
    return _lib.Config(*[base[f] for f, _ in _lib.Config._fields_])


def _sizes(cfg):
    s = _lib.Sizes()
    rc = _lib.load().tkv_required_bytes(C.byref(cfg), C.byref(s))
    return rc, s


def test_sizes_match_row_layout():
    rc, s = _sizes(_cfg())
    assert rc == 0
    assert s.layer_bytes == 66048 and s.row_bytes == 792576
    assert s.pool_bytes == 256 * 792576 and s.mirror_bytes == 3072 * 792576
    assert s.slab_bytes == 12 * 3072 * 4 * 128 * 2
    rc, s = _sizes(_cfg(num_layers=1, num_q_heads=8, num_kv_heads=1, page_size=16, kv_format=_lib.KV_BF16,
                        num_logical_pages=256, num_slots=64, max_pages_per_req=256))
    assert rc == 0 and s.row_bytes == 8192


def test_nvfp4_is_refused_naming_the_knob():
    rc, _ = _sizes(_cfg(kv_format=_lib.KV_NVFP4))
    assert rc == -2
    assert b"kv_format" in _lib.load().tkv_last_error()


@pytest.mark.parametrize("kw,knob", [
    (dict(head_dim=64), b"head_dim"),
    (dict(num_q_heads=16), b"num_q_heads"),
    (dict(page_size=32), b"page_size"),
    (dict(max_width=70000), b"max_width"),
    (dict(num_slots=0), b"num_slots"),
])
def test_bad_shapes_rejected(kw, knob):
    rc, _ = _sizes(_cfg(**kw))
    assert rc == -1
    assert knob in _lib.load().tkv_last_error()
