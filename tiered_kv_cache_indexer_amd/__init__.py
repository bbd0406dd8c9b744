"""Tiered KV-cache sparse decode for MI355X (gfx950).

The hot path of a sparse-attention decode step over a paged KV cache whose
backing store is a pinned host mirror (FreeToken PR #499, "host-RAM KV tier
for sparse-attention models"): indexer top-k page selection, compaction with
a drop counter, a device-side LRU over GPU slots, a fused host->device page
fetch across layers, sparse paged attention, and the write-through store.
All of it runs in hand-written HIP kernels behind the C ABI of
``include/tkv.h``; :class:`TieredKV` is a thin PyTorch-facing binding with the
same call names.
"""
from ._lib import (ERR_BAD_MISS, ERR_CAPACITY, ERR_NOT_RESIDENT, ERR_PAGE_RANGE, KV_BF16,  # noqa: F401
                   KV_FP8, KV_NVFP4, TkvError)
from .tier import TieredKV  # noqa: F401
