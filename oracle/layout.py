"""Byte layout of one logical page's row, shared by the host mirror and a GPU
pool slot (they must hold identical bytes: FreeToken PR #499, "Design", the
write-through mirror means no slot ever holds bytes the mirror lacks).

One row holds the page for ALL layers (PR #499 "Design": one copy moves K+V
of a page across all layers; PR #525 commit summary: the copy descriptor
also carries the scale banks).  Per layer, at offset ``layer * layer_bytes``:

* fp8:  K codes  uint8 [Hkv][page][d]
        V codes  uint8 [Hkv][d][page]     (transposed: a token's values are a column)
        K scales f32   [page]          (one scale per token over Hkv*d values)
        V scales f32   [page]
* bf16: K        bf16  [Hkv][page][d]
        V        bf16  [Hkv][page][d]
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class RowLayout:
    num_layers: int
    num_kv_heads: int
    page_size: int
    head_dim: int
    fp8: bool

    @property
    def code_bytes(self) -> int:
        """Bytes of one of K or V codes/values for one layer-page."""
        elt = 1 if self.fp8 else 2
        return self.num_kv_heads * self.page_size * self.head_dim * elt

    @property
    def layer_bytes(self) -> int:
        scales = 2 * 4 * self.page_size if self.fp8 else 0
        return 2 * self.code_bytes + scales

    @property
    def row_bytes(self) -> int:
        return self.num_layers * self.layer_bytes

    def k_off(self, layer: int) -> int:
        return layer * self.layer_bytes

    def v_off(self, layer: int) -> int:
        return layer * self.layer_bytes + self.code_bytes

    def ks_off(self, layer: int) -> int:
        assert self.fp8
        return layer * self.layer_bytes + 2 * self.code_bytes

    def vs_off(self, layer: int) -> int:
        assert self.fp8
        return layer * self.layer_bytes + 2 * self.code_bytes + 4 * self.page_size
