"""store_kv with the write-through mirror (FreeToken PR #499 "Design";
PR #525 commit summary, mirror_store_quant).

Per token and per tensor (K, V) over all Hkv*d values:

    amax  = max |x|
    scale = fp32(amax / 448)        (1.0 when amax == 0)
    code  = e4m3(fp32(x / scale))   (one correctly rounded fp32 division)

The mirror receives the quantiser's output -- codes and scales, the same
bytes the pool holds (PR #525 commit summary, mirror_store_quant: an earlier
mirror that kept the values from before quantisation left fp8 pages wrong
with no error raised).  For a
bf16 cache the bf16 values are stored verbatim and there are no scales.

The indexer slab entry of a page is the mean of its written bf16 keys,
rounded once to bf16: ``slab = bf16(fp32(sum_t K[t]) / n_written)``.

When a write begins a page (its first token is the page's offset 0), the
token positions of that page after the write are zero-filled, so that a slot
that previously held another page holds exactly the mirror's bytes.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_from_f32, bf16_round, e4m3_encode
from .layout import RowLayout


def quantize_tokens(x: np.ndarray):
    """x float32 [n][Hkv][d] (bf16-exact values) -> (codes uint8 [n][Hkv][d], scales f32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    amax = np.abs(x.reshape(n, -1)).max(axis=1).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    q = (x / scale[:, None, None]).astype(np.float32)   # fp32 / fp32: correctly rounded
    return e4m3_encode(q), scale


def write_tokens(row: np.ndarray, lay: RowLayout, layer: int, off: int,
                 k: np.ndarray, v: np.ndarray) -> None:
    """Write tokens [off, off+n) of one page/layer into a row (uint8 view)."""
    n = k.shape[0]
    H, P, D = lay.num_kv_heads, lay.page_size, lay.head_dim
    assert 0 <= off and off + n <= P
    if lay.fp8:
        kc, ks = quantize_tokens(k)
        vc, vs = quantize_tokens(v)
        kblk = row[lay.k_off(layer):lay.k_off(layer) + lay.code_bytes].reshape(H, P, D)
        vblk = row[lay.v_off(layer):lay.v_off(layer) + lay.code_bytes].reshape(H, D, P)
        kblk[:, off:off + n, :] = kc.transpose(1, 0, 2)
        vblk[:, :, off:off + n] = vc.transpose(1, 2, 0)
        row[lay.ks_off(layer):lay.ks_off(layer) + 4 * P].view(np.float32)[off:off + n] = ks
        row[lay.vs_off(layer):lay.vs_off(layer) + 4 * P].view(np.float32)[off:off + n] = vs
        if off == 0:
            kblk[:, n:, :] = 0
            vblk[:, :, n:] = 0
            row[lay.ks_off(layer):lay.ks_off(layer) + 4 * P].view(np.float32)[n:] = 0
            row[lay.vs_off(layer):lay.vs_off(layer) + 4 * P].view(np.float32)[n:] = 0
    else:
        kblk = row[lay.k_off(layer):lay.k_off(layer) + lay.code_bytes].view(np.uint16).reshape(H, P, D)
        vblk = row[lay.v_off(layer):lay.v_off(layer) + lay.code_bytes].view(np.uint16).reshape(H, P, D)
        kblk[:, off:off + n, :] = bf16_bits_from_f32(k).transpose(1, 0, 2)
        vblk[:, off:off + n, :] = bf16_bits_from_f32(v).transpose(1, 0, 2)
        if off == 0:
            kblk[:, n:, :] = 0
            vblk[:, n:, :] = 0


def slab_entry(k_written: np.ndarray) -> np.ndarray:
    """Mean of a page's written keys, k_written float32 [n][Hkv][d] -> float32
    [Hkv][d] holding bf16 values: bf16(fp32(exact sum) / n).  The fp64 sum is
    exact for the keys the tier certifies (see OracleTier._certify_slab)."""
    n = k_written.shape[0]
    s = k_written.astype(np.float64).sum(axis=0).astype(np.float32)
    return bf16_round(s / np.float32(n))


def read_kv(row: np.ndarray, lay: RowLayout, layer: int):
    """Dequantised K and V of one layer of a row: float64 [Hkv][page][d] each."""
    from .codecs import e4m3_decode, bf16_bits_to_f32
    H, P, D = lay.num_kv_heads, lay.page_size, lay.head_dim
    if lay.fp8:
        kc = row[lay.k_off(layer):lay.k_off(layer) + lay.code_bytes].reshape(H, P, D)
        vc = row[lay.v_off(layer):lay.v_off(layer) + lay.code_bytes].reshape(H, D, P).transpose(0, 2, 1)
        ks = row[lay.ks_off(layer):lay.ks_off(layer) + 4 * P].view(np.float32)
        vs = row[lay.vs_off(layer):lay.vs_off(layer) + 4 * P].view(np.float32)
        k = e4m3_decode(kc).astype(np.float64) * ks.astype(np.float64)[None, :, None]
        v = e4m3_decode(vc).astype(np.float64) * vs.astype(np.float64)[None, :, None]
    else:
        k = bf16_bits_to_f32(row[lay.k_off(layer):lay.k_off(layer) + lay.code_bytes]
                             .view(np.uint16).reshape(H, P, D)).astype(np.float64)
        v = bf16_bits_to_f32(row[lay.v_off(layer):lay.v_off(layer) + lay.code_bytes]
                             .view(np.uint16).reshape(H, P, D)).astype(np.float64)
    return k, v
