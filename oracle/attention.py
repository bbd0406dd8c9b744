"""Sparse paged attention over the selected pages (FreeToken PR #499,
"Design": after ensure the block table is translated logical->physical and
the sparse paged attention kernel reads only the selected pages; vLLM RFC
#33980, "Proposed Change": attention over the top-k KV only).

For a query row and query head h (KV group g = h // (Hq/Hkv)):

    T   = tokens 64*i + j of the selected, resident pages i with position
          < ctx_len (and <= the row's own position for a prefill row)
    z_t = (q_h . k_t) / sqrt(d)         k_t, v_t dequantised (code * scale)
    o   = sum_t softmax(z)_t v_t        (zero vector when T is empty)

all in fp64.  No sink, soft-cap or bias.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [Hq][d]; k, v [Hkv][T][d] (fp64) -> out [Hq][d] fp64."""
    Hq, d = q.shape
    Hkv, T, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, d), dtype=np.float64)
    if T == 0:
        return out
    for h in range(Hq):
        g = h // G
        z = (k[g] @ q[h].astype(np.float64)) / np.sqrt(d)
        z = z - z.max()
        p = np.exp(z)
        p /= p.sum()
        out[h] = p @ v[g]
    return out


def dense_reference(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Textbook softmax(q K^T / sqrt(d)) V with the KV head repeated per group,
    written as whole-matrix products (the sparse == dense pin)."""
    Hq, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=0)                   # [Hq][T][d]
    vv = np.repeat(v, G, axis=0)
    logits = np.einsum("hd,htd->ht", q.astype(np.float64), kk) / np.sqrt(d)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return np.einsum("ht,htd->hd", w, vv)
