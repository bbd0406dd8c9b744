"""CPU oracle for the tiered KV-cache sparse decode path -- TEST INFRASTRUCTURE.

A plain, slow, obviously correct NumPy implementation of what the HIP library
computes, written from the pages that describe the method:

* FreeToken PR #499, "feat(kvcache): host-RAM KV tier for sparse-attention
  models (--kv-host-pages)" -- sections "What", "Why this works for sparse
  attention", "Design" (write-through mirror, device-side LRU, fused page
  copy across layers, logical->physical block table, fixed-shape
  compact_selected_pages with a drop counter), "Known limitations";
* FreeToken PR #525, "feat(kvcache): host-resident prefix tier for hybrid GDN
  models" -- the commit summary (mirror_store_quant: the mirror takes e4m3
  codes plus fp32 scales read after quantisation; set_select_width: the
  batch's selection must fit the pool) and the downstream commit (formats
  whose scales the mirror cannot hold are refused with an error naming the
  knob);
* vLLM issue #33980, "[RFC]: Sparse attention KV cache offloading" --
  "Proposed Change" (only the top-k KV is brought to the GPU).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
and never reads anything the HIP path produced: both consume the same seeded
inputs from ``workload``.

Floating point is fp64 wherever the result is a plain definition (scores,
attention); fp32 exactly where the method fixes fp32 (the per-token fp8
scale and the division by it, the indexer key).
"""
