"""Seeded synthetic inputs for the tiered KV-cache decode path.

This package is input generation only.  It holds none of the method's
arithmetic (no scoring, top-k, LRU, quantisation or attention): it produces
the key/value tokens, queries, page-importance bias and block tables that
both the CPU oracle and the HIP library consume.

The bulk key/value/prefill-query tensors come from one counter-based
generator, Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011), mapped through an inverse-normal
lookup table onto an exact grid.  It is implemented twice: in NumPy
(``gen.py``, which is NumPy's own ``Philox`` bit generator) and in HIP
(``csrc/gen.hip``), so the GPU can generate gigabytes of context without a
host upload while the oracle regenerates any page on its own.
"""
from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
