"""The five synthetic workloads and their reduced test variants.

Shapes follow the decode setting of FreeToken PR #499 ("host-RAM KV tier for
sparse-attention models"): 64-token pages, an indexer budget of 2,048 tokens,
fp8 KV, 12 sparse-attention layers, a pool of 1,635 GPU pages ("Measured",
Config A).  Every field here is a size or a seed: nothing in this file
computes any step of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_format: str            # "bf16" or "fp8"
    contexts: tuple           # cached context tokens per request
    topk: int                 # pages kept per query row (block_topk)
    num_slots: int            # GPU pool slots
    steps: int                # decode steps (or prefill chunks)
    query: str = "iid"        # "iid" | "ar" | "ar_literal"
    bias: str = "none"        # "none" | "zipf"
    permute_pages: bool = False
    setup_chunk: int = 4096   # tokens written per setup call
    prefill_tokens: int = 0   # >0: one prefill chunk of this many new tokens
    append: bool = False      # decode steps append one token per request
    zipf_s: float = 1.1
    values: str = "grid"      # "grid": N(0,1) on the 2^-4 / 2^-5 grids; "bf16": N(0,1) rounded to bf16
    description: str = field(default="", compare=False)

    # ---- derived sizes (plain arithmetic on the fields above) ----
    @property
    def batch(self) -> int:
        return len(self.contexts)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def pages_of(self, b: int) -> int:
        """Pages request b holds after setup (and after the prefill chunk, or
        after the last appended decode token)."""
        toks = self.contexts[b] + (self.prefill_tokens if b == 0 else 0) + (self.steps if self.append else 0)
        return -(-toks // self.page_size)

    @property
    def num_logical_pages(self) -> int:
        return sum(self.pages_of(b) for b in range(self.batch))

    @property
    def max_pages(self) -> int:
        return max(self.pages_of(b) for b in range(self.batch))

    @property
    def max_sel_pages(self) -> int:
        """Decode cap 2*block_topk + 8; the prefill union cap is the whole
        visible page range of the chunk's request."""
        if self.prefill_tokens:
            return min(self.num_slots, self.pages_of(0))
        return 2 * self.topk + 8


WORKLOADS = {
    # config 1: the correctness config
    "c1": Workload(
        name="c1_tiny_bf16", seed=1001, num_layers=1, num_q_heads=8, num_kv_heads=1,
        head_dim=128, page_size=16, kv_format="bf16", contexts=(4096,), topk=16,
        num_slots=64, steps=8, query="iid", setup_chunk=1024,
        description="1 layer, 8q/1kv, page 16, ctx 4,096, bf16 KV, top-16, 64 slots, 8 steps"),
    # config 2: pool holds every page -> no misses after setup; HBM-bound
    "c2": Workload(
        name="c2_64k_resident", seed=1002, num_layers=12, num_q_heads=32, num_kv_heads=4,
        head_dim=128, page_size=64, kv_format="fp8", contexts=(65536,), topk=32,
        num_slots=1024, steps=64, query="ar",
        description="12 layers, 32q/4kv, page 64, ctx 65,536, fp8, top-32 pages, 1,024 slots, 64 steps"),
    # config 3: the headline: 196k context, 256-slot pool, Zipf page bias -> LRU thrash
    "c3": Workload(
        name="c3_196k_thrash", seed=1003, num_layers=12, num_q_heads=32, num_kv_heads=4,
        head_dim=128, page_size=64, kv_format="fp8", contexts=(196608,), topk=32,
        num_slots=256, steps=128, query="ar", bias="zipf",
        description="12 layers, ctx 196,608, fp8, top-2,048 tokens, 256 slots, Zipf(1.1) bias, 128 steps"),
    # config 4: batch 4, mixed contexts, permuted logical pages
    "c4": Workload(
        name="c4_batch4_mixed", seed=1004, num_layers=12, num_q_heads=32, num_kv_heads=4,
        head_dim=128, page_size=64, kv_format="fp8", contexts=(32768, 98304, 196608, 262144),
        topk=32, num_slots=1635, steps=64, query="ar", permute_pages=True,
        description="batch 4, ctx {32k,96k,196k,262,144}, fp8, top-32/request, 1,635 slots, 64 steps"),
    # config 5: one prefill chunk of 4,096 tokens over 65,536 cached
    "c5": Workload(
        name="c5_prefill_4k_over_64k", seed=1005, num_layers=12, num_q_heads=32, num_kv_heads=4,
        head_dim=128, page_size=64, kv_format="fp8", contexts=(65536,), topk=32,
        num_slots=1635, steps=1, query="ar", prefill_tokens=4096,
        description="prefill 4,096 new over 65,536 cached, 12 layers, per-query top-32 pages"),
}

# Reduced variants with the same structure, small enough for the oracle to run
# every layer of every step in seconds.
WORKLOADS.update({
    "c2s": replace(WORKLOADS["c2"], name="c2_small", contexts=(8192,), num_slots=128,
                   num_layers=3, steps=6, setup_chunk=2048),
    "c3s": replace(WORKLOADS["c3"], name="c3_small_thrash", contexts=(16384,), num_slots=24,
                   num_layers=4, steps=8, setup_chunk=1024, topk=8),
    "c4s": replace(WORKLOADS["c4"], name="c4_small_mixed", contexts=(2048, 4096, 6432, 8192),
                   num_slots=160, num_layers=2, steps=5, setup_chunk=2048, topk=8),
    # pools of 3x the batch width: a split decode call's copies chain on the previous call's
    "c3sc": replace(WORKLOADS["c3"], name="c3_small_thrash_chain", contexts=(16384,), num_slots=72,
                    num_layers=5, steps=8, setup_chunk=2048, topk=8, query="iid"),
    "c4sc": replace(WORKLOADS["c4"], name="c4_small_mixed_chain", contexts=(2048, 4096, 6432, 8192),
                    num_slots=288, num_layers=3, steps=5, setup_chunk=2048, topk=8, query="iid"),
    "c5s": replace(WORKLOADS["c5"], name="c5_small_prefill", contexts=(4096,), prefill_tokens=512,
                   num_slots=160, num_layers=2, setup_chunk=2048, topk=8),
})

# The same structure with general bf16 inputs: keys, values and queries are
# N(0,1) rounded to bfloat16 (no grid), as the configs describe them.
WORKLOADS.update({
    "c2s_bf16": replace(WORKLOADS["c2s"], name="c2_small_offgrid", values="bf16"),
    "c3s_bf16": replace(WORKLOADS["c3s"], name="c3_small_thrash_offgrid", values="bf16"),
    "c5s_bf16": replace(WORKLOADS["c5s"], name="c5_small_prefill_offgrid", values="bf16"),
})

# Decode with one appended token per request per step (the new token's K/V
# stored with write-through before each layer's selection).
WORKLOADS.update({
    "c3a": replace(WORKLOADS["c3"], name="c3_196k_thrash_append", append=True, steps=48),
    "c3sa": replace(WORKLOADS["c3s"], name="c3_small_thrash_append", append=True),
    "c4sa": replace(WORKLOADS["c4s"], name="c4_small_mixed_append", append=True, steps=6),
})


def get_workload(key: str) -> Workload:
    return WORKLOADS[key]
