"""The GPU's fp32 -> e4m3 encoder (OCP E4M3FN: nearest, ties to even,
saturating at 448, sign kept on zero; FreeToken PR #525 commit summary:
the mirror takes e4m3 codes read after quantisation) against the oracle's
on every one of the 2^32 fp32 bit patterns, in chunks of 2^24.  NaN inputs
must give a NaN code (low seven bits set); every other input the oracle's
code exactly.  The oracle's side runs in spawned CPU worker processes (they
never touch the GPU); the GPU encodes each chunk in one launch."""
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

from tests.gpu_compare import say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24


def _oracle_chunk(i: int) -> bytes:
    from oracle.codecs import e4m3_encode
    x = (np.arange(CHUNK, dtype=np.uint64) + np.uint64(i) * np.uint64(CHUNK)).astype(np.uint32).view(np.float32)
    return e4m3_encode(x).tobytes()


def test_e4m3_encoder_exhaustive():
    from workload import get_workload
    from workload.gpu_run import GpuWorkload
    g = GpuWorkload(get_workload("c1"))
    n_chunks = (1 << 32) // CHUNK
    workers = max(1, min(16, (os.cpu_count() or 1)))
    say(f"[codec] exhaustive e4m3 encode: {n_chunks} chunks of 2^24, {workers} CPU workers")
    base = torch.arange(CHUNK, dtype=torch.int32, device="cuda")
    bad_total = 0
    examples = []
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        for i, ref_bytes in enumerate(pool.imap(_oracle_chunk, range(n_chunks), chunksize=1)):
            off = i * CHUNK - (1 << 32 if i * CHUNK >= 1 << 31 else 0)   # the chunk's first pattern as int32
            bits = base + off
            got = g.tier.e4m3_encode(bits.view(torch.float32)).cpu().numpy()
            ref = np.frombuffer(ref_bytes, dtype=np.uint8)
            nan = (ref & 0x7F) == 0x7F           # the oracle gives a NaN code only for NaN inputs
            ok = np.where(nan, (got & 0x7F) == 0x7F, got == ref)
            bad = np.nonzero(~ok)[0]
            bad_total += bad.size
            if bad.size and len(examples) < 5:
                examples += [(hex(i * CHUNK + int(j)), int(got[j]), int(ref[j])) for j in bad[:5]]
            if i % 64 == 63:
                say(f"[codec] {i + 1}/{n_chunks} chunks, {bad_total} mismatches")
    assert bad_total == 0, f"{bad_total} mismatches, e.g. (pattern, gpu, oracle) {examples}"
