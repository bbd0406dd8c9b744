"""GPU side of the seeded input generator (see ``gen.py`` for the definition).

``libtkvgen.so`` runs Philox4x64-10 on the device so that gigabytes of
synthetic context need no host generation or upload; ``gen.py`` produces the
same values on the host (NumPy's own Philox), which is what the oracle uses.
"""
from __future__ import annotations

import ctypes as C
import os
import shutil
import subprocess

import numpy as np
import torch

from . import gen
from .configs import Workload

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtkvgen.so")
_lib = None
_tables = {}


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "csrc", "gen.hip"), "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for gen.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} missing: build with workload.gpu_gen.build()")
        _lib = C.CDLL(LIB)
        _lib.tkvgen_tokens.restype = C.c_int
        _lib.tkvgen_tokens.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_uint64, C.c_int, C.c_int,
                                       C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p]
    return _lib


def _table(kind: int, values: str, device) -> torch.Tensor:
    key = (kind == gen.KIND_Q, values, str(device))
    if key not in _tables:
        if values == "bf16":
            t = gen.bf16_table().view(np.int16)
        else:
            t = gen.q_table() if kind == gen.KIND_Q else gen.kv_table()
        _tables[key] = torch.from_numpy(t.copy()).to(device)
    return _tables[key]


def tokens(wl: Workload, kind: int, layer: int, req: int, start: int, count: int, out=None,
           stream=None) -> torch.Tensor:
    """bf16 [count][H][d] on the GPU: keys/values (H = Hkv, 64-token... page blocks)
    or prefill queries (kind 2: H = Hq, 64-token blocks, positions relative to the chunk)."""
    if kind == gen.KIND_Q:
        H, bt, e = wl.num_q_heads, 64, gen.Q_EXP
    else:
        H, bt, e = wl.num_kv_heads, wl.page_size, gen.KV_EXP
    D = wl.head_dim
    if out is None:
        out = torch.empty((count, H, D), dtype=torch.bfloat16, device="cuda")
    tab = _table(kind, wl.values, out.device)
    if wl.values == "bf16":
        e = -1                                   # the table holds bf16 bit patterns
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _load().tkvgen_tokens(out.data_ptr(), tab.data_ptr(), e, wl.seed, kind, layer, req, start,
                               count, bt, H * D, s)
    if rc != 0:
        raise RuntimeError(f"tkvgen_tokens failed ({rc})")
    return out
