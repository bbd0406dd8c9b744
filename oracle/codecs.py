"""Number formats: bfloat16 and OCP FP8 E4M3FN, from their definitions.

FreeToken PR #525's commit summary has the host mirror hold "e4m3 codes +
fp32 scales"; PR #499 ("Measured", Config A) runs with an fp8 KV cache.  The
pages do not name the e4m3 variant; this oracle takes OCP E4M3FN (the format
gfx950 converts natively): 1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits, subnormals down to 2^-9, largest finite value 448, no
infinities, NaN = S.1111.111.  Encoding rounds to the nearest representable
value with ties to the even code, saturates magnitudes >= 448 (infinities
included) to +-448, keeps the sign of zero, and maps NaN to the NaN code of
the same sign.

bfloat16 here is the upper half of an IEEE binary32, rounded to nearest with
ties to even.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ----------------------------------------------------------------- bfloat16 --
def bf16_bits_from_f32(x) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, 0x7FC0 | ((u >> 16) & 0x8000), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """binary32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits_from_f32(x))


# --------------------------------------------------------------- e4m3 (OCP) --
def _e4m3_code_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return s * (8 + m) * 2.0 ** (e - 10)  # normal: (1 + m/8) * 2^(e-7)


# all non-negative finite codes 0x00..0x7E and their values (ascending)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = np.array([_e4m3_code_value(int(c)) for c in _POS_CODES], dtype=np.float64)
assert np.all(np.diff(_POS_VALUES) > 0) and _POS_VALUES[-1] == E4M3_MAX


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float32 values (exact)."""
    table = np.array([_e4m3_code_value(c) for c in range(256)], dtype=np.float32)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> uint8 codes (nearest, ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    a = np.abs(flat.astype(np.float64))
    sign = np.signbit(flat).astype(np.int64) << 7
    # neighbours in the ascending value table
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a >= E4M3_MAX, 0x7E, code)          # saturate (inf included)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | sign).astype(np.uint8).reshape(x.shape)
