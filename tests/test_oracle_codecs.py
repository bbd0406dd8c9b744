"""Pins for the oracle's number formats (bfloat16 and OCP E4M3FN).

The oracle encodes by nearest-value search over its code table; these tests
pin it to (a) the OFP8 specification's defining values, (b) PyTorch's own
float8_e4m3fn and bfloat16 casts (library routines, round-to-nearest-even),
and (c) a brute-force argmin over every code with the ties-to-even rule.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle.codecs import (bf16_bits_from_f32, bf16_bits_to_f32, e4m3_decode,
                           e4m3_encode)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_values.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        out.append((int(c, 16), float(v)))
    return out


def test_e4m3_decode_matches_spec_points():
    for code, val in _golden():
        got = float(e4m3_decode(np.array([code], dtype=np.uint8))[0])
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


_ALL_VALUES = None


def _brute(x: float) -> int:
    """argmin over all finite codes of |x - value|, ties -> even code, then saturation."""
    global _ALL_VALUES
    if _ALL_VALUES is None:
        _ALL_VALUES = [float(v) for v in e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
    if math.isnan(x):
        return 0x7F | (0x80 if math.copysign(1, x) < 0 else 0)
    sign = 0x80 if math.copysign(1, x) < 0 else 0
    a = abs(x)
    if a >= 448.0:
        return 0x7E | sign
    best, bd = None, None
    for c in range(0x7F):
        d = abs(a - _ALL_VALUES[c])
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | sign


def _midpoints():
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    return np.concatenate([mids32, up, dn])


def test_e4m3_encode_brute_force_on_midpoints_and_random():
    rng = np.random.default_rng(5)
    xs = np.concatenate([_midpoints(), -_midpoints(),
                         rng.standard_normal(3000).astype(np.float32) * 60,
                         (rng.standard_normal(500) * 1e-3).astype(np.float32),
                         np.array([0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e30, np.inf, -np.inf,
                                   np.nan, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11],
                                  dtype=np.float32)])
    got = e4m3_encode(xs)
    exp = np.array([_brute(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, exp)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(6)
    xs = np.concatenate([_midpoints(), -_midpoints(),
                         (rng.uniform(-448, 448, 200000)).astype(np.float32),
                         (rng.standard_normal(200000) * 0.02).astype(np.float32)])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(xs), ref)


def test_e4m3_saturates_and_keeps_signed_zero():
    xs = np.array([500.0, -1e9, np.inf, -np.inf, -0.0, -2.0 ** -12], dtype=np.float32)
    assert e4m3_encode(xs).tolist() == [0x7E, 0xFE, 0x7E, 0xFE, 0x80, 0x80]


def test_bf16_matches_torch():
    rng = np.random.default_rng(7)
    base = rng.standard_normal(100000).astype(np.float32) * 10
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    xs = np.concatenate([base, ties.view(np.float32),
                         np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40], dtype=np.float32)])
    xs = xs[np.isfinite(xs) | np.isinf(xs)]
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(xs), ref)


def test_bf16_nan_stays_nan():
    out = bf16_bits_to_f32(bf16_bits_from_f32(np.array([np.nan], dtype=np.float32)))
    assert np.isnan(out[0])


@pytest.mark.parametrize("x", [1.0, -2.5, 0.0078125, 448.0])
def test_bf16_exact_values_unchanged(x):
    assert float(bf16_bits_to_f32(bf16_bits_from_f32(np.array([x], dtype=np.float32)))[0]) == x
