"""Writes quant_tokens.json: tokens whose fp8 bytes are fixed by the
quantiser's definition (FreeToken PR #525, commit summary: the mirror takes
the codes and scales produced by the quantiser; per-token scale as read in
the design notes):

    scale = fp32(amax / 448)           one correctly rounded division
    code  = e4m3(fp32(x / scale))      one correctly rounded division, then
                                       round to the nearest E4M3FN value,
                                       ties to the even code, saturating

Every value here is computed with exact rationals (``fractions.Fraction``)
and explicit round-to-nearest-even, from the IEEE binary32 and OCP E4M3FN
definitions -- nothing is imported from the oracle.  The script also records
what the reciprocal-multiply form (scale = amax * fp32(1/448), code =
e4m3(fp32(x * fp32(1/scale)))) would produce, so the test can show the tokens
separate the two.

Run:  python tests/golden/make_quant_golden.py
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def f32_bits(v: Fraction) -> int:
    """Round a rational to the nearest binary32 (ties to even); returns the bits."""
    if v == 0:
        return 0
    sign = 0x80000000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)); binary32 keeps 24 significant bits down to 2^-149
    q = max(e - 23, -149)
    m = a / Fraction(2) ** q
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** q
    return sign | struct.unpack("<I", struct.pack("<f", float(val)))[0]


def f32_val(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits))[0])


def bf16_val(bits16: int) -> Fraction:
    return f32_val(bits16 << 16)


def e4m3_table():
    """(value, code) of every finite non-negative OCP E4M3FN code: exponent
    bias 7, subnormals m * 2^-9, S.1111.111 is NaN."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((v, code))
    return out


E4M3 = e4m3_table()


def e4m3_code(v: Fraction, negative: bool) -> int:
    """Nearest E4M3FN value to |v| by exhaustive search, ties to the even
    code, magnitudes above 448 saturate to 448; ``negative`` is the sign bit
    of the quotient (kept on zero: a scale is positive, so it is x's)."""
    sign = 0x80 if negative else 0
    a = abs(v)
    if a >= 448:
        return sign | 0x7E
    best = min(E4M3, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return sign | best[1]


def quantize(xs_bits):
    xs = [bf16_val(b) for b in xs_bits]
    amax = max(abs(x) for x in xs)
    scale_bits = 0x3F800000 if amax == 0 else f32_bits(amax / 448)
    scale = f32_val(scale_bits)
    codes = [e4m3_code(f32_val(f32_bits(x / scale)), b >> 15 == 1) for x, b in zip(xs, xs_bits)]
    return scale_bits, codes


def quantize_reciprocal(xs_bits):
    xs = [bf16_val(b) for b in xs_bits]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        scale_bits = 0x3F800000
    else:
        r448 = f32_val(f32_bits(Fraction(1, 448)))
        scale_bits = f32_bits(amax * r448)
    scale = f32_val(scale_bits)
    inv = f32_val(f32_bits(1 / scale))
    codes = [e4m3_code(f32_val(f32_bits(x * inv)), b >> 15 == 1) for x, b in zip(xs, xs_bits)]
    return scale_bits, codes


def bf16_bits(x: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, f"{x} is not a bf16 value"
    return b >> 16


# Tokens of 8 values (one KV head of 8 dims): the amax element, elements that
# land in the e4m3 subnormal range near a rounding midpoint, ordinary values.
TOKENS = [
    # amax 0.5390625: fp32(amax/448) and amax*fp32(1/448) differ by one ulp
    [0.5390625, 8.225440979003906e-06, 2.467632293701172e-05, -4.935264587402344e-05,
     9.870529174804688e-05, -0.25, 0.0, 0.125],
    # amax 0.7109375 (negative): same, other midpoints
    [-0.7109375, 4.649162292480469e-06, 1.0848045349121094e-05, 1.704692840576172e-05,
     2.014636993408203e-05, 0.5, -0.0, 0.001953125],
    # amax 0.765625
    [0.765625, -5.0067901611328125e-06, 1.1682510375976562e-05, 2.1696090698242188e-05,
     4.172325134277344e-05, 4.839897155761719e-05, 0.375, -0.09375],
    # an all-zero token: scale 1, codes 0 (and -0 keeps its sign)
    [0.0, -0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
    # amax 448 * 2^-3: the scale is exactly 2^-3 and every value below is exact
    [56.0, 1.0, -2.0, 0.5, 0.0625, 3.0, -56.0, 7.0],
]


def main():
    out = {"source": "FreeToken PR #525, commit summary (mirror_store_quant); per-token scale reading "
                     "scale = fp32(amax/448), code = e4m3(fp32(x/scale)), OCP E4M3FN, ties to even",
           "shape": [1, 8],
           "tokens": []}
    for t in TOKENS:
        xb = [bf16_bits(x) for x in t]
        sb, codes = quantize(xb)
        rsb, rcodes = quantize_reciprocal(xb)
        out["tokens"].append({
            "x_bf16_bits": [f"0x{b:04x}" for b in xb],
            "scale_f32_bits": f"0x{sb:08x}",
            "codes": [f"0x{c:02x}" for c in codes],
            "reciprocal_form_scale_f32_bits": f"0x{rsb:08x}",
            "reciprocal_form_codes": [f"0x{c:02x}" for c in rcodes],
        })
    path = os.path.join(HERE, "quant_tokens.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
