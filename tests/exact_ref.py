"""Exact pure-Python references used to pin the oracle (test helpers only).

Nothing here is shared with the oracle or the library: it restates the
definitions with Python integers and ``fractions.Fraction`` so that a mistake in
either C implementation shows up as a mismatch.  Slow by design; used on small
inputs only.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# The 127 non-negative finite E4M3FN values, built from "sign, 4-bit exponent
# with bias 7, 3-bit fraction; exponent field 0 is subnormal" (OCP OFP8).
E4M3_POS = []
for _e in range(16):
    for _f in range(8):
        if _e == 15 and _f == 7:
            continue
        if _e == 0:
            E4M3_POS.append((_e * 8 + _f, Fraction(_f, 8) * Fraction(1, 2 ** 6)))
        else:
            E4M3_POS.append((_e * 8 + _f, (1 + Fraction(_f, 8)) * Fraction(2) ** (_e - 7)))
assert len(E4M3_POS) == 127 and E4M3_POS[-1] == (0x7E, Fraction(448))


def nearest_e4m3(v: Fraction, negative: bool = False) -> int:
    """Code nearest to |v| by exhaustive search over all 127 values; ties to even; saturating."""
    a = abs(v)
    sign = 0x80 if negative else 0x00
    if a > 448:
        return sign | 0x7E
    best = None
    for code, val in E4M3_POS:
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return sign | best[1]


def f32_round(fr: Fraction) -> float:
    """Round an exact rational to the nearest fp32 (ties to even), subnormals included."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # below 2^-126: subnormal grid, spacing 2^-149
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        val = math.inf
    out = float(val) if val != math.inf else math.inf
    # confirm it is an fp32 value
    assert out == struct.unpack("<f", struct.pack("<f", out))[0]
    return -out if neg else out


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def quantize_exact(values, amax=None):
    """Scale and codes of one group, with exact arithmetic.

    s = fp32(amax / 448); each code = nearest_e4m3(fp32(x / s)); s == 0 gives
    signed zero codes.
    """
    if amax is None:
        amax = max(abs(v) for v in values)
    s = f32_round(Fraction(amax) / 448)
    codes = []
    for x in values:
        neg = math.copysign(1.0, x) < 0
        if s == 0.0 or x == 0.0:   # signed zero (Fraction drops the sign of -0.0)
            codes.append(0x80 if neg else 0x00)
            continue
        r = f32_round(Fraction(x) / Fraction(s))
        codes.append(nearest_e4m3(Fraction(r), negative=math.copysign(1.0, r) < 0))
    return s, codes


def decode_exact(code: int) -> Fraction:
    for c, v in E4M3_POS:
        if c == (code & 0x7F):
            return -v if code & 0x80 else v
    raise ValueError("NaN code")


def best_pair(scores):
    """Kept pair of a group of 4 by brute force over the 6 pairs: the largest score
    sum; among pairs with the same sum and the same sorted score multiset the
    lexicographically smallest.  Equivalent to "stable top-2" (ties -> lower index).
    """
    best = None
    for i in range(4):
        for j in range(i + 1, 4):
            # a pair is admissible only if every dropped score is <= every kept score
            dropped = [scores[k] for k in range(4) if k not in (i, j)]
            if max(dropped) > min(scores[i], scores[j]):
                continue
            key = (i, j)
            if best is None or key < best:
                best = key
    return best
