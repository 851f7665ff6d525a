"""Exact-rational reference used to pin the oracle (tests only).

Every BF16 value and every dequantised weight (q - 8) * s is a dyadic
rational, so products and sums can be formed exactly with ``fractions``.
This file decodes the IEEE bit patterns and performs round-to-nearest-even
from those definitions, independently of the C oracle, so that it can catch
a mistake there.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

INF = object()  # marker for overflow results


def bf16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a finite BF16 bit pattern (sign, 8-bit exponent, 7-bit fraction)."""
    h = int(h) & 0xFFFF
    sign = -1 if h & 0x8000 else 1
    exp = (h >> 7) & 0xFF
    frac = h & 0x7F
    if exp == 0xFF:
        raise ValueError("not finite")
    if exp == 0:  # subnormal: 0.f * 2^-126
        return sign * Fraction(frac, 1 << 7) * Fraction(1, 1 << 126)
    val = Fraction(128 + frac, 128)
    e = exp - 127
    return sign * (val * (Fraction(1 << e) if e >= 0 else Fraction(1, 1 << -e)))


def f32_to_fraction(f) -> Fraction:
    return Fraction(float(np.float32(f)))


def _round_to_precision(v: Fraction, mant_bits: int, emin: int, emax: int):
    """Round |v| to a binary format with ``mant_bits`` significant bits, ties to even.

    Returns a Fraction, or INF on overflow.  Works from the definition: pick the
    binade 2^e <= |v| < 2^(e+1) (e clamped at emin for subnormals), the quantum is
    2^(e - mant_bits + 1), round |v| / quantum to an integer, ties to even.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # binade search
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits + 1)
    units = a / quantum
    fl = units.numerator // units.denominator
    rem = units - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return INF
    return sign * r


def round_bf16(v: Fraction):
    """Exact RNE of a rational to BF16 (8 significant bits, emin -126, emax 127)."""
    return _round_to_precision(v, 8, -126, 127)


def round_f32(v: Fraction):
    """Exact RNE of a rational to binary32 (24 significant bits)."""
    return _round_to_precision(v, 24, -126, 127)


def fraction_to_bf16_bits(v) -> int:
    """Bit pattern of a value already representable in BF16 (or INF marker)."""
    if v is INF:
        raise ValueError("overflow")
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < -126:  # subnormal
        frac = a / Fraction(2) ** (-133)
        assert frac.denominator == 1
        return sign | int(frac)
    mant = a / Fraction(2) ** (e - 7)
    assert mant.denominator == 1 and 128 <= mant < 256
    return sign | ((e + 127) << 7) | (int(mant) - 128)


def dequant_exact(code: int, scale_bits: int) -> Fraction:
    return ((int(code) & 0xF) - 8) * bf16_bits_to_fraction(scale_bits)


def gemm_exact(A_bits, a_row_div, codes, scales, topk_ids, route: int, n: int) -> Fraction:
    """sum_k A[route // a_row_div, k] * (q[e,n,k] - 8) * s[e,n,k//32], exactly."""
    e = int(np.asarray(topk_ids).reshape(-1)[route])
    K = codes.shape[2]
    row = A_bits[route // a_row_div]
    total = Fraction(0)
    for k in range(K):
        total += bf16_bits_to_fraction(row[k]) * dequant_exact(codes[e, n, k], scales[e, n, k // 32])
    return total


def binary_span_bits(values) -> int:
    """Bits from the leading bit of the largest |partial sum or term| down to the last bit of the
    finest term; if it is <= 53 a binary64 running sum of the terms is exact."""
    vals = [v for v in values if v != 0]
    if not vals:
        return 0
    partial = Fraction(0)
    biggest = max(abs(v) for v in vals)
    for v in vals:
        partial += v
        biggest = max(biggest, abs(partial))
    hi = biggest.numerator.bit_length() - biggest.denominator.bit_length() + 1
    lo = min(-(v.denominator.bit_length() - 1) for v in vals)  # denominators are powers of two
    return hi - lo
