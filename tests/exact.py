"""Exact-rational helpers for pinning the oracle.

These re-derive rounding from first principles with ``fractions.Fraction`` and
integer floor division, a different route from the oracle's float64
scaling + ``np.rint``.  They are only used by tests.
"""
from __future__ import annotations

import struct
from fractions import Fraction
from math import isqrt

# (significand bits p, minimum normal exponent, largest finite value)
FMT = {
    "f32": (24, -126, Fraction((2 ** 24 - 1) * 2 ** 104)),
    "f16": (11, -14, Fraction(65504)),
    "bf16": (8, -126, Fraction((2 ** 8 - 1) * 2 ** 120)),
    "e4m3fn": (4, -6, Fraction(448)),
    "f64": (53, -1022, Fraction((2 ** 53 - 1) * 2 ** 971)),
}


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(q: Fraction, fmt: str, saturate: bool = False):
    """Nearest value of ``fmt`` to the rational ``q``, ties to even.

    Returns a Fraction, or the string 'inf'/'-inf' on overflow (non-saturating).
    """
    p, emin, maxf = FMT[fmt]
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = _floor_log2(a)
    ulp_exp = max(e - (p - 1), emin - (p - 1))
    unit = Fraction(2) ** ulp_exp
    t = a / unit
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * unit
    if r > maxf:
        if saturate:
            r = maxf
        else:
            return "inf" if sign > 0 else "-inf"
    return sign * r


def f32_bits_to_fraction(u: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]
    return Fraction(f)


def fraction_to_f32_bits(q: Fraction) -> int:
    """q must already be an exactly representable fp32 value."""
    return struct.unpack("<I", struct.pack("<f", float(q)))[0]


def f16_bits_to_fraction(u: int) -> Fraction:
    return Fraction(struct.unpack("<e", struct.pack("<H", u & 0xFFFF))[0])


def fraction_to_f16_bits(q) -> int:
    if isinstance(q, str):
        return 0x7C00 if q == "inf" else 0xFC00
    return struct.unpack("<H", struct.pack("<e", float(q)))[0]


def bf16_bits_to_fraction(u: int) -> Fraction:
    return f32_bits_to_fraction((u & 0xFFFF) << 16)


def fraction_to_bf16_bits(q) -> int:
    if isinstance(q, str):
        return 0x7F80 if q == "inf" else 0xFF80
    b = fraction_to_f32_bits(q)
    assert b & 0xFFFF == 0
    return b >> 16


def e4m3fn_code_to_fraction(c: int) -> Fraction:
    """Decode by the OCP e4m3fn table: S.EEEE.MMM, bias 7, no infinities."""
    s = -1 if c & 0x80 else 1
    E = (c >> 3) & 0xF
    m = c & 7
    if E == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7)


def all_finite_e4m3fn():
    """(code, value) for every finite e4m3fn code (0x7f / 0xff are NaN)."""
    return [(c, e4m3fn_code_to_fraction(c)) for c in range(256) if (c & 0x7F) != 0x7F]


def nearest_e4m3fn_bruteforce(q: Fraction) -> int:
    """Nearest finite e4m3fn code by exhaustive search; ties go to the code
    with an even mantissa LSB; values beyond 448 saturate.  +0 for zero."""
    if q > 448:
        return 0x7E
    if q < -448:
        return 0xFE
    best = None
    for c, v in all_finite_e4m3fn():
        if c == 0x80:          # prefer +0 for an exact zero
            continue
        d = abs(v - q)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    # a negative input that rounds to zero keeps its sign
    if c == 0 and q < 0:
        c = 0x80
    return c


def sqrt_rounded(v: Fraction, fmt: str = "f64") -> Fraction:
    """Nearest ``fmt`` value to sqrt(v) for a rational v > 0, ties to even,
    from an integer square root (no floating point)."""
    p = FMT[fmt][0]
    # scale v by 4**j so that the integer square root carries p + 8 bits
    j = 0
    while v * Fraction(4) ** j < Fraction(2) ** (2 * (p + 8)):
        j += 1
    while v * Fraction(4) ** j >= Fraction(2) ** (2 * (p + 10)):
        j -= 1
    t = v * Fraction(4) ** j
    n = isqrt(t.numerator // t.denominator)
    exact = Fraction(n * n) == t
    # sqrt(v) = (n + f) / 2**j with 0 <= f < 1 (f = 0 iff exact); n has at
    # least p + 8 bits, so rounding n + f to p bits never sees a tie unless
    # f = 0, and then n decides it alone
    if exact:
        return round_fraction(Fraction(n, 2 ** j) if j >= 0 else Fraction(n * 2 ** -j), fmt)
    # inexact: round (n + 1/2) / 2**j; no p-bit tie can fall strictly inside
    # (n, n + 1), so the midpoint stands for the whole interval
    mid = Fraction(2 * n + 1, 2)
    return round_fraction(mid / Fraction(2) ** j, fmt)
