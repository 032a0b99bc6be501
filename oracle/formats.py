"""Number formats used by the oracle: decode to float64 and round-to-nearest-even.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the package's ``smoke()`` check and the benchmark's CPU-baseline leg do.

Formats handled (all binary floating point with an implicit leading 1):

=========  =====  ======  ==================  ==========================
name       sig p  emin    max finite          overflow
=========  =====  ======  ==================  ==========================
f16        11     -14     65504               +-inf (IEEE binary16)
bf16        8     -126    (2 - 2**-7)*2**127   +-inf
e4m3fn      4     -6      448                 saturates to +-448 (OCP
                                              "FN": no inf, 0x7f/0xff NaN)
=========  =====  ======  ==================  ==========================

``round_to_format`` is written from the definition of round-to-nearest,
ties-to-even: in the binade [2**e, 2**(e+1)) the representable values are
spaced 2**(e - p + 1); below the smallest normal the spacing is fixed at
2**(emin - p + 1).  Scaling by that spacing is exact in float64, ``np.rint``
rounds half to even, and scaling back is exact.
"""
from __future__ import annotations

import numpy as np

FORMATS = {
    "f16": dict(p=11, emin=-14, maxfinite=65504.0, saturate=False),
    "bf16": dict(p=8, emin=-126, maxfinite=float((2 - 2 ** -7) * 2.0 ** 127), saturate=False),
    "e4m3fn": dict(p=4, emin=-6, maxfinite=448.0, saturate=True),
}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    Returns float64 holding exactly representable values of ``fmt`` (or +-inf
    on overflow for the IEEE formats; saturated for e4m3fn).  NaN stays NaN.
    """
    f = FORMATS[fmt]
    p, emin = f["p"], f["emin"]
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite_nz = np.isfinite(ax) & (ax > 0)
    safe = np.where(finite_nz, ax, 1.0)
    # frexp: safe = m * 2**ex with m in [0.5, 1)  ->  binade [2**(ex-1), 2**ex)
    _, ex = np.frexp(safe)
    e = ex.astype(np.int64) - 1                      # 2**e <= ax < 2**(e+1)
    q = np.maximum(e - (p - 1), emin - (p - 1))      # log2 of the spacing
    spacing = np.ldexp(1.0, q)
    r = np.rint(safe / spacing) * spacing            # exact scaling, RNE
    r = np.where(finite_nz, r, ax)
    if f["saturate"]:
        r = np.where(np.isfinite(r), np.minimum(r, f["maxfinite"]), r)
    else:
        r = np.where(r > f["maxfinite"], np.inf, r)
    return np.copysign(r, x)


# ---------------------------------------------------------------------------
# Bit-level decode / encode.
# ---------------------------------------------------------------------------

def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_values_to_bits(v) -> np.ndarray:
    """Encode values that are already exactly representable in binary16."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_values_to_bits(v) -> np.ndarray:
    """Encode values already exactly representable in bfloat16."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def e4m3fn_bits_to_f64(bits) -> np.ndarray:
    """Decode OCP e4m3fn codes: bias 7, 3 mantissa bits, subnormals m*2**-9."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    E = (b >> 3) & 0xF
    mant = b & 0x7
    val = np.where(E == 0, mant * 2.0 ** -9, (1.0 + mant / 8.0) * np.ldexp(1.0, E - 7))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3fn_values_to_bits(v) -> np.ndarray:
    """Encode values already exactly representable in e4m3fn (finite)."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.int64) << 7
    av = np.abs(v)
    safe = np.where(av > 0, av, 1.0)
    _, ex = np.frexp(safe)
    e = ex.astype(np.int64) - 1
    normal = (av >= 2.0 ** -6)
    E = np.where(normal, e + 7, 0)
    mant = np.where(normal, (safe / np.ldexp(1.0, e) - 1.0) * 8.0, av / 2.0 ** -9)
    mant = np.rint(mant).astype(np.int64)
    code = np.where(av > 0, (E << 3) | mant, 0)
    return (sign | code).astype(np.uint8)


def decode(bits, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return f16_bits_to_f64(bits)
    if fmt == "bf16":
        return bf16_bits_to_f64(bits)
    if fmt == "e4m3fn":
        return e4m3fn_bits_to_f64(bits)
    if fmt == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(fmt)


def round_and_encode(x, fmt: str) -> np.ndarray:
    """float64 -> bits of ``fmt`` with a single round-to-nearest-even."""
    r = round_to_format(x, fmt)
    if fmt == "f16":
        return f16_values_to_bits(r)
    if fmt == "bf16":
        return bf16_values_to_bits(r)
    if fmt == "e4m3fn":
        return e4m3fn_values_to_bits(r)
    raise ValueError(fmt)
