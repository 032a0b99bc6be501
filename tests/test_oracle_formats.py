"""Pins for the oracle's number formats (CPU only).

Every check compares ``oracle.formats`` with something other than itself:
exact-rational rounding (``tests/exact.py``), exhaustive nearest-value search,
numpy's binary16 conversion, torch's bfloat16 / float8_e4m3fn casts, and spot
values of the OCP 8-bit floating point specification.
"""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import exact as X


def _probe_values(fmt, n_random=4000, seed=0):
    """Random float64 values plus exact midpoints and their float64 neighbours."""
    rng = random.Random(seed)
    p, emin, maxf = X.FMT[fmt]
    vals = []
    for _ in range(n_random):
        e = rng.randint(emin - p - 2, int(np.log2(float(maxf))) + 1)
        vals.append(rng.choice((-1, 1)) * rng.random() * 2.0 ** e)
    # midpoints between neighbouring representable values, and +-1 ulp of them
    for _ in range(n_random // 4):
        e = rng.randint(emin - p + 1, int(np.log2(float(maxf))) - 1)
        unit = 2.0 ** (max(e - (p - 1), emin - (p - 1)))
        base = (rng.randint(2 ** (p - 1), 2 ** p - 1)) * unit if e >= emin else rng.randint(0, 2 ** (p - 1)) * unit
        mid = base + unit / 2
        for v in (mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)):
            vals.append(float(v) * rng.choice((-1, 1)))
    return np.array(vals, dtype=np.float64)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_round_to_format_matches_exact_rationals(fmt):
    vals = _probe_values(fmt)
    got = F.round_to_format(vals, fmt)
    for v, g in zip(vals, got):
        want = X.round_fraction(Fraction(float(v)), fmt)
        if isinstance(want, str):
            assert np.isinf(g) and (g > 0) == (want == "inf")
        else:
            assert Fraction(float(g)) == want, (fmt, v, g, want)


def test_e4m3fn_rounding_matches_exact_and_bruteforce():
    vals = _probe_values("e4m3fn", n_random=1500)
    vals = np.clip(vals, -600, 600)
    got = F.round_and_encode(vals, "e4m3fn")
    for v, c in zip(vals, got):
        q = Fraction(float(v))
        want = X.round_fraction(q, "e4m3fn", saturate=True)
        assert X.e4m3fn_code_to_fraction(int(c)) == want, (v, c, want)
        assert int(c) == X.nearest_e4m3fn_bruteforce(q), (v, c)


def test_f16_matches_numpy_conversion():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                           _probe_values("f16")])
    assert np.array_equal(F.round_and_encode(vals, "f16"), vals.astype(np.float16).view(np.uint16))


def test_bf16_matches_torch_cast_on_fp32_inputs():
    # torch converts fp32 -> bf16 with a single RNE; restrict to fp32 inputs
    rng = np.random.default_rng(2)
    v32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    t = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.round_and_encode(v32.astype(np.float64), "bf16"), t)


def test_e4m3fn_matches_torch_cast_in_range():
    rng = np.random.default_rng(3)
    v32 = (rng.uniform(-448, 448, 40000) * 2.0 ** rng.integers(-14, 1, 40000)).astype(np.float32)
    t = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.round_and_encode(v32.astype(np.float64), "e4m3fn"), t)


def test_e4m3fn_spot_values_from_ocp_spec():
    cases = {448.0: 0x7E, -448.0: 0xFE, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08, 1.0: 0x38,
             0.875 * 2.0 ** -6: 0x07, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             464.0: 0x7E, 1e9: 0x7E, -1e9: 0xFE, 240.0: 0x77, 0.0: 0x00}
    got = F.round_and_encode(np.array(list(cases)), "e4m3fn")
    assert [int(c) for c in got] == list(cases.values())


def test_decoders_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    dec = F.e4m3fn_bits_to_f64(codes)
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert np.isnan(dec[c])
        else:
            assert Fraction(float(dec[c])) == X.e4m3fn_code_to_fraction(c)
    b16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = F.f16_bits_to_f64(b16)
    bf = F.bf16_bits_to_f64(b16)
    for u in range(0, 65536, 97):
        if (u & 0x7C00) != 0x7C00:
            assert Fraction(float(h[u])) == X.f16_bits_to_fraction(u)
        if (u & 0x7F80) != 0x7F80:
            assert Fraction(float(bf[u])) == X.bf16_bits_to_fraction(u)


def test_encode_decode_roundtrip_all_finite_codes():
    b16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for fmt, dec in (("f16", F.f16_bits_to_f64), ("bf16", F.bf16_bits_to_f64)):
        v = dec(b16)
        fin = np.isfinite(v)
        back = F.round_and_encode(v[fin], fmt)
        assert np.array_equal(back, b16[fin]), fmt
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.round_and_encode(F.e4m3fn_bits_to_f64(codes), "e4m3fn"), codes)
