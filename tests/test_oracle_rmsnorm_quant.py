"""Pins for the oracle's fused RMSNorm + dynamic per-token quantisation (CPU).

* Exact rationals: the normalised values are re-derived with integer
  arithmetic (exact sum of squares, correctly rounded fp64 division, square
  root and reciprocal from an integer square root, fp32 products, rounding to
  the activation dtype) and must match bit for bit.
* A row whose mean square plus eps is exactly 1 has r = 1: the operation then
  reduces to plain per-token quantisation of x * gamma, which pins the mean
  over K, eps inside the square root, the gamma product and the composition
  with the quantiser.
* The normalised values agree with torch's ``rms_norm`` in float64 within the
  rounding of the activation dtype, with eps large enough that a misplaced eps
  or a K - 1 divisor would show.
* Power-of-two scaling of x leaves codes and scales unchanged; a zero row gives
  scale 0 and codes 0; a row with one nonzero element maps it to +-qmax.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import w4_oracle as O
from tests import exact as X
from tests.test_oracle_quant import _exact_quant_row

TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
TO_FRAC = {"f16": X.f16_bits_to_fraction, "bf16": X.bf16_bits_to_fraction}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _frac_to_bits(q: Fraction, dtype: str) -> int:
    if dtype == "f16":
        return X.fraction_to_f16_bits(q)
    return X.fraction_to_f32_bits(q) >> 16          # q is already a bf16 value


def _exact_normalised_row(xrow_bits, grow_bits, dtype, eps):
    """(r, fp32 values, dtype bits) of one row, from exact rationals."""
    xs = [TO_FRAC[dtype](int(b)) for b in xrow_bits]
    gs = [TO_FRAC[dtype](int(b)) for b in grow_bits]
    K = len(xs)
    ss = X.round_fraction(sum(v * v for v in xs), "f64")
    var = X.round_fraction(X.round_fraction(ss / K, "f64") + Fraction(float(np.float32(eps))), "f64")
    inv = X.round_fraction(1 / X.sqrt_rounded(var, "f64"), "f64")
    r = X.round_fraction(inv, "f32")
    ys, bits = [], []
    for v, g in zip(xs, gs):
        y = X.round_fraction(X.round_fraction(v * r, "f32") * g, "f32")
        ys.append(y)
        bits.append(_frac_to_bits(X.round_fraction(y, dtype), dtype))
    return r, ys, bits


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_normalised_values_match_exact_rationals(dtype, eps):
    g = torch.Generator().manual_seed(11)
    x = (torch.randn((4, 40), generator=g) * torch.tensor([1.0, 3e-3, 50.0, 1.0])[:, None]).to(TORCH[dtype])
    gamma = (torch.rand((40,), generator=g) * 1.5 + 0.25).to(TORCH[dtype])
    r, y32 = O.rmsnorm_rows(_bits(x), dtype, _bits(gamma), eps)
    codes, scales, y = O.rmsnorm_quant_per_token(_bits(x), dtype, _bits(gamma), eps, "i8")
    for m in range(x.shape[0]):
        re, ye, be = _exact_normalised_row(_bits(x)[m], _bits(gamma), dtype, eps)
        assert Fraction(float(r[m])) == re, m
        assert [Fraction(float(v)) for v in y32[m]] == ye, m
        assert list(y[m]) == be, m
        # the codes quantise the values rounded to the activation dtype
        s_exp, c_exp = _exact_quant_row([TO_FRAC[dtype](b) for b in be], "i8")
        assert Fraction(float(scales[m])) == s_exp and list(codes[m]) == c_exp, m


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_unit_mean_square_reduces_to_plain_quantisation(dtype, q_dtype):
    # 1023 entries of +-1 and one 0: ss / K + eps = 1023/1024 + 1/1024 = 1
    K = 1024
    g = torch.Generator().manual_seed(5)
    sign = torch.where(torch.rand((2, K), generator=g) < 0.5, -1.0, 1.0)
    sign[0, 17] = 0.0
    sign[1, 1000] = 0.0
    x = sign.to(TORCH[dtype])
    gamma = (torch.rand((K,), generator=g) * 1.5 + 0.25).to(TORCH[dtype])
    codes, scales, y = O.rmsnorm_quant_per_token(_bits(x), dtype, _bits(gamma), 2.0 ** -10, q_dtype)
    xg = (sign * gamma.float()).to(TORCH[dtype])        # exact: +-gamma or 0
    assert np.array_equal(y, _bits(xg))
    c2, s2 = O.quant_act_per_token(_bits(xg), dtype, q_dtype)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)


@pytest.mark.parametrize("dtype,rtol", [("f16", 2.0 ** -10), ("bf16", 2.0 ** -7)])
@pytest.mark.parametrize("eps", [1e-5, 0.5])
def test_normalised_values_match_torch_rms_norm(dtype, rtol, eps):
    g = torch.Generator().manual_seed(3)
    x = (torch.randn((6, 96), generator=g) * 0.7).to(TORCH[dtype])
    gamma = (torch.randn((96,), generator=g)).to(TORCH[dtype])
    _, _, y = O.rmsnorm_quant_per_token(_bits(x), dtype, _bits(gamma), eps, "i8")
    ref = torch.nn.functional.rms_norm(x.double(), (96,), weight=gamma.double(), eps=float(np.float32(eps)))
    got = torch.from_numpy(y.view(np.int16)).view(TORCH[dtype]).double()
    tiny = 2.0 ** -24 if dtype == "f16" else 2.0 ** -133
    assert torch.all((got - ref).abs() <= rtol * ref.abs() + tiny)


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_power_of_two_scaling_leaves_codes_unchanged(q_dtype):
    g = torch.Generator().manual_seed(9)
    x = torch.randn((5, 256), generator=g).to(torch.float16)
    gamma = (torch.rand((256,), generator=g) + 0.5).to(torch.float16)
    c1, s1, y1 = O.rmsnorm_quant_per_token(_bits(x), "f16", _bits(gamma), 1e-30, q_dtype)
    c2, s2, y2 = O.rmsnorm_quant_per_token(_bits(x * 8), "f16", _bits(gamma), 1e-30, q_dtype)
    assert np.array_equal(y1, y2) and np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("q_dtype,qmax", [("i8", 127), ("fp8", 448)])
def test_zero_row_and_single_nonzero_element(q_dtype, qmax):
    x = torch.zeros((2, 64), dtype=torch.float16)
    x[1, 9] = -3.0
    gamma = torch.full((64,), 1.5, dtype=torch.float16)
    codes, scales, y = O.rmsnorm_quant_per_token(_bits(x), "f16", _bits(gamma), 1e-6, q_dtype)
    assert scales[0] == 0 and not np.any(codes[0]) and not np.any(y[0])
    # y[1, 9] = -3 / sqrt(9 / 64 + 1e-6) * 1.5 ~= -12: the row maximum, so code -qmax
    y19 = float(torch.from_numpy(y[1:2, 9:10].view(np.int16)).view(torch.float16))
    assert abs(y19 + 12.0) < 0.01
    dec = O.activation_integers(codes, q_dtype).astype(np.float64) * O.ACT_UNIT[q_dtype]
    assert dec[1, 9] == -qmax and np.count_nonzero(dec[1]) == 1


def test_eps_must_be_positive():
    x = np.zeros((1, 8), np.uint16)
    with pytest.raises(ValueError):
        O.rmsnorm_quant_per_token(x, "f16", x[0], 0.0, "i8")
