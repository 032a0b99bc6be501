"""Pins for the oracle's dynamic per-token quantisation (CPU only).

The expected codes are re-derived with exact rationals (fp32 division rounded
by ``tests/exact.py``), cross-checked against torch's CPU ``round`` (half to
even) and ``float8_e4m3fn`` cast, an exhaustive nearest-code search, and
closed-form properties (error bound, amax maps to +-qmax, power-of-two
scale invariance, zero rows).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import w4_oracle as O
from tests import exact as X


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16)


def _exact_quant_row(xrow, q_dtype):
    qmax = 127 if q_dtype == "i8" else 448
    amax = max(abs(v) for v in xrow)
    s = X.round_fraction(amax / qmax, "f32")
    codes = []
    for v in xrow:
        if s == 0:
            codes.append(0)
            continue
        qv = X.round_fraction(v / s, "f32")
        if q_dtype == "i8":
            fl = qv.numerator // qv.denominator
            rem = qv - fl
            n = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            codes.append(max(-127, min(127, n)))
        else:
            qv = max(Fraction(-448), min(Fraction(448), qv))
            codes.append(X.nearest_e4m3fn_bruteforce(qv))
    return s, codes


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
@pytest.mark.parametrize("dist", ["normal", "wide"])
def test_quant_matches_exact_rationals(x_dtype, q_dtype, dist):
    x = workloads.activations(6, 160, x_dtype, seed=17, dist=dist)
    xb = _bits(x)
    q, s = O.quant_act_per_token(xb, x_dtype, q_dtype)
    dec = X.f16_bits_to_fraction if x_dtype == "f16" else X.bf16_bits_to_fraction
    for m in range(x.shape[0]):
        row = [dec(int(b)) for b in xb[m]]
        s_exp, codes = _exact_quant_row(row, q_dtype)
        assert Fraction(float(s[m])) == s_exp
        got = q[m].astype(np.int64) if q_dtype == "i8" else q[m].astype(np.int64)
        if q_dtype == "i8":
            assert got.tolist() == codes
        else:
            # +0 / -0: both encodings of zero are zero; compare values for 0x00/0x80
            g = [0 if c in (0, 0x80) else c for c in got.tolist()]
            e = [0 if c in (0, 0x80) else c for c in codes]
            assert g == e


def test_int8_quant_matches_torch_round():
    x = workloads.activations(64, 4096, "f16", seed=3)
    q, s = O.quant_act_per_token(_bits(x), "f16", "i8")
    xs = x.float()
    amax = xs.abs().amax(dim=1)
    st = amax / 127.0
    assert np.array_equal(st.numpy(), s)
    qt = torch.round(xs / st[:, None]).clamp(-127, 127).to(torch.int8)
    assert np.array_equal(qt.numpy(), q)


def test_fp8_quant_matches_torch_cast():
    x = workloads.activations(64, 2048, "bf16", seed=4)
    q, s = O.quant_act_per_token(_bits(x), "bf16", "fp8")
    xs = x.float()
    st = xs.abs().amax(dim=1) / 448.0
    assert np.array_equal(st.numpy(), s)
    v = (xs / st[:, None]).clamp(-448, 448)
    qt = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(qt, q)


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_quant_properties(q_dtype):
    x = workloads.activations(32, 1024, "f16", seed=8)
    xb = _bits(x)
    q, s = O.quant_act_per_token(xb, "f16", q_dtype)
    xv = x.double().numpy()
    qmax = 127 if q_dtype == "i8" else 448
    deq = (q.astype(np.float64) if q_dtype == "i8"
           else O.activation_integers(q, "fp8") / 512.0) * s[:, None].astype(np.float64)
    amax_idx = np.abs(xv).argmax(axis=1)
    for m in range(xv.shape[0]):
        val = deq[m, amax_idx[m]] / s[m]
        assert abs(val) == qmax
        if q_dtype == "i8":
            # rounding error at most half a step (plus the fp32 quotient's rounding)
            assert np.all(np.abs(xv[m] - deq[m]) <= 0.5 * s[m] * (1 + 2 ** -20))
        else:
            # relative error of e4m3: at most 2**-4 of the value, or half the
            # subnormal step 2**-10 (in units of s)
            err = np.abs(xv[m] - deq[m])
            assert np.all(err <= np.maximum(np.abs(xv[m]) * 2.0 ** -4, 2.0 ** -10 * s[m]) * (1 + 2 ** -20))


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_quant_power_of_two_invariance(q_dtype):
    x = workloads.activations(8, 512, "f16", seed=9)
    q1, s1 = O.quant_act_per_token(_bits(x), "f16", q_dtype)
    x4 = (x.float() * 4).to(torch.float16)
    assert torch.equal(x4.float(), x.float() * 4)       # exact scaling
    q2, s2 = O.quant_act_per_token(_bits(x4), "f16", q_dtype)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1 * 4, s2)


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_quant_zero_row_and_single_element(q_dtype):
    x = workloads.activations(3, 256, "f16", seed=2)
    x[1] = 0
    x[2] = 0
    x[2, 77] = -3.0
    q, s = O.quant_act_per_token(_bits(x), "f16", q_dtype)
    assert s[1] == 0 and np.all(q[1] == 0)
    assert s[2] == np.float32(3.0) / np.float32(127 if q_dtype == "i8" else 448)
    if q_dtype == "i8":
        assert q[2, 77] == -127 and np.count_nonzero(q[2]) == 1
    else:
        assert q[2, 77] == 0xFE and np.count_nonzero(q[2]) == 1


def test_hand_worked_int8_example():
    # amax = 2 -> s = fp32(2/127) = 2113665 / 2**27.
    # 1.0 / s = 63.50000024 exactly; its fp32 rounding is the tie 63.5, which
    # rounds half to even -> 64.  0.5 / s -> 31.75 -> 32 ; 0.25 / s -> 15.875 -> 16.
    x = torch.tensor([[0.5, -1.0, 2.0, 0.25, 0.0, -2.0]], dtype=torch.float16)
    q, s = O.quant_act_per_token(_bits(x), "f16", "i8")
    assert Fraction(float(s[0])) == Fraction(2113665, 2 ** 27)
    assert q[0].tolist() == [32, -64, 127, 16, 0, -127]
