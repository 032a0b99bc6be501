"""Pins for the oracle's dynamic per-tensor quantisation (CPU only).

* Exact rationals: the codes of every element are re-derived from the
  tensor's absolute maximum with exact fp32 rounding (tests/exact.py).
* A one-row tensor, and a tensor whose rows share one absolute maximum, have
  per-tensor codes equal to the per-token ones (the two definitions meet).
* Scaling the tensor by a power of two leaves the codes unchanged; an
  all-zero tensor has scale 0 and codes 0; the element holding the maximum
  maps to +-qmax; the scale is the same for every row.
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


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_per_tensor_matches_exact_rationals(dtype, q_dtype):
    g = torch.Generator().manual_seed(4)
    x = (torch.randn((5, 24), generator=g) * torch.tensor([1.0, 0.01, 30.0, 1.0, 0.5])[:, None]).to(TORCH[dtype])
    codes, scales = O.quant_act_per_tensor(_bits(x), dtype, q_dtype)
    vals = [[TO_FRAC[dtype](int(b)) for b in row] for row in _bits(x)]
    flat = [v for row in vals for v in row]
    # quantising all elements as one row gives the per-tensor scale and codes
    s_exp, c_exp = _exact_quant_row(flat, q_dtype)
    assert all(Fraction(float(s)) == s_exp for s in scales)
    got = codes.astype(np.int64).ravel().tolist()
    if q_dtype == "fp8":
        # both encodings of zero (0x00, 0x80) are zero
        got = [0 if c in (0, 0x80) else c for c in got]
        c_exp = [0 if c in (0, 0x80) else c for c in c_exp]
    assert got == c_exp


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_per_tensor_meets_per_token(q_dtype):
    g = torch.Generator().manual_seed(6)
    x1 = torch.randn((1, 300), generator=g).to(torch.float16)
    a = O.quant_act_per_tensor(_bits(x1), "f16", q_dtype)
    b = O.quant_act_per_token(_bits(x1), "f16", q_dtype)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # rows with one shared maximum |x| = 3
    x = torch.randn((6, 128), generator=g).clamp(-2.5, 2.5)
    x[:, 7] = torch.tensor([3.0, -3.0, 3.0, 3.0, -3.0, 3.0])
    x = x.to(torch.float16)
    a = O.quant_act_per_tensor(_bits(x), "f16", q_dtype)
    b = O.quant_act_per_token(_bits(x), "f16", q_dtype)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("q_dtype,qmax", [("i8", 127), ("fp8", 448)])
def test_per_tensor_properties(q_dtype, qmax):
    g = torch.Generator().manual_seed(8)
    x = torch.randn((7, 64), generator=g).to(torch.float16)
    c1, s1 = O.quant_act_per_tensor(_bits(x), "f16", q_dtype)
    c2, s2 = O.quant_act_per_tensor(_bits(x * 4), "f16", q_dtype)
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * 4)
    assert np.all(s1 == s1[0])
    m, k = np.unravel_index(np.argmax(np.abs(x.float().numpy())), x.shape)
    dec = O.activation_integers(c1, q_dtype).astype(np.float64) * O.ACT_UNIT[q_dtype]
    assert abs(dec[m, k]) == qmax
    z, sz = O.quant_act_per_tensor(np.zeros((3, 16), np.uint16), "f16", q_dtype)
    assert not np.any(z) and not np.any(sz)
