"""CPU checks of the W4A8 acceptance rule the GPU parity tests apply.

fp16 outputs must meet |d| <= 2e-3 |ref| + 1e-3 alone; bf16 outputs may also
pass as a correct rounding of a value within the fp32 evaluation bound of the
exact result (bf16's half-ulp exceeds 2e-3 relative).
"""
import numpy as np

from oracle import formats as F
from tests.parity import w4a8_accept


def _ref(exact, mag, dtype):
    exact = np.asarray(exact, dtype=np.float64)
    return dict(out=F.round_and_encode(exact, dtype), exact=exact, mag=np.asarray(mag, dtype=np.float64))


def test_fp16_outputs_need_the_stated_tolerance():
    # near zero with a large magnitude: the rounding-bound clause would admit
    # ~1.3e-3, the stated tolerance only 1e-3
    ref = _ref([[0.0, 0.0]], [[1000.0, 1000.0]], "f16")
    got = F.round_and_encode(np.array([[1.2e-3, 0.9e-3]]), "f16")
    ok, st = w4a8_accept(got, ref, "f16", "i8", G=170)
    assert not ok[0, 0] and ok[0, 1]
    ok_strict, _ = w4a8_accept(got, ref, "f16", "i8", G=170, strict=True)
    assert not ok_strict[0, 0]


def test_bf16_outputs_may_be_a_rounding_within_the_bound():
    x = 1.0 + 3 * 2.0 ** -9            # between two bf16 values (spacing 2**-7)
    ref = _ref([[x]], [[2.0 ** 8]], "bf16")
    # the neighbour one bf16 ulp away is outside 2e-3 * |ref| + 1e-3 but a
    # correct rounding of a value within the bound
    other = F.round_and_encode(np.array([[1.0 + 2.0 ** -7]]), "bf16")
    if np.array_equal(other, ref["out"]):
        other = F.round_and_encode(np.array([[1.0]]), "bf16")
    ok, _ = w4a8_accept(other, ref, "bf16", "fp8", G=64)
    assert ok.all()
    far = F.round_and_encode(np.array([[1.1]]), "bf16")
    ok, _ = w4a8_accept(far, ref, "bf16", "fp8", G=64)
    assert not ok.any()
