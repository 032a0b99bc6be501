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


def test_fp8_partials_bound_separates_rounding_from_wrong_pairing():
    """The fp8 partials bound admits the exact sum's rounding but not a
    partial formed with the activations paired with the wrong k."""
    import workloads
    from oracle import w4_oracle as O
    from tests.parity import bits16, fp8_partials_bound
    wl = workloads.WORKLOADS["w4a8_fp8_g128_28672x8192"]
    c = workloads.make_case(wl, 6, N=32, K=256, seed_base=4)
    codes, _ = O.quant_act_per_token(bits16(c.a), "bf16", "fp8")
    exact = O.w4a8_group_partials(codes, "fp8", c.w_logical.numpy(), 256, "int4", 128) * 2.0 ** -9
    bound = fp8_partials_bound(codes, c.w_logical.numpy(), 256)
    assert np.all(bound >= 128 * 2.0 ** -24 * np.abs(exact))
    # rounding the exact sums to fp32 stays inside
    assert np.all(np.abs(exact.astype(np.float32).astype(np.float64) - exact) <= bound)
    # activations shifted by one k inside each group: far outside
    shifted = np.concatenate([np.roll(codes[:, g * 128:(g + 1) * 128], 1, axis=1) for g in range(2)], axis=1)
    wrong = O.w4a8_group_partials(shifted, "fp8", c.w_logical.numpy(), 256, "int4", 128) * 2.0 ** -9
    assert np.mean(np.abs(wrong - exact) > bound) > 0.9
