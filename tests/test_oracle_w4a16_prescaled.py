"""Pins for the oracle's W4A16 GEMM with pre-scaled zero-points (CPU only).

* Exact rationals on a small problem: out = RNE(sum_k a * (u * s - zs) + bias).
* Where z * s is exact in fp16 (scales with at most 7 significant bits,
  integer z), zs = z * s gives the raw zero-point GEMM's result bit for bit.
* zs = 0 gives the GEMM of u * s; doubling s and zs doubles the exact value.
"""

import numpy as np
import torch

from oracle import w4_oracle as O
from tests import exact as X


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _case(M, N, K, gs, seed, coarse=False):
    g = torch.Generator().manual_seed(seed)
    u = torch.randint(0, 16, (N, K), generator=g)
    wl = (u[:, 0::2] | (u[:, 1::2] << 4)).to(torch.uint8).numpy()
    G = K // gs
    if coarse:   # at most 7 significant bits: z * s is exact in fp16
        s = (torch.randint(64, 128, (N, G), generator=g).float() * 2.0 ** -12).to(torch.float16)
    else:
        s = (torch.rand((N, G), generator=g) * 0.015 + 0.005).to(torch.float16)
    z = torch.randint(0, 16, (N, G), generator=g)
    a = torch.randn((M, K), generator=g).to(torch.float16)
    bias = (torch.randn((N,), generator=g) * 0.1).to(torch.float16)
    return u.numpy(), wl, s, z, a, bias


def test_prescaled_matches_exact_rationals():
    M, N, K, gs = 2, 16, 256, 128
    u, wl, s, z, a, bias = _case(M, N, K, gs, seed=3)
    zs = (z.float() * s.float() * 1.37).to(torch.float16)     # any stored value
    r = O.w4a16_gemm_prescaled_zeros(_bits(a), "f16", wl, K, _bits(s), _bits(zs), gs, _bits(bias))
    A = [[X.f16_bits_to_fraction(int(b)) for b in row] for row in _bits(a)]
    S = [[X.f16_bits_to_fraction(int(b)) for b in row] for row in _bits(s)]
    ZS = [[X.f16_bits_to_fraction(int(b)) for b in row] for row in _bits(zs)]
    B = [X.f16_bits_to_fraction(int(b)) for b in _bits(bias)]
    for m in range(M):
        for n in range(N):
            v = sum(A[m][k] * (int(u[n, k]) * S[n][k // gs] - ZS[n][k // gs]) for k in range(K)) + B[n]
            assert int(r["out"][m, n]) == X.fraction_to_f16_bits(X.round_fraction(v, "f16")), (m, n)


def test_exact_products_reduce_to_raw_zero_points():
    M, N, K, gs = 3, 32, 512, 128
    u, wl, s, z, a, bias = _case(M, N, K, gs, seed=5, coarse=True)
    zs = (z.float() * s.float()).to(torch.float16)
    assert torch.equal(zs.float(), z.float() * s.float())       # exact
    r1 = O.w4a16_gemm_prescaled_zeros(_bits(a), "f16", wl, K, _bits(s), _bits(zs), gs, _bits(bias))
    r2 = O.w4a16_gemm(_bits(a), "f16", wl, K, "uint4", _bits(s), _bits(z.to(torch.float16)), gs, _bits(bias))
    assert np.array_equal(r1["out"], r2["out"])
    assert np.allclose(r1["exact"], r2["exact"], rtol=1e-13, atol=1e-13)


def test_zero_terms_and_scaling():
    M, N, K, gs = 2, 16, 256, 128
    u, wl, s, z, a, _ = _case(M, N, K, gs, seed=8, coarse=True)
    zero = torch.zeros_like(s)
    r0 = O.w4a16_gemm_prescaled_zeros(_bits(a), "f16", wl, K, _bits(s), _bits(zero), gs)
    r8 = O.w4a16_gemm(_bits(a), "f16", wl, K, "uint4", _bits(s), _bits(zero), gs)      # raw z = 0
    assert np.array_equal(r0["out"], r8["out"])
    zs = (z.float() * s.float() * 0.5).to(torch.float16)
    r1 = O.w4a16_gemm_prescaled_zeros(_bits(a), "f16", wl, K, _bits(s), _bits(zs), gs)
    r2 = O.w4a16_gemm_prescaled_zeros(_bits(a), "f16", wl, K, _bits(s * 2), _bits(zs * 2), gs)
    assert np.allclose(r2["exact"], 2 * r1["exact"], rtol=1e-13, atol=1e-13)
