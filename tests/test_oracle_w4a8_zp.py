"""Pins for the oracle's asymmetric (zero-point) W4A8 GEMM (CPU only).

* Pure-Python brute force with exact rationals on small problems (grouped and
  per channel, int8 and fp8 activations, non-square so that a transposed
  zero-point table or a mis-grouped k fails): out = s_a * sum_g s_w *
  sum_k a * (u - z) + bias.
* Every zero-point 8 gives the symmetric uint4b8 result (the same bits).
* Adding 1 to every code and its group's zero-point leaves the result unchanged.
* A group whose codes all equal its zero-point contributes nothing.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import w4_oracle as O


def _case(M, N, K, gs, q_dtype, seed):
    g = torch.Generator().manual_seed(seed)
    u = torch.randint(0, 16, (N, K), generator=g)
    wl = (u[:, 0::2] | (u[:, 1::2] << 4)).to(torch.uint8).numpy()
    G = K // gs
    z = torch.randint(0, 16, (N, G), generator=g).numpy()
    x = torch.randn((M, K), generator=g).to(torch.float16)
    codes, sa = O.quant_act_per_token(x.view(torch.int16).numpy().view(np.uint16), "f16", q_dtype)
    sw = (torch.rand((N, G), generator=g) * 0.015 + 0.005).numpy().astype(np.float32)
    bias = (torch.randn((N,), generator=g) * 0.1).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    return u.numpy(), wl, z, codes, sa, sw, bias


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
@pytest.mark.parametrize("M,N,K,gs", [(3, 16, 384, 128), (2, 32, 256, 256)])
def test_zero_point_gemm_matches_bruteforce(q_dtype, M, N, K, gs):
    u, wl, z, codes, sa, sw, bias = _case(M, N, K, gs, q_dtype, seed=M * N + K)
    G = K // gs
    ref = O.w4a8_gemm(codes, q_dtype, sa, wl, K, "uint4", sw if G > 1 else sw[:, 0], "f32", gs, "f16",
                      bias, zeros=z)
    A = O.activation_integers(codes, q_dtype)
    unit = Fraction(1) if q_dtype == "i8" else Fraction(1, 512)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for gi in range(G):
                part = 0
                for k in range(gi * gs, (gi + 1) * gs):
                    part += int(A[m, k]) * (int(u[n, k]) - int(z[n, gi]))
                tot += Fraction(float(sw[n, gi])) * part
            v = Fraction(float(sa[m])) * tot * unit + Fraction(float(F.decode(bias[n:n + 1], "f16")[0]))
            # the oracle evaluates in float64: within a few ulps of the magnitude sum
            got = Fraction(float(ref["exact"][m, n]))
            assert abs(got - v) <= Fraction(1, 2 ** 48) * Fraction(float(ref["mag"][m, n])), (m, n)


def test_zero_point_eight_is_uint4b8():
    M, N, K, gs = 4, 48, 512, 128
    u, wl, z, codes, sa, sw, bias = _case(M, N, K, gs, "i8", seed=5)
    z8 = np.full_like(z, 8)
    a = O.w4a8_gemm(codes, "i8", sa, wl, K, "uint4", sw, "f32", gs, "f16", bias, zeros=z8)
    b = O.w4a8_gemm(codes, "i8", sa, wl, K, "uint4b8", sw, "f32", gs, "f16", bias)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["exact"], b["exact"])


def test_shifting_codes_and_zero_points_together():
    M, N, K, gs = 3, 32, 256, 128
    g = torch.Generator().manual_seed(9)
    u = torch.randint(0, 15, (N, K), generator=g)          # room for +1
    z = torch.randint(0, 15, (N, K // gs), generator=g).numpy()
    pack = lambda t: (t[:, 0::2] | (t[:, 1::2] << 4)).to(torch.uint8).numpy()
    x = torch.randn((M, K), generator=g).to(torch.float16)
    codes, sa = O.quant_act_per_token(x.view(torch.int16).numpy().view(np.uint16), "f16", "i8")
    sw = np.full((N, K // gs), 0.01, np.float32)
    a = O.w4a8_gemm(codes, "i8", sa, pack(u), K, "uint4", sw, "f32", gs, "f16", zeros=z)
    b = O.w4a8_gemm(codes, "i8", sa, pack(u + 1), K, "uint4", sw, "f32", gs, "f16", zeros=z + 1)
    assert np.array_equal(a["exact"], b["exact"])
    # a group whose codes all equal its zero-point contributes nothing
    u2 = u.clone()
    u2[:, :gs] = torch.from_numpy(z[:, :1]).repeat(1, gs)
    p = O.w4a8_group_partials(codes, "i8", pack(u2), K, "uint4", gs, zeros=z)
    assert not np.any(p[0]) and np.any(p[1])
