"""Pins for the oracle's W4A16 group partials and for the error magnitude
``mag`` both GEMM oracles return (CPU only).

* ``w4a16_group_partials``: D[g, m, n] = sum_{k in g} a[m, k] * (u[n, k] - z[n, g])
  (the W4A16 API page, docstring of the skinny-format kernel: each nibble
  minus its group's zero-point, 8 when no zero-points are given) against
  exact rationals, with codes and values decoded inline here; fp16 and bf16
  activations, groups of 128, 64, 32 and per channel, with and without
  zero-points.  The identity sum_g s[n, g] * D[g] = the GEMM's exact value
  ties the partials to the output the GEMM tests pin separately.
* ``mag`` (the sum of the absolute values of every term of an output: the
  per-group products of activation, weight and scale, times the activation
  scale, plus |bias|) against the same sum in exact rationals, W4A8 int8 and
  fp8, grouped and per channel, and W4A16.
* Planted mistakes in the oracle (a neighbouring group's zero-point, the
  constant 8 when zero-points are given, |sum| instead of sum |.|) each make
  one of these pins fail.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import w4_oracle as O
from tests import exact as X


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _code(wl, n, k):
    return (int(wl[n, k >> 1]) >> (4 * (k & 1))) & 15


def _dec(dtype):
    return X.bf16_bits_to_fraction if dtype == "bf16" else X.f16_bits_to_fraction


def _w4a16_case(a_dtype, M, N, K, gs, seed, zeros=True, bias=False):
    """A small W4A16 case with [N, K/gs] scales and zero-points in a_dtype."""
    name = "w4a16_bf16_g128_4096x4096"
    wl = workloads.WORKLOADS[name]
    c = workloads.make_case(wl, M, N=N, K=K, with_bias=bias, seed_base=seed)
    dt = torch.bfloat16 if a_dtype == "bf16" else torch.float16
    g = torch.Generator().manual_seed(seed + 7)
    G = K // gs
    c.a = c.a.float().to(dt)
    c.w_scales = (torch.rand((N, G), generator=g) * 0.015 + 0.005).to(dt)
    c.zeros = torch.randint(0, 16, (N, G), generator=g).to(dt) if zeros else None
    if c.bias is not None:
        c.bias = c.bias.float().to(dt)
    return c


def _exact_w4a16_partials(c, a_dtype, gs):
    """D[g][m][n] and the per-output sum of |terms| as exact rationals."""
    K = c.a.shape[1]
    wl = c.w_logical.numpy()
    M, N, G = c.a.shape[0], wl.shape[0], K // gs
    dec = _dec(a_dtype)
    ab = _bits(c.a)
    A = [[dec(int(ab[m, k])) for k in range(K)] for m in range(M)]
    zb = None if c.zeros is None else _bits(c.zeros)
    sb = _bits(c.w_scales)
    D = [[[None] * N for _ in range(M)] for _ in range(G)]
    mag = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for g in range(G):
            z = Fraction(8) if zb is None else dec(int(zb[n, g]))
            s = dec(int(sb[n, g]))
            ks = range(g * gs, (g + 1) * gs)
            w = [_code(wl, n, k) - z for k in ks]
            for m in range(M):
                D[g][m][n] = sum(A[m][k] * wk for k, wk in zip(ks, w))
                mag[m][n] += abs(s) * sum(abs(A[m][k]) * abs(wk) for k, wk in zip(ks, w))
    if c.bias is not None:
        bb = _bits(c.bias)
        for m in range(M):
            for n in range(N):
                mag[m][n] += abs(dec(int(bb[n])))
    return D, mag


def _oracle_partials(c, a_dtype, gs):
    z = None if c.zeros is None else _bits(c.zeros)
    return O.w4a16_group_partials(_bits(c.a), a_dtype, c.w_logical.numpy(), c.a.shape[1], "uint4", z, gs)


def check_w4a16_partials(a_dtype, gs, zeros=True, M=2, N=16, K=256, seed=11):
    """The oracle's D against exact rationals.  Every product a * (u - z) is
    exact in float64; the sum of 128 of them is exact for fp16 activations
    (all multiples of 2**-24 below 2**27) and within K * 2**-53 * sum|terms|
    for bf16."""
    c = _w4a16_case(a_dtype, M, N, K, gs, seed, zeros)
    D = _oracle_partials(c, a_dtype, gs)
    Dx, _ = _exact_w4a16_partials(c, a_dtype, gs)
    ab = _bits(c.a)
    dec = _dec(a_dtype)
    G = K // gs
    if D.shape != (G, M, N):
        return False
    for g in range(G):
        for m in range(M):
            absa = sum(abs(dec(int(ab[m, k]))) for k in range(g * gs, (g + 1) * gs))
            for n in range(N):
                err = abs(Fraction(float(D[g, m, n])) - Dx[g][m][n])
                bound = Fraction(0) if a_dtype == "f16" else Fraction(gs, 2 ** 53) * 15 * absa
                if err > bound:
                    return False
    return True


@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("gs", [128, 64, 32, 256])
def test_w4a16_partials_match_exact_rationals(a_dtype, gs):
    assert check_w4a16_partials(a_dtype, gs, zeros=True)


@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
def test_w4a16_partials_without_zero_points_subtract_8(a_dtype):
    assert check_w4a16_partials(a_dtype, 128, zeros=False)


@pytest.mark.parametrize("a_dtype,gs", [("bf16", 128), ("f16", 64), ("bf16", 32)])
def test_w4a16_scaled_partials_sum_to_the_gemm(a_dtype, gs):
    """sum_g s[n, g] * D[g, m, n] is the GEMM's exact value (no bias)."""
    K = 512
    c = _w4a16_case(a_dtype, 3, 32, K, gs, seed=5)
    D = _oracle_partials(c, a_dtype, gs)
    s = np.array([[float(v) for v in row] for row in c.w_scales.float()])
    tot = np.einsum("gmn,ng->mn", D, s)
    r = O.w4a16_gemm(_bits(c.a), a_dtype, c.w_logical.numpy(), K, "uint4", _bits(c.w_scales),
                     _bits(c.zeros), gs)
    assert np.allclose(tot, r["exact"], rtol=1e-13, atol=1e-13)


def test_w4a16_partials_window_matches_full():
    c = _w4a16_case("bf16", 6, 48, 256, 128, seed=3)
    z = _bits(c.zeros)
    full = O.w4a16_group_partials(_bits(c.a), "bf16", c.w_logical.numpy(), 256, "uint4", z, 128)
    rows, cols = np.array([1, 4, 5]), np.array([0, 17, 33, 47])
    sub = O.w4a16_group_partials(_bits(c.a), "bf16", c.w_logical.numpy(), 256, "uint4", z, 128,
                                 rows=rows, cols=cols)
    assert np.array_equal(sub, full[:, rows][:, :, cols])


# ---------------------------------------------------------------------------
# mag: the sum of |terms| of each output.
# ---------------------------------------------------------------------------

def check_w4a16_mag(a_dtype="bf16", gs=128, bias=True):
    K = 256
    c = _w4a16_case(a_dtype, 2, 16, K, gs, seed=9, bias=bias)
    r = O.w4a16_gemm(_bits(c.a), a_dtype, c.w_logical.numpy(), K, "uint4", _bits(c.w_scales),
                     _bits(c.zeros), gs, None if c.bias is None else _bits(c.bias))
    _, mag = _exact_w4a16_partials(c, a_dtype, gs)
    want = np.array([[float(v) for v in row] for row in mag])
    return np.allclose(r["mag"], want, rtol=1e-13, atol=0)


def _w4a8_exact_mag(c, codes, sa, gs, q_dtype):
    """s_a[m] * sum_g |s_w[n, g]| * sum_{k in g} |A[m, k]| |w[n, k]| * unit + |bias[n]|."""
    K = c.a.shape[1]
    wl = c.w_logical.numpy()
    M, N, G = codes.shape[0], wl.shape[0], K // gs

    def a_val(m, k):
        v = int(codes[m, k])
        if q_dtype == "i8":
            return Fraction(v - 256 if v >= 128 else v)
        return X.e4m3fn_code_to_fraction(v & 0xFF)

    def w_val(n, k):
        cc = _code(wl, n, k)
        return cc - 16 if cc >= 8 else cc

    s = c.w_scales
    out = np.zeros((M, N))
    for m in range(M):
        sam = Fraction(float(sa[m]))
        for n in range(N):
            tot = Fraction(0)
            for g in range(G):
                sw = Fraction(float(s[n])) if s.dim() == 1 else Fraction(float(s[n, g].float()))
                tot += abs(sw) * sum(abs(a_val(m, k)) * abs(w_val(n, k)) for k in range(g * gs, (g + 1) * gs))
            v = abs(sam) * tot
            if c.bias is not None:
                v += abs(Fraction(float(c.bias[n].float())))
            out[m, n] = float(v)
    return out


def check_w4a8_mag(name, M=2, N=16, K=256, bias=True):
    wl = workloads.WORKLOADS[name]
    c = workloads.make_case(wl, M, N=N, K=K, with_bias=bias, seed_base=17)
    codes, sa = O.quant_act_per_token(_bits(c.a), wl.a_dtype, wl.q_dtype)
    gs = K if wl.group_size == wl.K else wl.group_size
    s = c.w_scales.numpy() if wl.s_dtype == "f32" else _bits(c.w_scales)
    r = O.w4a8_gemm(codes, wl.q_dtype, sa, c.w_logical.numpy(), K, wl.wtype, s, wl.s_dtype, gs, wl.out_dtype,
                    None if c.bias is None else _bits(c.bias))
    want = _w4a8_exact_mag(c, codes, sa, gs, wl.q_dtype)
    return np.allclose(r["mag"], want, rtol=1e-13, atol=0)


@pytest.mark.parametrize("name", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o", "w4a8_fp8_g128_28672x8192"])
def test_w4a8_mag_matches_exact_rationals(name):
    assert check_w4a8_mag(name)


@pytest.mark.parametrize("a_dtype,gs", [("bf16", 128), ("f16", 64), ("bf16", 32)])
def test_w4a16_mag_matches_exact_rationals(a_dtype, gs):
    assert check_w4a16_mag(a_dtype, gs)


# ---------------------------------------------------------------------------
# Planted mistakes.
# ---------------------------------------------------------------------------

def test_mutation_neighbouring_group_zero_point_is_caught(monkeypatch):
    real = O.w4a16_group_partials

    def broken(a_bits, a_dtype, w_logical, K, wtype, zeros_bits, group_size, rows=None, cols=None):
        z = np.asarray(zeros_bits).reshape(w_logical.shape[0], -1)
        return real(a_bits, a_dtype, w_logical, K, wtype, np.roll(z, 1, axis=1), group_size, rows, cols)
    monkeypatch.setattr(O, "w4a16_group_partials", broken)
    assert not check_w4a16_partials("f16", 128)


def test_mutation_constant_8_with_zero_points_is_caught(monkeypatch):
    real = O.w4a16_group_partials

    def broken(a_bits, a_dtype, w_logical, K, wtype, zeros_bits, group_size, rows=None, cols=None):
        return real(a_bits, a_dtype, w_logical, K, wtype, None, group_size, rows, cols)
    monkeypatch.setattr(O, "w4a16_group_partials", broken)
    assert not check_w4a16_partials("bf16", 64)


def test_mutation_abs_of_sum_for_mag_is_caught(monkeypatch):
    real8, real16 = O.w4a8_gemm, O.w4a16_gemm

    def broken8(*args, **kw):
        r = real8(*args, **kw)
        return dict(r, mag=np.abs(r["exact"]))

    def broken16(*args, **kw):
        r = real16(*args, **kw)
        return dict(r, mag=np.abs(r["exact"]))
    monkeypatch.setattr(O, "w4a8_gemm", broken8)
    monkeypatch.setattr(O, "w4a16_gemm", broken16)
    assert not check_w4a8_mag("w4a8_i8_g128_o")
    assert not check_w4a16_mag("bf16", 128)


def test_mutation_mag_without_activation_scale_is_caught(monkeypatch):
    real8 = O.w4a8_gemm

    def broken8(codes, q_dtype, a_scales, *args, **kw):
        r = real8(codes, q_dtype, a_scales, *args, **kw)
        sa = np.asarray(a_scales, dtype=np.float64)[:, None]
        return dict(r, mag=r["mag"] / sa)
    monkeypatch.setattr(O, "w4a8_gemm", broken8)
    assert not check_w4a8_mag("w4a8_fp8_g128_28672x8192", bias=False)
