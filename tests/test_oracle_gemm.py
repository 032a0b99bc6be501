"""Pins for the oracle's GEMMs (CPU only).

* group partials against pure-Python integer brute force (nibbles decoded
  inline with a different expression than the oracle's);
* outputs against exact rational arithmetic rounded by ``tests/exact.py``, on
  tiny shapes and on the whole M=16, N=256, K=512 per-channel problem;
* invariants of the definition (zero weights, identity weights, equal group
  scales == per-channel, K permutation inside groups, scale doubling, negation,
  zero-point conventions);
* mutation checks: plausible mistakes planted in the oracle (monkeypatched, on
  the CPU) make the pins above fail.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import w4_oracle as O
from tests import exact as X


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16)


def _code(wl, n, k):
    byte = int(wl[n, k // 2])
    return (byte >> (4 * (k % 2))) & 15


def _w_int4(wl, n, k):
    c = _code(wl, n, k)
    return c - 16 if c & 8 else c


def _a_int(codes, m, k, q_dtype):
    c = int(codes[m, k])
    if q_dtype == "i8":
        return c if c < 128 else c - 256
    v = X.e4m3fn_code_to_fraction(c & 0xFF) * 512
    assert v.denominator == 1
    return int(v)


def _brute_partials(codes, q_dtype, wl, K, gs):
    codes = np.asarray(codes).view(np.uint8) if q_dtype == "i8" else np.asarray(codes)
    M, N = codes.shape[0], wl.shape[0]
    G = K // gs
    W = [[_w_int4(wl, n, k) for k in range(K)] for n in range(N)]
    A = [[_a_int(codes, m, k, q_dtype) for k in range(K)] for m in range(M)]
    P = np.zeros((G, M, N), dtype=np.int64)
    for g in range(G):
        for m in range(M):
            Am = A[m][g * gs:(g + 1) * gs]
            for n in range(N):
                Wn = W[n][g * gs:(g + 1) * gs]
                P[g, m, n] = sum(a * w for a, w in zip(Am, Wn))
    return P


def _case(name, M, N=None, K=None, with_bias=False, seed_base=None):
    wl = workloads.WORKLOADS[name]
    return workloads.make_case(wl, M, with_bias=with_bias, N=N, K=K, seed_base=seed_base)


def _quant(c):
    return O.quant_act_per_token(_bits(c.a), c.wl.a_dtype, c.wl.q_dtype)


def _sw_fraction(c, n, g):
    s = c.w_scales
    if s.dim() == 1:
        return Fraction(float(s[n]))
    return Fraction(float(s[n, g].float()))


def _exact_w4a8(c, codes, sa, gs):
    """Exact rational output bits of the W4A8 definition (test-side)."""
    K = c.a.shape[1]
    wl = c.w_logical.numpy()
    P = _brute_partials(codes, c.wl.q_dtype, wl, K, gs)
    unit = Fraction(1) if c.wl.q_dtype == "i8" else Fraction(1, 512)
    G, M, N = P.shape
    out = np.zeros((M, N), dtype=np.uint16)
    for m in range(M):
        sam = Fraction(float(sa[m]))
        for n in range(N):
            acc = sum(_sw_fraction(c, n, g) * int(P[g, m, n]) for g in range(G))
            v = sam * acc * unit
            if c.bias is not None:
                v += Fraction(float(c.bias[n].float()))
            r = X.round_fraction(v, c.wl.out_dtype)
            out[m, n] = X.fraction_to_f16_bits(r) if c.wl.out_dtype == "f16" else X.fraction_to_bf16_bits(r)
    return P, out


def _oracle_w4a8(c, codes, sa, gs, rows=None, cols=None):
    return O.w4a8_gemm(codes, c.wl.q_dtype, sa, c.w_logical.numpy(), c.a.shape[1], c.wl.wtype,
                       c.w_scales.view(torch.int16).numpy() if c.wl.s_dtype != "f32" else c.w_scales.numpy(),
                       c.wl.s_dtype, gs, c.wl.out_dtype,
                       None if c.bias is None else _bits(c.bias), rows=rows, cols=cols)


# ---------------------------------------------------------------------------
# Pins.
# ---------------------------------------------------------------------------

def check_partials_brute(name="w4a8_i8_g128_o", M=3, N=16, K=256):
    c = _case(name, M, N=N, K=K)
    codes, sa = _quant(c)
    gs = 128 if c.wl.group_size != c.wl.K else K
    P = O.w4a8_group_partials(codes, c.wl.q_dtype, c.w_logical.numpy(), K, c.wl.wtype, gs)
    return np.array_equal(P, _brute_partials(codes, c.wl.q_dtype, c.w_logical.numpy(), K, gs))


def check_outputs_exact(name, M, N, K, with_bias):
    c = _case(name, M, N=N, K=K, with_bias=with_bias)
    codes, sa = _quant(c)
    gs = K if c.wl.group_size == c.wl.K else c.wl.group_size
    _, want = _exact_w4a8(c, codes, sa, gs)
    got = _oracle_w4a8(c, codes, sa, gs)["out"]
    return np.array_equal(got, want)


@pytest.mark.parametrize("name", ["w4a8_i8_g128_o", "w4a8_fp8_g128_28672x8192", "w4a8_i8_pc_256x512"])
def test_partials_match_integer_bruteforce(name):
    assert check_partials_brute(name)


@pytest.mark.parametrize("name,M,N,K,bias", [
    ("w4a8_i8_pc_256x512", 3, 16, 128, False),
    ("w4a8_i8_g128_o", 2, 32, 256, True),
    ("w4a8_fp8_g128_28672x8192", 3, 16, 384, False),
    ("w4a8_fp8_g128_28672x8192", 1, 16, 256, True),
])
def test_w4a8_outputs_match_exact_rationals(name, M, N, K, bias):
    assert check_outputs_exact(name, M, N, K, bias)


@pytest.mark.slow
def test_w4a8_small_config_exact_everywhere():
    """All 16 x 256 outputs of the M=16, N=256, K=512 per-channel problem,
    bit for bit against exact rationals."""
    assert check_outputs_exact("w4a8_i8_pc_256x512", 16, 256, 512, False)


def _exact_w4a16(c, gs):
    K = c.a.shape[1]
    wl = c.w_logical.numpy()
    M, N = c.a.shape[0], wl.shape[0]
    G = K // gs
    dec = X.bf16_bits_to_fraction if c.wl.a_dtype == "bf16" else X.f16_bits_to_fraction
    ab = _bits(c.a)
    A = [[dec(int(ab[m, k])) for k in range(K)] for m in range(M)]
    sb = _bits(c.w_scales)
    zb = None if c.zeros is None else _bits(c.zeros)
    out = np.zeros((M, N), dtype=np.uint16)
    ex = np.zeros((M, N))
    for n in range(N):
        U = [_code(wl, n, k) for k in range(K)]
        for m in range(M):
            tot = Fraction(0)
            for g in range(G):
                z = Fraction(8) if zb is None else dec(int(zb[n, g]))
                d = sum(A[m][k] * (U[k] - z) for k in range(g * gs, (g + 1) * gs))
                tot += dec(int(sb[n, g])) * d
            if c.bias is not None:
                tot += dec(int(_bits(c.bias)[n]))
            r = X.round_fraction(tot, c.wl.a_dtype)
            out[m, n] = X.fraction_to_bf16_bits(r) if c.wl.a_dtype == "bf16" else X.fraction_to_f16_bits(r)
            ex[m, n] = float(tot)
    return out, ex


def _oracle_w4a16(c, gs, zeros="given"):
    z = None if (c.zeros is None or zeros is None) else _bits(c.zeros)
    return O.w4a16_gemm(_bits(c.a), c.wl.a_dtype, c.w_logical.numpy(), c.a.shape[1], c.wl.wtype,
                        _bits(c.w_scales), z, gs, None if c.bias is None else _bits(c.bias))


@pytest.mark.parametrize("M,N,K,bias", [(2, 16, 256, False), (3, 32, 128, True)])
def test_w4a16_outputs_match_exact_rationals(M, N, K, bias):
    c = _case("w4a16_bf16_g128_4096x4096", M, N=N, K=K, with_bias=bias)
    want, ex = _exact_w4a16(c, 128)
    r = _oracle_w4a16(c, 128)
    assert np.allclose(r["exact"], ex, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["out"], want)


@pytest.mark.parametrize("gs", [64, 32])
def test_w4a16_small_groups_match_exact_rationals(gs):
    """Groups of 64 and 32 (the W4A16 API page's kernel narrows its K tile to
    the group size): scales and zero-points [N, K/gs], exact rationals."""
    c = _case("w4a16_bf16_g128_4096x4096", 2, N=16, K=256, with_bias=True)
    g = torch.Generator().manual_seed(gs)
    G = 256 // gs
    c.w_scales = (torch.rand((16, G), generator=g) * 0.015 + 0.005).to(torch.bfloat16)
    c.zeros = torch.randint(0, 16, (16, G), generator=g).to(torch.bfloat16)
    want, ex = _exact_w4a16(c, gs)
    r = _oracle_w4a16(c, gs)
    assert np.allclose(r["exact"], ex, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["out"], want)


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------

def test_zero_weights_give_bias():
    c = _case("w4a8_i8_g128_o", 4, N=32, K=256, with_bias=True)
    c.w_logical.zero_()
    codes, sa = _quant(c)
    r = _oracle_w4a8(c, codes, sa, 128)
    assert np.array_equal(r["out"], np.broadcast_to(_bits(c.bias), r["out"].shape))
    c.bias = None
    r = _oracle_w4a8(c, codes, sa, 128)
    assert np.all(F.f16_bits_to_f64(r["out"]) == 0)


@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
def test_identity_weights_reproduce_quantised_activations(q_dtype):
    K = 256
    name = "w4a8_i8_pc_256x512" if q_dtype == "i8" else "w4a8_fp8_g128_28672x8192"
    c = _case(name, 5, N=K, K=K)
    vals = torch.eye(K, dtype=torch.int16)
    c.w_logical = workloads.store_nibbles(vals)
    gs = K
    c.w_scales = torch.ones((K,) if c.w_scales.dim() == 1 else (K, 1), dtype=c.w_scales.dtype)
    codes, sa = _quant(c)
    r = _oracle_w4a8(c, codes, sa, gs)
    deq = O.activation_integers(codes, q_dtype) * (1.0 if q_dtype == "i8" else 2.0 ** -9)
    want = F.round_and_encode(deq * sa[:, None].astype(np.float64), c.wl.out_dtype)
    assert np.array_equal(r["out"], want)


def test_equal_group_scales_equal_per_channel():
    c = _case("w4a8_i8_g128_down", 4, N=48, K=512)
    codes, sa = _quant(c)
    per_ch = c.w_scales[:, 0].float().contiguous()              # fp16 values, exact in fp32
    grp = c.w_scales[:, :1].repeat(1, 4).contiguous()
    rg = O.w4a8_gemm(codes, "i8", sa, c.w_logical.numpy(), 512, "int4",
                     _bits(grp), "f16", 128, "f16")
    rc = O.w4a8_gemm(codes, "i8", sa, c.w_logical.numpy(), 512, "int4",
                     per_ch.numpy(), "f32", 512, "f16")
    assert np.array_equal(rg["out"], rc["out"])


def test_k_permutation_inside_groups():
    c = _case("w4a8_i8_g128_o", 3, N=32, K=256)
    codes, sa = _quant(c)
    rng = np.random.default_rng(0)
    perm = np.concatenate([g * 128 + rng.permutation(128) for g in range(2)])
    vals = c.w_values[:, perm]
    r0 = _oracle_w4a8(c, codes, sa, 128)
    c.w_logical = workloads.store_nibbles(vals)
    r1 = _oracle_w4a8(c, codes[:, perm], sa, 128)
    assert np.array_equal(r0["out"], r1["out"])


def test_scale_doubling_and_negation():
    c = _case("w4a8_i8_pc_256x512", 4, N=32, K=256)
    codes, sa = _quant(c)
    r0 = _oracle_w4a8(c, codes, sa, 256)
    c.w_scales = c.w_scales * 2
    r1 = _oracle_w4a8(c, codes, sa, 256)
    assert np.array_equal(F.f16_bits_to_f64(r1["out"]), 2 * F.f16_bits_to_f64(r0["out"]))
    c.w_scales = c.w_scales / 2
    vals = c.w_values.clamp(-7, 7)
    c.w_logical = workloads.store_nibbles(vals)
    ra = _oracle_w4a8(c, codes, sa, 256)
    c.w_logical = workloads.store_nibbles(-vals)
    rb = _oracle_w4a8(c, codes, sa, 256)
    assert np.array_equal(F.f16_bits_to_f64(ra["out"]), -F.f16_bits_to_f64(rb["out"]))


def test_uint4b8_equals_int4_with_flipped_sign_bit():
    c = _case("w4a8_i8_g128_o", 3, N=32, K=256)
    codes, sa = _quant(c)
    r0 = _oracle_w4a8(c, codes, sa, 128)
    flipped = (c.w_logical.numpy() ^ np.uint8(0x88))
    r1 = O.w4a8_gemm(codes, "i8", sa, flipped, 256, "uint4b8", _bits(c.w_scales), "f16", 128, "f16")
    assert np.array_equal(r0["out"], r1["out"])


def test_w4a16_zero_point_conventions():
    c = _case("w4a16_bf16_g128_4096x4096", 3, N=32, K=256)
    # explicit z = 8 equals the symmetric (no zero-point) path
    c.zeros = torch.full_like(c.zeros, 8.0)
    a = _oracle_w4a16(c, 128)
    b = _oracle_w4a16(c, 128, zeros=None)
    assert np.array_equal(a["out"], b["out"])
    # Machete's pre-scaled form: (u * s - z') @ a with z' = z * s (exact in float64)
    c = _case("w4a16_bf16_g128_4096x4096", 2, N=16, K=256)
    r = _oracle_w4a16(c, 128)
    u = O.nibbles(c.w_logical.numpy(), 256).astype(np.float64)
    s = F.bf16_bits_to_f64(_bits(c.w_scales))
    z = F.bf16_bits_to_f64(_bits(c.zeros))
    s_k = np.repeat(s, 128, axis=1)
    zs_k = np.repeat(z * s, 128, axis=1)
    deq = u * s_k - zs_k
    a64 = F.bf16_bits_to_f64(_bits(c.a))
    assert np.allclose(a64 @ deq.T, r["exact"], rtol=1e-12, atol=1e-12)


def test_sampled_rows_cols_match_full():
    c = _case("w4a8_i8_g128_o", 8, N=64, K=256)
    codes, sa = _quant(c)
    full = _oracle_w4a8(c, codes, sa, 128)
    rows, cols = np.array([0, 5, 7]), np.array([3, 17, 40, 63])
    sub = _oracle_w4a8(c, codes, sa, 128, rows=rows, cols=cols)
    assert np.array_equal(sub["out"], full["out"][np.ix_(rows, cols)])


# ---------------------------------------------------------------------------
# Mutation checks: a planted mistake must make a pin fail.
# ---------------------------------------------------------------------------

def _swap_nibbles(w_logical, K):
    b = np.asarray(w_logical, dtype=np.uint8)
    out = np.empty((b.shape[0], K), dtype=np.int64)
    out[:, 0::2] = b >> 4
    out[:, 1::2] = b & 0xF
    return out


def test_mutation_swapped_nibbles_is_caught(monkeypatch):
    monkeypatch.setattr(O, "nibbles", _swap_nibbles)
    assert not check_partials_brute()


def test_mutation_unsigned_int4_is_caught(monkeypatch):
    real = O.weight_values
    monkeypatch.setattr(O, "weight_values",
                        lambda wl, K, wtype: real(wl, K, "uint4" if wtype == "int4" else wtype))
    assert not check_partials_brute()


def test_mutation_missing_activation_scale_is_caught(monkeypatch):
    real = O.w4a8_gemm

    def broken(codes, q_dtype, a_scales, *args, **kw):
        return real(codes, q_dtype, np.ones_like(a_scales), *args, **kw)
    monkeypatch.setattr(O, "w4a8_gemm", broken)
    assert not check_outputs_exact("w4a8_i8_pc_256x512", 2, 16, 128, False)


def test_mutation_wrong_group_boundary_is_caught(monkeypatch):
    real = O.w4a8_group_partials

    def broken(codes, q_dtype, w_logical, K, wtype, group_size, rows=None, cols=None):
        P = real(codes, q_dtype, w_logical, K, wtype, group_size, rows, cols)
        return P[::-1].copy()                    # groups paired with the wrong scales
    monkeypatch.setattr(O, "w4a8_group_partials", broken)
    assert not check_outputs_exact("w4a8_i8_g128_o", 2, 16, 256, False)


def test_mutation_truncating_quantiser_is_caught(monkeypatch):
    real_rint = np.rint
    monkeypatch.setattr(O.np, "rint", np.trunc)
    try:
        c = _case("w4a8_i8_pc_256x512", 2, N=16, K=128)
        q, s = O.quant_act_per_token(_bits(c.a), "f16", "i8")
    finally:
        monkeypatch.setattr(O.np, "rint", real_rint)
    xs = c.a.float()
    st = xs.abs().amax(dim=1) / 127.0
    qt = torch.round(xs / st[:, None]).clamp(-127, 127).to(torch.int8).numpy()
    assert not np.array_equal(q, qt)
