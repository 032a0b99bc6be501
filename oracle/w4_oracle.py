"""Plain CPU oracle of the 4-bit-weight mixed-precision GEMM path.

TEST INFRASTRUCTURE ONLY.  The library (``mixed_precision_quantized_prepack_amd``)
never imports, links or executes anything in ``oracle/``; only ``tests/``, the
``smoke()`` check in ``__graft_entry__`` and the benchmark's ``cpu_baseline``
leg do.  It shares no code with the HIP path: the only common module is the
seeded input generator (``workloads.py``), which holds none of the method's
arithmetic.

Pages this follows (cited by page title and section):

* "Machete (Mixed Precision Cutlass-Based GEMM)" README, *Overview*: the GEMM
  is a matmul of the activations with the dequantised weight, where the
  dequantised weight is the integer code times its scale, minus a zero term.
  The weight is [N, K] and the output is [M, N], i.e. out = a . dequant(W)^T.
* Same README, *API*: the weight is prepacked once, before any GEMM call.
* vLLM API page "...mixed_precision.rdna_hybrid_w4a16", docstrings of
  ``_triton_w4a16_skinny_fmt_kernel`` / ``triton_w4a16_skinny_fmt_gemm``:
  W4A16 dequantisation is (nibble - zero) * scale with raw per-group
  zero-points [N, K/G] in the activation dtype; without zero-points a constant
  8 is subtracted; scales are [N, K/G]; output [M, N] in the activation dtype;
  the ExLlama nibble order inside a 32-bit word.
* vLLM PR "[Kernel] Initial Machete W4A8 support + Refactors", *summary*:
  QQQ-style W4A8 with int8 or fp8 activations; the prepack is a pure data
  shuffle, independent of the weight's signedness convention.
* vLLM PR "[ Kernel ] Enable Dynamic Per Token fp8", *summary* and review
  discussion: activations are quantised dynamically with one scale per token
  (row); the epilogue applies per-token x per-channel scales.
* pytorch/ao PR "support W4A8 Marlin kernel", *summary* and limitations
  comment: W4A8 with int4 weights, int8 activations, per-channel or per-group
  scales, symmetric weights only.

Readings where the pages are silent (each one is also listed in the design
notes):

* Activation scale = absmax / 127 (int8) or absmax / 448 (fp8 e4m3fn); codes
  are round-to-nearest-even of the fp32 quotient x / scale (a correctly rounded
  IEEE fp32 division); int8 codes are clamped to [-127, 127]; fp8 codes are
  OCP e4m3fn with saturation at +-448.  A row of zeros gets scale 0 and codes 0.
* Fused RMSNorm + per-token quantisation returns exactly what an RMSNorm
  producing its output in the activation dtype, followed by the per-token
  quantisation above, would.  The normalisation takes the exact sum of
  squares (rounded once to float64), the reciprocal square root of
  mean + eps in float64 rounded to fp32, and the products x * r * gamma in
  fp32 in that order.
* The logical (unpacked) weight is [N, K/2] bytes, even k in the low nibble.
* Everything downstream of the stored inputs is exact or float64: integer
  partial sums are exact, scales are applied in float64 and the output is
  rounded once to fp16/bf16 (round to nearest even).

Dot products use float64 matrix products (a library primitive).  For the
W4A8 paths every operand is an integer (int8 codes, or fp8 codes times 2**9)
and every partial sum is an integer below 2**53 in magnitude, so these
products are exact whatever order the library sums in.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import formats as F

# ---------------------------------------------------------------------------
# Step 1: logical nibbles -> integer weight values.
# ---------------------------------------------------------------------------

WTYPES = ("int4", "uint4", "uint4b8")


def nibbles(w_logical: np.ndarray, K: int) -> np.ndarray:
    """Raw 4-bit codes [N, K] (0..15) of the logical byte array [N, K/2]."""
    b = np.asarray(w_logical, dtype=np.uint8)
    N = b.shape[0]
    assert b.shape == (N, K // 2)
    out = np.empty((N, K), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def weight_values(w_logical: np.ndarray, K: int, wtype: str) -> np.ndarray:
    """Integer weight values [N, K] as int64.

    int4    : two's-complement nibble, value in [-8, 7]
    uint4   : value = code, in [0, 15]
    uint4b8 : value = code - 8 (the "uint4 with bias 8" type of the Machete
              PR; the W4A16 kernel page subtracts the same constant 8 when no
              zero-points are given)
    """
    c = nibbles(w_logical, K)
    if wtype == "int4":
        return c - 16 * (c >= 8)
    if wtype == "uint4":
        return c
    if wtype == "uint4b8":
        return c - 8
    raise ValueError(wtype)


# ---------------------------------------------------------------------------
# Step 2: the prepacked weight layout ("PB-v1").
#
# The weight is cut into 16 (n) x 128 (k) blocks of 1 KiB, stored n-block
# major.  Inside a block, "lane" l = 16*kq + r owns row r = n % 16 and the 32
# consecutive k in [32*kq, 32*kq + 32); its 16 bytes are four little-endian
# 32-bit words, word kw holding k in [8*kw, 8*kw + 8) of that range.  The
# nibble position of k-offset j (0..7) inside the word depends on the operand
# class the GEMM expands it to:
#   "i8"  (int8 / fp8 operands): j -> bit 8*j for j < 4, bit 8*(j-4)+4 else
#   "f16" (fp16 / bf16 operands): j -> bit 4*(j//2) + 16*(j%2)  (ExLlama order)
# The layout is independent of the weight type (INT4 / UINT4 / UINT4B8): it
# only moves nibbles.
# ---------------------------------------------------------------------------

OPERANDS = ("i8", "f16")


def pb_v1_position(n, k, K: int, operand: str):
    """(word index, bit shift) of logical element (n, k).  Vectorised."""
    n = np.asarray(n, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    nb, r = n // 16, n % 16
    kb, kk = k // 128, k % 128
    kq, kw, j = kk // 32, (kk % 32) // 8, kk % 8
    lane = 16 * kq + r
    block = nb * (K // 128) + kb
    word = block * 256 + lane * 4 + kw
    if operand == "i8":
        shift = np.where(j < 4, 8 * j, 8 * (j - 4) + 4)
    elif operand == "f16":
        shift = 4 * (j // 2) + 16 * (j % 2)
    else:
        raise ValueError(operand)
    return word, shift


def prepack_B(w_logical: np.ndarray, N: int, K: int, operand: str,
              row_chunk: int = 1024) -> np.ndarray:
    """Logical [N, K/2] bytes -> PB-v1 bytes (N*K/2), by the index formula."""
    assert N % 16 == 0 and K % 128 == 0
    words = np.zeros(N * K // 8, dtype=np.uint32)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        c = nibbles(w_logical[n0:n1], K).astype(np.uint32)
        nn = np.arange(n0, n1, dtype=np.int64)[:, None]
        # Elements with the same k % 8 land in distinct words, so each of the
        # eight passes is a plain scatter with no repeated index.
        for j in range(8):
            ks = np.arange(j, K, 8, dtype=np.int64)[None, :]
            word, shift = pb_v1_position(nn, ks, K, operand)
            words[word.ravel()] |= (c[:, j::8] << shift.astype(np.uint32)).ravel()
    return words.view(np.uint8).copy()


def exllama_to_logical(words: np.ndarray, N: int, K: int) -> np.ndarray:
    """ExLlama-shuffled int32 words [N, K/8] -> logical [N, K/2] bytes.

    vLLM API page "...mixed_precision.rdna_hybrid_w4a16", docstring of
    ``_triton_w4a16_skinny_fmt_kernel``: each word holds 8 consecutive k
    (k = 8 w + j) with k-offset j at bit (j // 2) * 4 + (j % 2) * 16.
    """
    W = np.asarray(words).view(np.uint32).reshape(N, K // 8)
    vals = np.empty((N, K), dtype=np.uint8)
    for j in range(8):
        vals[:, j::8] = (W >> np.uint32((j // 2) * 4 + (j % 2) * 16)) & np.uint32(0xF)
    return (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)


def prepack_B_from_exllama(words: np.ndarray, N: int, K: int, operand: str) -> np.ndarray:
    """PB-v1 bytes of a weight given as ExLlama-shuffled words [N, K/8]: the
    same bytes as prepacking its logical form."""
    return prepack_B(exllama_to_logical(words, N, K), N, K, operand)


def unprepack_B(packed: np.ndarray, N: int, K: int, operand: str) -> np.ndarray:
    """PB-v1 bytes -> logical [N, K/2] bytes, walking the packed words.

    Written from the packed side (word -> (n, k)) rather than by inverting
    ``pb_v1_position``, so that the two directions check each other.
    """
    words = np.asarray(packed, dtype=np.uint8).view(np.uint32)
    KB = K // 128
    d = np.arange(words.size, dtype=np.int64)
    block, lane, kw = d // 256, (d % 256) // 4, d % 4
    nb, kb = block // KB, block % KB
    kq, r = lane // 16, lane % 16
    n = nb * 16 + r
    kbase = kb * 128 + kq * 32 + kw * 8
    vals = np.zeros((N, K), dtype=np.int64)
    for p in range(8):                         # nibble p sits at bits 4p..4p+3
        code = (words >> np.uint32(4 * p)) & np.uint32(0xF)
        if operand == "i8":
            j = p // 2 if p % 2 == 0 else 4 + p // 2
        else:
            j = 2 * (p % 4) + p // 4
        vals[n, kbase + j] = code
    out = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
    return out


# ---------------------------------------------------------------------------
# Step 3: dynamic per-token activation quantisation.
# ---------------------------------------------------------------------------

QMAX = {"i8": np.float32(127.0), "fp8": np.float32(448.0)}


def quant_act_per_token(x_bits: np.ndarray, x_dtype: str, q_dtype: str):
    """Per-row (per-token) symmetric quantisation.

    amax[m] = max_k |x[m, k]|                      (exact in fp32)
    s[m]    = fp32(amax[m] / qmax)                  qmax = 127 (int8) or 448 (fp8)
    v       = fp32(x / s[m])                        correctly rounded division
    int8    : q = clamp(round_half_even(v), -127, 127)
    fp8     : q = e4m3fn(round_half_even(clamp(v, -448, 448)))
    amax = 0: s = 0, q = 0.

    Returns (codes, scales): int8 codes [M, K] (or uint8 e4m3fn bit patterns)
    and fp32 scales [M].
    """
    x = F.decode(x_bits, x_dtype).astype(np.float32)          # exact widening
    M = x.shape[0]
    if x.shape[1] == 0:
        raise ValueError("K must be positive")
    amax = np.abs(x).max(axis=1) if M else np.zeros((0,), np.float32)
    qmax = QMAX[q_dtype]
    s = (amax / qmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / s[:, None]).astype(np.float32)
    v = np.where(s[:, None] > 0, v, np.float32(0.0))
    if q_dtype == "i8":
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)
    elif q_dtype == "fp8":
        vc = np.clip(v, np.float32(-448.0), np.float32(448.0)).astype(np.float64)
        q = F.round_and_encode(vc, "e4m3fn")
    else:
        raise ValueError(q_dtype)
    return q, s


def quant_act_per_tensor(x_bits: np.ndarray, x_dtype: str, q_dtype: str):
    """Dynamic per-tensor symmetric quantisation: one scale for the whole
    [M, K] tensor.

    vLLM PR "[ Kernel ] Enable Dynamic Per Token fp8", *results* and review
    discussion: dynamic per-tensor scaling is the alternative to per-token
    (one scale, computed at run time over the whole tensor).  The codes are
    formed as in ``quant_act_per_token`` with that one scale:

    amax = max_{m,k} |x[m, k]|;  s = fp32(amax / qmax);  v = fp32(x / s)
    int8 : q = clamp(round_half_even(v), -127, 127)
    fp8  : q = e4m3fn(round_half_even(clamp(v, -448, 448)))
    amax = 0: s = 0, q = 0.

    Returns (codes [M, K], scales [M] fp32, every entry s).
    """
    x = F.decode(x_bits, x_dtype).astype(np.float32)          # exact widening
    M, K = x.shape
    if K == 0:
        raise ValueError("K must be positive")
    amax = np.abs(x).max() if M else np.float32(0.0)
    s = np.float32(np.float32(amax) / QMAX[q_dtype])
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / s).astype(np.float32)
    if s == 0:
        v = np.zeros_like(x)
    if q_dtype == "i8":
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)
    elif q_dtype == "fp8":
        vc = np.clip(v, np.float32(-448.0), np.float32(448.0)).astype(np.float64)
        q = F.round_and_encode(vc, "e4m3fn")
    else:
        raise ValueError(q_dtype)
    return q, np.full((M,), s, dtype=np.float32)


def rmsnorm_rows(x_bits: np.ndarray, x_dtype: str, gamma_bits: np.ndarray, eps: float):
    """The normalisation step of ``rmsnorm_quant_per_token`` before its final
    rounding to the activation dtype: returns (r [M] fp32, y [M, K] fp32).

    ss[m]   = sum_k x[m, k]**2               exact, rounded once to float64
    var[m]  = fp64(fp64(ss[m] / K) + eps)      eps given as fp32
    r[m]    = fp32(fp64(1 / fp64(sqrt(var[m]))))
    y[m, k] = fp32(fp32(x[m, k] * r[m]) * gamma[k])

    Each square of an fp16/bf16 value is exact in float64 and math.fsum
    returns the correctly rounded sum, so ss does not depend on any summation
    order.  eps must be positive.
    """
    if not eps > 0:
        raise ValueError("eps must be positive")
    x = F.decode(x_bits, x_dtype)                       # float64, exact
    g = F.decode(gamma_bits, x_dtype)
    M, K = x.shape
    if K == 0:
        raise ValueError("K must be positive")
    eps64 = float(np.float32(eps))
    r = np.empty((M,), dtype=np.float32)
    for m in range(M):
        ss = math.fsum((x[m] * x[m]).tolist())          # squares exact in float64
        var = ss / K + eps64
        r[m] = np.float32(1.0 / math.sqrt(var))
    y = (x.astype(np.float32) * r[:, None]) * g.astype(np.float32)[None, :]
    return r, y


def rmsnorm_quant_per_token(x_bits: np.ndarray, x_dtype: str, gamma_bits: np.ndarray, eps: float,
                            q_dtype: str):
    """RMSNorm followed by dynamic per-token quantisation, as one operation.

    vLLM PR "[ Kernel ] Enable Dynamic Per Token fp8", review discussion: one
    scale per token makes it easy to fuse the RMSNorm that precedes a linear
    layer with the quantisation of its output.  The pages fix neither the
    normalisation's precision nor the rounding between the two steps; the
    reading taken here is that the fused operation returns exactly what the
    RMSNorm, producing its output in the activation dtype, followed by
    ``quant_act_per_token`` would: y = dtype(rmsnorm_rows(x)) rounded to
    nearest even, then codes, scales = quant_act_per_token(y).

    Returns (codes, scales, y_bits).
    """
    _, y32 = rmsnorm_rows(x_bits, x_dtype, gamma_bits, eps)
    y_bits = F.round_and_encode(y32.astype(np.float64), x_dtype)
    codes, scales = quant_act_per_token(y_bits, x_dtype, q_dtype)
    return codes, scales, y_bits


def activation_integers(codes: np.ndarray, q_dtype: str) -> np.ndarray:
    """Quantised activations as exact integers (int64).

    int8: the code itself.  fp8 e4m3fn: every finite value is a multiple of
    2**-9, so value * 2**9 is an integer (|.| <= 448 * 512 = 229376).
    """
    if q_dtype == "i8":
        return np.asarray(codes, dtype=np.int8).astype(np.int64)
    v = F.e4m3fn_bits_to_f64(codes) * 512.0
    return np.rint(v).astype(np.int64)


ACT_UNIT = {"i8": 1.0, "fp8": 2.0 ** -9}   # value of one integer step


# ---------------------------------------------------------------------------
# Step 4: exact per-group partial sums (W4A8).
# ---------------------------------------------------------------------------

def _exact_int_matmul(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Exact int64 product A @ B.T for integer matrices whose partial sums
    stay below 2**53 (checked), computed with a float64 matmul."""
    bound = np.abs(A).max(initial=0) * np.abs(B).max(initial=0) * A.shape[1]
    assert bound < 2 ** 53
    return np.rint(A.astype(np.float64) @ B.astype(np.float64).T).astype(np.int64)


def zero_point_weights(w_logical: np.ndarray, K: int, zeros: np.ndarray, group_size: int) -> np.ndarray:
    """Asymmetric weights: w[n, k] = u[n, k] - z[n, k // group_size] (int64).

    u is the raw 4-bit code (0..15) and z the integer zero-point of the
    weight's group; [Marlin W4A8 PR] review (symmetric quantisation only is
    named as a limit of QQQ), with the zero-point convention of the W4A16 API
    page (raw zero-points, subtracted before the scale).
    """
    u = nibbles(w_logical, K)
    z = np.asarray(zeros, dtype=np.int64).reshape(u.shape[0], -1)
    assert z.shape[1] * group_size == K
    return u - np.repeat(z, group_size, axis=1)


def w4a8_group_partials(codes: np.ndarray, q_dtype: str, w_logical: np.ndarray, K: int,
                        wtype: str, group_size: int, rows=None, cols=None,
                        zeros: Optional[np.ndarray] = None) -> np.ndarray:
    """P[g, m, n] = sum_{k in group g} A_int[m, k] * w[n, k]   (int64, exact).

    A_int is the int8 code (int8 activations) or 512 * fp8 value (fp8
    activations), so for fp8 the partial's value is P * 2**-9.  ``rows`` /
    ``cols`` restrict the computation to a sub-matrix of the output.  With
    ``zeros`` ([N, G] integers) the weights are the asymmetric u - z (wtype
    must be "uint4").
    """
    gs = K if group_size in (-1, K) else group_size
    assert K % gs == 0
    A = activation_integers(codes if rows is None else codes[rows], q_dtype)
    wl = w_logical if cols is None else w_logical[cols]
    if zeros is None:
        W = weight_values(wl, K, wtype)
    else:
        assert wtype == "uint4"
        z = np.asarray(zeros).reshape(w_logical.shape[0], -1)
        W = zero_point_weights(wl, K, z if cols is None else z[cols], gs)
    G = K // gs
    P = np.empty((G, A.shape[0], W.shape[0]), dtype=np.int64)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        P[g] = _exact_int_matmul(A[:, sl], W[:, sl])
    return P


# ---------------------------------------------------------------------------
# Step 5: epilogues and the whole GEMMs.
# ---------------------------------------------------------------------------

def _scales_f64(s: np.ndarray, s_dtype: str) -> np.ndarray:
    if s_dtype == "f32":
        return np.asarray(s, dtype=np.float32).astype(np.float64)
    return F.decode(np.asarray(s).view(np.uint16), s_dtype)


def w4a8_gemm(codes: np.ndarray, q_dtype: str, a_scales: np.ndarray,
              w_logical: np.ndarray, K: int, wtype: str,
              w_scales: np.ndarray, s_dtype: str, group_size: int,
              out_dtype: str, bias_bits: Optional[np.ndarray] = None,
              rows=None, cols=None, zeros: Optional[np.ndarray] = None) -> dict:
    """W4A8 GEMM:  out[m, n] = RNE_out( s_a[m] * sum_g s_w[n, g] * P[g, m, n] * unit
                                         + bias[n] )

    P are the exact integer partials above (with ``zeros``: of the asymmetric
    weights u - z); unit = 1 (int8) or 2**-9 (fp8).
    Per-channel scales are [N] (one group spanning K).  All arithmetic after
    the stored inputs is float64 and the result is rounded once.

    Returns a dict with
      ``out``   : output bits (uint16) [m, n] in ``out_dtype``
      ``exact`` : the float64 value before the final rounding
      ``mag``   : float64 sum of |terms| (s_a * sum_g |s_w| * sum_k |a||w| +
                  |bias|), used to bound a different evaluation order's error.
    """
    gs = K if group_size in (-1, K) else group_size
    G = K // gs
    P = (w4a8_group_partials(codes, q_dtype, w_logical, K, wtype, gs, rows, cols) if zeros is None else
         w4a8_group_partials(codes, q_dtype, w_logical, K, wtype, gs, rows, cols, zeros=zeros))
    A = activation_integers(codes if rows is None else codes[rows], q_dtype)
    wl = w_logical if cols is None else w_logical[cols]
    if zeros is None:
        Wabs = np.abs(weight_values(wl, K, wtype))
    else:
        z = np.asarray(zeros).reshape(w_logical.shape[0], -1)
        Wabs = np.abs(zero_point_weights(wl, K, z if cols is None else z[cols], gs))
    sw = _scales_f64(w_scales, s_dtype)
    sw = sw.reshape(sw.shape[0], -1)
    if cols is not None:
        sw = sw[cols]
    assert sw.shape[1] == G
    sa = np.asarray(a_scales, dtype=np.float32).astype(np.float64)
    if rows is not None:
        sa = sa[rows]
    unit = ACT_UNIT[q_dtype]
    acc = np.zeros((A.shape[0], Wabs.shape[0]), dtype=np.float64)
    mag = np.zeros_like(acc)
    Aabs = np.abs(A)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        acc += sw[None, :, g] * P[g].astype(np.float64)
        mag += np.abs(sw[None, :, g]) * _exact_int_matmul(Aabs[:, sl], Wabs[:, sl]).astype(np.float64)
    exact = sa[:, None] * acc * unit
    mag = np.abs(sa[:, None]) * mag * unit
    if bias_bits is not None:
        b = F.decode(np.asarray(bias_bits).view(np.uint16), out_dtype)
        if cols is not None:
            b = b[cols]
        exact = exact + b[None, :]
        mag = mag + np.abs(b)[None, :]
    return dict(out=F.round_and_encode(exact, out_dtype), exact=exact, mag=mag)


def w4a16_gemm(a_bits: np.ndarray, a_dtype: str, w_logical: np.ndarray, K: int, wtype: str,
               scales_bits: np.ndarray, zeros_bits: Optional[np.ndarray], group_size: int,
               bias_bits: Optional[np.ndarray] = None, rows=None, cols=None) -> dict:
    """W4A16 GEMM: out[m, n] = RNE_a( sum_g s[n, g] * sum_{k in g} a[m, k] * (u[n, k] - z[n, g])
                                       + bias[n] )

    u is the raw 4-bit code (0..15).  z is the raw zero-point (stored in the
    activation dtype, integer valued) or the constant 8 when ``zeros_bits`` is
    None.  Scales and output use the activation dtype.  Products are exact in
    float64; sums carry float64 rounding only (relative 1e-16 level).
    """
    gs = K if group_size in (-1, K) else group_size
    G = K // gs
    a = F.decode(a_bits if rows is None else a_bits[rows], a_dtype)
    wl = w_logical if cols is None else w_logical[cols]
    if wtype not in ("uint4", "uint4b8"):
        raise ValueError("W4A16 weights are unsigned 4-bit codes")
    u = nibbles(wl, K).astype(np.float64)
    s = F.decode(np.asarray(scales_bits).view(np.uint16), a_dtype).reshape(-1, G)
    if zeros_bits is None:
        z = np.full_like(s, 8.0)
    else:
        z = F.decode(np.asarray(zeros_bits).view(np.uint16), a_dtype).reshape(-1, G)
    if cols is not None:
        s, z = s[cols], z[cols]
    acc = np.zeros((a.shape[0], u.shape[0]), dtype=np.float64)
    mag = np.zeros_like(acc)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        wq = u[:, sl] - z[:, g:g + 1]
        acc += s[None, :, g] * (a[:, sl] @ wq.T)
        mag += np.abs(s[None, :, g]) * (np.abs(a[:, sl]) @ np.abs(wq).T)
    exact = acc
    if bias_bits is not None:
        b = F.decode(np.asarray(bias_bits).view(np.uint16), a_dtype)
        if cols is not None:
            b = b[cols]
        exact = exact + b[None, :]
        mag = mag + np.abs(b)[None, :]
    return dict(out=F.round_and_encode(exact, a_dtype), exact=exact, mag=mag)


def w4a16_gemm_prescaled_zeros(a_bits: np.ndarray, a_dtype: str, w_logical: np.ndarray, K: int,
                               scales_bits: np.ndarray, zs_bits: np.ndarray, group_size: int,
                               bias_bits: Optional[np.ndarray] = None, rows=None, cols=None) -> dict:
    """W4A16 GEMM with pre-scaled zero-points (Machete README, *Overview*: the
    dequantised weight is the code times its scale minus a zero term that
    already carries the scale):

        out[m, n] = RNE_a( sum_k a[m, k] * (u[n, k] * s[n, g(k)] - zs[n, g(k)]) + bias[n] )

    u is the raw 4-bit code (0..15); s and zs are stored in the activation
    dtype.  Sums in float64 (products of the stored values are exact).
    """
    gs = K if group_size in (-1, K) else group_size
    G = K // gs
    a = F.decode(a_bits if rows is None else a_bits[rows], a_dtype)
    wl = w_logical if cols is None else w_logical[cols]
    u = nibbles(wl, K).astype(np.float64)
    s = F.decode(np.asarray(scales_bits).view(np.uint16), a_dtype).reshape(-1, G)
    zs = F.decode(np.asarray(zs_bits).view(np.uint16), a_dtype).reshape(-1, G)
    if cols is not None:
        s, zs = s[cols], zs[cols]
    acc = np.zeros((a.shape[0], u.shape[0]), dtype=np.float64)
    mag = np.zeros_like(acc)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        w = u[:, sl] * s[:, g:g + 1] - zs[:, g:g + 1]
        acc += a[:, sl] @ w.T
        mag += np.abs(a[:, sl]) @ np.abs(w).T
    exact = acc
    if bias_bits is not None:
        b = F.decode(np.asarray(bias_bits).view(np.uint16), a_dtype)
        if cols is not None:
            b = b[cols]
        exact = exact + b[None, :]
        mag = mag + np.abs(b)[None, :]
    return dict(out=F.round_and_encode(exact, a_dtype), exact=exact, mag=mag)


def w4a16_group_partials(a_bits: np.ndarray, a_dtype: str, w_logical: np.ndarray, K: int,
                         wtype: str, zeros_bits: Optional[np.ndarray], group_size: int,
                         rows=None, cols=None) -> np.ndarray:
    """D[g, m, n] = sum_{k in g} a[m, k] * (u[n, k] - z[n, g])   (float64)."""
    gs = K if group_size in (-1, K) else group_size
    G = K // gs
    a = F.decode(a_bits if rows is None else a_bits[rows], a_dtype)
    wl = w_logical if cols is None else w_logical[cols]
    u = nibbles(wl, K).astype(np.float64)
    if zeros_bits is None:
        z = np.full((u.shape[0], G), 8.0)
    else:
        z = F.decode(np.asarray(zeros_bits).view(np.uint16), a_dtype).reshape(-1, G)
        if cols is not None:
            z = z[cols]
    D = np.empty((G, a.shape[0], u.shape[0]), dtype=np.float64)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        D[g] = a[:, sl] @ (u[:, sl] - z[:, g:g + 1]).T
    return D
