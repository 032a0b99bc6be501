"""Helpers shared by the GPU parity tests: seeded cases on the device, oracle
results for the same bytes, and the acceptance rules.

Acceptance rules
----------------
* prepack bytes, quantised codes, activation scales and int32 group partials:
  bit-exact.
* W4A8 outputs: an fp16 element passes if
    |gpu - ref| <= 2e-3 * |ref| + 1e-3          (ref = the oracle's rounded output)
  and nothing else admits it.  A bf16 element passes that test, or, since
  bf16's half-ulp (up to 2**-8 relative) exceeds 2e-3, if it is a correct
  rounding of some value within E of the oracle's exact value x:
    RNE(x - E) <= gpu <= RNE(x + E),  E = n_round * 2**-24 * mag,
  where mag = sum of |terms| (from the oracle) and n_round bounds the fp32
  roundings of the GPU's evaluation order (per-group products and fused adds,
  the split-K sums, the final scale and bias; plus the 128-term MFMA sums for
  the fp32-accumulating paths).
  The strict rule (tests that check each output against its own terms) is
  the rounding-bound clause, and for fp16 outputs the first test as well.
* W4A16 outputs: |gpu - ref| <= 1e-2 * max|ref| over the whole output.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import formats as F
from oracle import w4_oracle as O

DEV = "cuda:0"


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def scales_np(t: torch.Tensor):
    if t.dtype == torch.float32:
        return t.cpu().numpy(), "f32"
    return bits16(t), {torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def n_round(q_dtype: str, G: int, splits: int = 16) -> int:
    """fp32 roundings on any path from the exact terms to the output: two per
    group (scale product, fused add), up to 16 split sums, a few for the final
    scale and bias, and for fp32-accumulating MFMAs the 128-term group sums."""
    n = 2 * G + 8 + splits
    return n if q_dtype == "i8" else n + 128


def fp8_partials_bound(codes: np.ndarray, w_logical: np.ndarray, K: int, wtype: str = "int4",
                       rows=None, cols=None) -> np.ndarray:
    """Per-group bound [G, M, N] on |GPU fp8 partial - exact partial|.

    The partial is the sum of the group's 128 exact products a*w, formed by
    one fp8 MFMA.  That instruction does not sum them as a sequence of IEEE
    fp32 additions: measured on MI355X, its result can differ from the exact
    sum by up to about 2**-12 of the largest product's binade (it behaves
    like products aligned to the largest one with ~12-13 bits kept below it),
    which exceeds gamma_128 * sum|a*w| on some outputs.  The bound is the
    larger of gamma_128 * sum|a*w| and 2**-10 * 2**floor(log2 max|a*w|)."""
    A = O.activation_integers(codes if rows is None else codes[rows], "fp8").astype(np.float64) * 2.0 ** -9
    wl = w_logical if cols is None else w_logical[cols]
    W = O.weight_values(wl, K, wtype).astype(np.float64)
    G = K // 128
    out = np.empty((G, A.shape[0], W.shape[0]))
    for g in range(G):
        Ag, Wg = np.abs(A[:, g * 128:(g + 1) * 128]), np.abs(W[:, g * 128:(g + 1) * 128])
        s = Ag @ Wg.T
        mx = np.max(Ag[:, None, :] * Wg[None, :, :], axis=2)
        win = np.where(mx > 0, 2.0 ** (np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - 10), 0.0)
        out[g] = np.maximum(128 * 2.0 ** -24 * s, win)
    return out


def w4a8_accept(gpu_bits: np.ndarray, ref: dict, out_dtype: str, q_dtype: str, G: int, strict: bool = False):
    """Per-element acceptance.  fp16 outputs: the tolerance |d| <= 2e-3 |ref|
    + 1e-3 alone; bf16 outputs: that or the rounding-bound clause.  strict:
    the rounding-bound clause, whose width scales with each output's own terms
    (the absolute 1e-3 of the first test would pass any error on outputs of
    that size), and for fp16 both."""
    got = F.decode(gpu_bits, out_dtype)
    want = F.decode(ref["out"], out_dtype)
    ok1 = np.abs(got - want) <= 2e-3 * np.abs(want) + 1e-3
    E = n_round(q_dtype, G) * 2.0 ** -24 * ref["mag"]
    lo = F.round_to_format(ref["exact"] - E, out_dtype)
    hi = F.round_to_format(ref["exact"] + E, out_dtype)
    ok2 = (got >= lo) & (got <= hi)
    if out_dtype == "f16":
        ok = ok1 & ok2 if strict else ok1
    else:
        ok = ok2 if strict else ok1 | ok2
    stats = dict(n=int(got.size), exact=int(np.sum(gpu_bits == ref["out"])),
                 bad=int(np.sum(~ok)), max_abs=float(np.max(np.abs(got - want), initial=0.0)))
    return ok, stats


def assert_w4a8(gpu_out: torch.Tensor, ref: dict, out_dtype: str, q_dtype: str, G: int, label="",
                strict: bool = False):
    ok, st = w4a8_accept(bits16(gpu_out), ref, out_dtype, q_dtype, G, strict)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        got = F.decode(bits16(gpu_out), out_dtype)
        want = F.decode(ref["out"], out_dtype)
        detail = [(tuple(i), float(got[tuple(i)]), float(want[tuple(i)]), float(ref["exact"][tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{label}: {st['bad']} of {st['n']} outside tolerance; first {detail}")
    return st


def assert_w4a16(gpu_out: torch.Tensor, ref: dict, a_dtype: str, label=""):
    got = F.decode(bits16(gpu_out), a_dtype)
    want = F.decode(ref["out"], a_dtype)
    tol = 1e-2 * np.max(np.abs(want), initial=0.0)
    err = np.abs(got - want)
    assert np.all(err <= tol), f"{label}: max err {err.max()} > {tol}"
    return dict(n=int(got.size), exact=int(np.sum(bits16(gpu_out) == ref["out"])), max_abs=float(err.max(initial=0)))


class DeviceCase:
    """A seeded case with its inputs on the GPU and helpers to query the oracle."""

    def __init__(self, wl_name: str, M: int, N=None, K=None, with_bias=False, seed_base=None,
                 wtype=None, zeros=True, a_dist="normal"):
        wl = workloads.WORKLOADS[wl_name]
        self.wl = wl
        self.case = workloads.make_case(wl, M, with_bias=with_bias, N=N, K=K, seed_base=seed_base,
                                        a_dist=a_dist)
        c = self.case
        self.M, self.K = c.a.shape
        self.N = c.w_logical.shape[0]
        self.gs = self.K if wl.group_size == wl.K else wl.group_size
        self.G = self.K // self.gs
        self.wtype = wtype or wl.wtype
        if self.wtype == "uint4b8" and wl.kind == "w4a8":
            # same codes read with bias 8: flip bit 3 so the values stay those of int4
            c.w_logical = c.w_logical ^ 0x88
        if not zeros:
            c.zeros = None
        self.a = c.a.to(DEV)
        self.w_logical = c.w_logical.to(DEV)
        self.w_scales = c.w_scales.to(DEV)
        self.zeros = None if c.zeros is None else c.zeros.to(DEV)
        self.bias = None if c.bias is None else c.bias.to(DEV)

    # ---- oracle side (CPU) ----
    def oracle_quant(self, rows=None):
        ab = bits16(self.case.a if rows is None else self.case.a[rows])
        return O.quant_act_per_token(ab, self.wl.a_dtype, self.wl.q_dtype)

    def oracle_w4a8(self, codes, sa, cols=None):
        """Oracle W4A8 output for the rows the given codes / scales belong to."""
        s, sd = scales_np(self.case.w_scales)
        bias = None if self.case.bias is None else bits16(self.case.bias)
        return O.w4a8_gemm(codes, self.wl.q_dtype, sa, self.case.w_logical.numpy(), self.K, self.wtype,
                           s, sd, self.gs, self.wl.out_dtype, bias, rows=None, cols=cols)

    def oracle_w4a16(self, rows=None, cols=None):
        c = self.case
        z = None if c.zeros is None else bits16(c.zeros)
        bias = None if c.bias is None else bits16(c.bias)
        a = bits16(c.a)
        return O.w4a16_gemm(a, self.wl.a_dtype, c.w_logical.numpy(), self.K, self.wtype,
                            bits16(c.w_scales), z, self.gs, bias, rows=rows, cols=cols)
