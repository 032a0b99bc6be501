"""GPU parity of the streaming kernel (int8 / fp8 activations, 16 < M <= 128):
int8 group partials bit-exact and fp8 partials within the fp32 bound, on
every tile shape (32 x 256, 32 x 128, 64 x 256, 64 x 128, 128 x 128) with ragged M and N and
several K splits; outputs within the W4A8 tolerance, per channel and grouped,
int4 and uint4b8 weights, with bias."""
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
from oracle import w4_oracle as O
from tests.parity import DeviceCase, assert_w4a8, fp8_partials_bound

pytestmark = pytest.mark.gpu

STREAM = 3


@contextlib.contextmanager
def options(split=0, bm=0, nt=0):
    w4.set_option("force_path", STREAM)
    w4.set_option("splitk", split)
    w4.set_option("tiled_bm", bm)
    w4.set_option("skinny_strips", nt)
    try:
        yield
    finally:
        for k in ("force_path", "splitk", "tiled_bm", "skinny_strips"):
            w4.set_option(k, 0)


# (M, tile rows, K splits, 16-column blocks per wave): 32 x 256, 32 x 128,
# 64 x 256, 64 x 128 and 128 x 128 tiles, ragged M, N = 272 ragged for both
# tile widths
SHAPES = [(17, 32, 1, 4), (32, 32, 3, 2), (33, 64, 2, 4), (64, 64, 5, 2), (65, 128, 1, 2), (128, 128, 4, 2),
          (100, 128, 2, 2), (20, 32, 2, 2), (60, 64, 1, 4)]


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o"])
@pytest.mark.parametrize("M,bm,split,nt", SHAPES)
@pytest.mark.parametrize("wtype", ["int4", "uint4b8"])
def test_stream_int8_partials_bit_exact(wl, M, bm, split, nt, wtype):
    print(f"stream partials {wl} M={M} bm={bm} split={split} nt={nt} {wtype}", flush=True)
    dc = DeviceCase(wl, M, N=272, K=1280, seed_base=M * 5 + bm, wtype=wtype)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(split, bm, nt):
        assert w4.gemm_plan(M, dc.N, dc.K, gs, w4.I8) == (STREAM, split, bm, 64 * nt)
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, gs, wtype=dc.wtype)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, dc.wtype, dc.gs)
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("M,bm,split,nt", [(20, 32, 2, 4), (64, 64, 1, 2), (120, 128, 3, 2), (40, 64, 2, 4)])
def test_stream_fp8_partials_within_bound(M, bm, split, nt):
    dc = DeviceCase("w4a8_fp8_g128_28672x8192", M, N=272, K=768, seed_base=M + 1)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "fp8")
    with options(split, bm, nt):
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, 128).cpu().numpy().astype(np.float64)
    codes = aq.cpu().numpy()
    exact = O.w4a8_group_partials(codes, "fp8", dc.case.w_logical.numpy(), dc.K, "int4", 128) * 2.0 ** -9
    bound = fp8_partials_bound(codes, dc.case.w_logical.numpy(), dc.K)
    err = np.abs(part - exact)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, [(tuple(int(v) for v in i), float(part[tuple(i)]), float(exact[tuple(i)]),
                            float(bound[tuple(i)])) for i in bad[:8]]


OUT_CASES = [("w4a8_i8_pc_256x512", "int4"), ("w4a8_i8_g128_o", "int4"), ("w4a8_i8_g128_o", "uint4b8"),
             ("w4a8_fp8_g128_28672x8192", "int4"), ("w4a8_fp8_g128_28672x8192", "uint4b8")]


@pytest.mark.parametrize("wl,wtype", OUT_CASES)
@pytest.mark.parametrize("M,bm,split,nt", SHAPES)
def test_stream_outputs(wl, wtype, M, bm, split, nt):
    print(f"stream outputs {wl} {wtype} M={M} bm={bm} split={split} nt={nt}", flush=True)
    dc = DeviceCase(wl, M, N=272, K=1280, with_bias=True, seed_base=M * 3 + split, wtype=wtype)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, sa = w4.quant_act_per_token(dc.a, dc.wl.q_dtype)
    out_dt = torch.float16 if dc.wl.out_dtype == "f16" else torch.bfloat16
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(split, bm, nt):
        out = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out_dt, wtype=dc.wtype, bias=dc.bias)
    codes, sa_o = dc.oracle_quant()
    ref = dc.oracle_w4a8(codes, sa_o)
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, label=f"stream {wl} M={M}")
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, strict=True, label=f"stream strict {wl} M={M}")


def test_stream_grouped_long_k_takes_enough_splits():
    """A grouped K range longer than the scale table is split until it fits
    (a forced split that leaves too many groups is refused)."""
    dc = DeviceCase("w4a8_i8_g128_o", 40, N=256, K=128 * 140, seed_base=2)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, sa = w4.quant_act_per_token(dc.a, "i8")
    with options(1, 0):
        # one split would leave 140 groups for a 64-group table
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(40, 256, dc.K, 128, w4.I8)
    with options(3, 0):
        path, split, bm, bn = w4.gemm_plan(40, 256, dc.K, 128, w4.I8)
        assert path == STREAM and (140 + split - 1) // split <= 8192 // bn
        out = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, 128, torch.float16)
    codes, sa_o = dc.oracle_quant()
    assert_w4a8(out, dc.oracle_w4a8(codes, sa_o), "f16", "i8", dc.G, label="stream long K")
