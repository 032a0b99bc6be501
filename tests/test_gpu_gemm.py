"""GPU parity of the W4A8 / W4A16 GEMMs against the oracle.

* int8 group partials: bit-exact, on both kernels, several K splits, ragged
  M and N tails (tiles of 16 x 16 MMA blocks, 64/128 rows and 128/256 columns
  per workgroup);
* fp8 / W4A16 group partials: within the fp32 accumulation bound;
* outputs: the acceptance rules of tests/parity.py;
* every workload at its full size on sampled rows and columns.
"""
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import formats as F
from oracle import w4_oracle as O
from tests.parity import DEV, DeviceCase, assert_w4a8, assert_w4a16, bits16, fp8_partials_bound

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def options(path=0, splitk=0, bm=0, strips=0):
    w4.set_option("force_path", path)
    w4.set_option("splitk", splitk)
    w4.set_option("tiled_bm", bm)
    w4.set_option("skinny_strips", strips)
    try:
        yield
    finally:
        for k in ("force_path", "splitk", "tiled_bm", "skinny_strips"):
            w4.set_option(k, 0)


def run_w4a8(dc: DeviceCase):
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, sa = w4.quant_act_per_token(dc.a, dc.wl.q_dtype)
    out_dt = torch.float16 if dc.wl.out_dtype == "f16" else torch.bfloat16
    gs = -1 if dc.gs == dc.K else dc.gs
    out = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out_dt, wtype=dc.wtype, bias=dc.bias)
    return out, aq, sa, packed


# ---------------------------------------------------------------------------
# Group partials.
# ---------------------------------------------------------------------------
SKINNY = [(1, 1), (3, 2), (16, 4), (7, 5)]           # (M, waves splitting K)
TILED = [(17, 1), (130, 1), (200, 3), (64, 4)]      # (M, K splits)


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o"])
@pytest.mark.parametrize("path,M,split", [(1, m, s) for m, s in SKINNY] + [(2, m, s) for m, s in TILED])
@pytest.mark.parametrize("wtype", ["int4", "uint4b8"])
def test_int8_partials_bit_exact(wl, path, M, split, wtype):
    dc = DeviceCase(wl, M, N=272, K=640, seed_base=M * 7 + path, wtype=wtype)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, sa = w4.quant_act_per_token(dc.a, "i8")
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(path, split):
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, gs, wtype=dc.wtype)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, dc.wtype, dc.gs)
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o", "w4a8_fp8_g128_28672x8192"])
@pytest.mark.parametrize("M,waves,strips", [(8, 4, 2), (12, 8, 2), (16, 3, 1), (13, 8, 1)])
def test_small_m_staged_partials(wl, M, waves, strips):
    """The small-M kernel from M = 8, whose activations are staged in LDS,
    with one and two strips (grouped two-strip forms are compiled for six
    waves per SIMD): int8 partials bit-exact, fp8 within its MFMA bound."""
    dc = DeviceCase(wl, M, N=512, K=1536, seed_base=M * 13 + waves)
    q = dc.wl.q_dtype
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, q)
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(1, waves, 0, strips):
        assert w4.gemm_plan(M, dc.N, dc.K, gs, w4.I8 if q == "i8" else w4.FP8_E4M3) == (1, waves, 16, 16 * strips)
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, gs)
    codes = aq.cpu().numpy()
    want = O.w4a8_group_partials(codes, q, dc.case.w_logical.numpy(), dc.K, "int4", dc.gs)
    if q == "i8":
        assert np.array_equal(part.cpu().numpy().astype(np.int64), want)
    else:
        got = part.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - want * 2.0 ** -9) <= fp8_partials_bound(codes, dc.case.w_logical.numpy(), dc.K))


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o"])
@pytest.mark.parametrize("M,split", [(17, 1), (130, 1), (200, 3), (256, 2)])
def test_int8_partials_bit_exact_tall_tiles(wl, M, split):
    """128-row tiles (128 x 256 per channel, 128 x 128 grouped), ragged M and N."""
    dc = DeviceCase(wl, M, N=272, K=640, seed_base=M * 11 + 5)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(2, split, 128):
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, gs)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, "int4", dc.gs)
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o"])
@pytest.mark.parametrize("M,split", [(17, 1), (100, 3), (128, 2)])
@pytest.mark.parametrize("wtype", ["int4", "uint4b8"])
def test_int8_partials_bit_exact_narrow_tiles(wl, M, split, wtype):
    """64 x 128 tiles (2 column blocks per wave), ragged M and N."""
    dc = DeviceCase(wl, M, N=272, K=640, seed_base=M * 13 + split, wtype=wtype)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    gs = -1 if dc.gs == dc.K else dc.gs
    with options(2, split, 64, 2):
        assert w4.gemm_plan(M, dc.N, dc.K, gs, w4.I8) == (2, split, 64, 128)
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, gs, wtype=dc.wtype)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, dc.wtype, dc.gs)
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o", "w4a8_fp8_g128_28672x8192"])
@pytest.mark.parametrize("M,split", [(33, 1), (130, 2)])
def test_w4a8_narrow_tiles_outputs(wl, M, split):
    dc = DeviceCase(wl, M, N=400, K=1280, with_bias=True, seed_base=M + split)
    with options(2, split, 64, 2):
        out, *_ = run_w4a8(dc)
    codes, sa = dc.oracle_quant()
    ref = dc.oracle_w4a8(codes, sa)
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, label=f"{wl} 64x128 M={M}")
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, strict=True, label=f"{wl} 64x128 strict M={M}")


@pytest.mark.parametrize("M,split,bm", [(130, 1, 256), (300, 3, 256), (520, 2, 256), (256, 1, 256),
                                        (70, 1, 128), (130, 2, 128), (200, 3, 128)])
@pytest.mark.parametrize("wtype", ["int4", "uint4b8"])
def test_int8_partials_bit_exact_pingpong(M, split, bm, wtype):
    """The ping-pong kernel's 256 x 256 and 128 x 256 tiles (two halves),
    ragged M (a half with no rows, a partial half) and N = 272 (a second
    column tile with one n-block), with and without K splits."""
    dc = DeviceCase("w4a8_i8_pc_256x512", M, N=272, K=1280, seed_base=M * 17 + split, wtype=wtype)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    with options(4, split, bm):
        assert w4.gemm_plan(M, dc.N, dc.K, -1, w4.I8) == (4, split, bm, 256)
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, -1, wtype=dc.wtype)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, dc.wtype, dc.K)
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("M,split,bm,wtype", [(200, 1, 256, "int4"), (400, 2, 256, "uint4b8"), (513, 1, 256, "int4"),
                                               (100, 2, 128, "int4"), (333, 1, 128, "uint4b8")])
def test_w4a8_pingpong_outputs(M, split, bm, wtype):
    dc = DeviceCase("w4a8_i8_pc_256x512", M, N=528, K=1536, with_bias=True, seed_base=M + 7, wtype=wtype)
    with options(4, split, bm):
        out_t, *_ = run_w4a8(dc)
    codes, sa = dc.oracle_quant()
    ref = dc.oracle_w4a8(codes, sa)
    assert_w4a8(out_t, ref, dc.wl.out_dtype, "i8", 1, label=f"ping-pong M={M}")
    assert_w4a8(out_t, ref, dc.wl.out_dtype, "i8", 1, strict=True, label=f"ping-pong strict M={M}")


def test_int8_partials_window():
    dc = DeviceCase("w4a8_i8_g128_o", 40, N=512, K=1024, seed_base=3)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    win = (5, 33, 48, 400)
    part = w4.w4a8_gemm_partials(aq, packed, dc.N, 128, window=win)
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, "int4", 128,
                                 rows=np.arange(5, 33), cols=np.arange(48, 400))
    assert np.array_equal(part.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("path,M,split,bm,strips", [(1, 5, 4, 0, 0), (2, 70, 2, 64, 0), (2, 70, 2, 128, 0),
                                                    (2, 150, 1, 128, 0), (2, 90, 3, 64, 2)])
def test_fp8_partials_within_bound(path, M, split, bm, strips):
    dc = DeviceCase("w4a8_fp8_g128_28672x8192", M, N=272, K=512, seed_base=11)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "fp8")
    with options(path, split, bm, strips):
        part = w4.w4a8_gemm_partials(aq, packed, dc.N, 128).cpu().numpy().astype(np.float64)
    codes = aq.cpu().numpy()
    P = O.w4a8_group_partials(codes, "fp8", dc.case.w_logical.numpy(), dc.K, "int4", 128)
    exact = P * 2.0 ** -9
    # the fp8 MFMA sums the 128 exact products with a precision of its own
    assert np.all(np.abs(part - exact) <= fp8_partials_bound(codes, dc.case.w_logical.numpy(), dc.K))


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("path,M,split", [(1, 4, 2), (2, 40, 1), (2, 100, 3)])
@pytest.mark.parametrize("zeros", [True, False])
def test_w4a16_partials_within_bound(a_dtype, path, M, split, zeros):
    wl = "w4a16_bf16_g128_4096x4096"
    dc = DeviceCase(wl, M, N=144, K=384, seed_base=21, zeros=zeros)
    a = dc.a if a_dtype == "bf16" else dc.a.float().to(torch.float16)
    z = None if dc.zeros is None else (dc.zeros if a_dtype == "bf16" else dc.zeros.float().to(torch.float16))
    packed = w4.prepack_B(dc.w_logical, "f16")
    with options(path, split):
        part = w4.w4a16_gemm_partials(a, packed, dc.N, 128, zeros=z).cpu().numpy().astype(np.float64)
    ab = bits16(a.cpu())
    zb = None if z is None else bits16(z.cpu())
    D = O.w4a16_group_partials(ab, a_dtype, dc.case.w_logical.numpy(), dc.K, "uint4", zb, 128)
    av = np.abs(F.decode(ab, a_dtype))
    # the bf16 path multiplies by (128 + c) and subtracts (128 + z) * sum(a)
    big = 300.0 if a_dtype == "bf16" else 16.0
    bound = np.stack([np.repeat(av[:, g * 128:(g + 1) * 128].sum(axis=1, keepdims=True), dc.N, axis=1)
                      for g in range(dc.G)]) * big * 140 * 2.0 ** -24
    assert np.all(np.abs(part - D) <= bound)


# ---------------------------------------------------------------------------
# Outputs.
# ---------------------------------------------------------------------------
W4A8_CASES = [
    ("w4a8_i8_pc_256x512", "int4"), ("w4a8_i8_g128_o", "int4"), ("w4a8_i8_g128_o", "uint4b8"),
    ("w4a8_fp8_g128_28672x8192", "int4"), ("w4a8_fp8_g128_28672x8192", "uint4b8"),
]


@pytest.mark.parametrize("wl,wtype", W4A8_CASES)
@pytest.mark.parametrize("M", [1, 5, 16, 17, 130, 257])
@pytest.mark.parametrize("bias", [False, True])
def test_w4a8_outputs(wl, wtype, M, bias):
    dc = DeviceCase(wl, M, N=272, K=640, with_bias=bias, seed_base=M + 1000, wtype=wtype)
    out, aq, sa, _ = run_w4a8(dc)
    codes, sa_o = dc.oracle_quant()
    ref = dc.oracle_w4a8(codes, sa_o)
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, label=f"{wl} M={M}")


@pytest.mark.parametrize("wl,K", [("w4a8_i8_g128_o", 16384), ("w4a8_i8_g128_o", 96000), ("w4a8_i8_g128_o", 106496),
                                  ("w4a8_fp8_g128_28672x8192", 53248)])
@pytest.mark.parametrize("M", [3, 12])
def test_w4a8_small_m_long_grouped_k(wl, K, M):
    """Grouped small-M problems with long K: the staged group-scale table
    holds up to 767 groups for one strip (K = 96000: 750 groups, 47 KiB);
    past that the plan uses the tiled kernel.  M = 12 also stages the
    activations (64 KiB for eight waves next to the table)."""
    dc = DeviceCase(wl, M, N=64, K=K, seed_base=K % 1000 + M)
    out, *_ = run_w4a8(dc)
    codes, sa = dc.oracle_quant()
    assert_w4a8(out, dc.oracle_w4a8(codes, sa), dc.wl.out_dtype, dc.wl.q_dtype, dc.G, label=f"{wl} K={K} M={M}")


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_fp8_g128_28672x8192", "w4a8_i8_g128_down"])
@pytest.mark.parametrize("path,split,bm", [(1, 1, 0), (1, 8, 0), (2, 1, 64), (2, 2, 64), (2, 5, 64),
                                           (2, 1, 128), (2, 3, 128)])
def test_w4a8_forced_paths_agree(wl, path, split, bm):
    M = 16 if path == 1 else (48 if bm == 64 else 150)
    dc = DeviceCase(wl, M, N=528, K=1280, seed_base=77)
    with options(path, split, bm):
        out, *_ = run_w4a8(dc)
    codes, sa = dc.oracle_quant()
    assert_w4a8(out, dc.oracle_w4a8(codes, sa), dc.wl.out_dtype, dc.wl.q_dtype, dc.G,
                label=f"{wl} path={path} split={split} bm={bm}")


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", [1, 4, 16, 33])
@pytest.mark.parametrize("zeros,group", [(True, 128), (False, 128), (True, -1)])
def test_w4a16_outputs(a_dtype, M, zeros, group):
    wl = "w4a16_bf16_g128_4096x4096"
    dc = DeviceCase(wl, M, N=272, K=512, seed_base=M + 2000, zeros=zeros)
    c = dc.case
    if group == -1:
        c.w_scales = c.w_scales[:, :1].contiguous()
        if c.zeros is not None:
            c.zeros = c.zeros[:, :1].contiguous()
        dc.gs, dc.G = dc.K, 1
    tdt = torch.bfloat16 if a_dtype == "bf16" else torch.float16
    if a_dtype == "f16":
        c.a = c.a.float().to(tdt)
        c.w_scales = c.w_scales.float().to(tdt)
        c.zeros = None if c.zeros is None else c.zeros.float().to(tdt)
        dc.wl = workloads.Workload(**{**dc.wl.__dict__, "a_dtype": "f16", "out_dtype": "f16"})
    a = c.a.to(DEV)
    s = c.w_scales.to(DEV)
    z = None if c.zeros is None else c.zeros.to(DEV)
    packed = w4.prepack_B(dc.w_logical, "f16")
    out = w4.w4a16_gemm(a, packed, s, z, group)
    ref = dc.oracle_w4a16()
    assert_w4a16(out, ref, a_dtype, label=f"W4A16 {a_dtype} M={M}")


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("path,M", [(1, 8), (2, 100)])
@pytest.mark.parametrize("sparse", [False, True])
def test_w4a16_within_rounding_bound(a_dtype, path, M, sparse):
    """Every W4A16 output within a rounding bound of its own (stricter than
    the 1e-2 * max|ref| contract), dense and with 15 of 16 codes equal to
    their zero-point.  The fp16 operand is the exact c - z, so the MFMA
    rounds relative to sum|a (c - z)|.  The bf16 operand is 128 + c and the
    (128 + z) * sum(a) term is subtracted after the MFMAs, so they round
    relative to sum|a| (128 + c) + (128 + z) sum|a|.  Either way the output
    is a correct rounding of a value within n * 2**-24 * (that magnitude,
    weighted by |s|) of the exact result, n = 128 MFMA terms + 2 per group
    for the fold + 24 for split sums and the final steps."""
    dc = DeviceCase("w4a16_bf16_g128_4096x4096", M, N=272, K=1024, seed_base=82)
    c = dc.case
    codes = O.weight_values(c.w_logical.numpy(), dc.K, "uint4")             # [N, K] in 0..15
    zg = F.decode(bits16(c.zeros), "bf16")                                 # [N, G]
    if sparse:
        keep = (torch.rand(dc.N, dc.K, generator=torch.Generator().manual_seed(83)) < 1 / 16).numpy()
        codes = np.where(keep, codes, np.repeat(zg, 128, axis=1).astype(np.int64))
        c.w_logical = workloads.store_nibbles(torch.from_numpy(codes).to(torch.int16))
        dc.w_logical = c.w_logical.to(DEV)
    tdt = torch.bfloat16 if a_dtype == "bf16" else torch.float16
    if a_dtype == "f16":
        c.a = c.a.float().to(tdt)
        c.w_scales = c.w_scales.float().to(tdt)
        c.zeros = c.zeros.float().to(tdt)
        dc.wl = workloads.Workload(**{**dc.wl.__dict__, "a_dtype": "f16", "out_dtype": "f16"})
    with options(path):
        out = w4.w4a16_gemm(c.a.to(DEV), w4.prepack_B(dc.w_logical, "f16"), c.w_scales.to(DEV),
                            c.zeros.to(DEV), 128)
    ref = dc.oracle_w4a16()
    av = np.abs(F.decode(bits16(c.a), a_dtype))                            # [M, K]
    sv = np.abs(F.decode(bits16(c.w_scales), a_dtype))                     # [N, G]
    mag = np.zeros((M, dc.N))
    for g in range(dc.G):
        ks = slice(g * 128, (g + 1) * 128)
        if a_dtype == "f16":
            t = av[:, ks] @ np.abs(codes[:, ks] - zg[:, g:g + 1]).T
        else:
            t = av[:, ks] @ (128.0 + codes[:, ks]).T + av[:, ks].sum(axis=1, keepdims=True) * (128.0 + zg[:, g])
        mag += t * sv[:, g]
    E = (128 + 2 * dc.G + 24) * 2.0 ** -24 * mag
    got = F.decode(bits16(out), a_dtype)
    lo = F.round_to_format(ref["exact"] - E, a_dtype)
    hi = F.round_to_format(ref["exact"] + E, a_dtype)
    bad = ~((got >= lo) & (got <= hi))
    assert not bad.any(), (f"{int(bad.sum())} outside; first "
                           f"{[(tuple(i), float(got[tuple(i)]), float(ref['exact'][tuple(i)])) for i in np.argwhere(bad)[:3]]}")


def test_w4a16_uint4b8_equals_zero_point_8():
    dc = DeviceCase("w4a16_bf16_g128_4096x4096", 8, N=256, K=512, seed_base=5, zeros=False)
    packed = w4.prepack_B(dc.w_logical, "f16")
    o1 = w4.w4a16_gemm(dc.a, packed, dc.w_scales, None, 128, wtype="uint4b8")
    z8 = torch.full_like(dc.w_scales, 8.0)
    o2 = w4.w4a16_gemm(dc.a, packed, dc.w_scales, z8, 128, wtype="uint4")
    assert torch.equal(o1, o2)


def test_outputs_are_deterministic():
    dc = DeviceCase("w4a8_fp8_g128_28672x8192", 96, N=1024, K=2048, seed_base=9)
    a, *_ = run_w4a8(dc)
    b, *_ = run_w4a8(dc)
    assert torch.equal(a, b)


def test_m_zero_is_a_no_op():
    dc = DeviceCase("w4a8_i8_g128_o", 4, N=64, K=256, seed_base=1)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq = torch.empty((0, 256), dtype=torch.int8, device=DEV)
    sa = torch.empty((0,), dtype=torch.float32, device=DEV)
    out = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, 128, torch.float16)
    assert out.shape == (0, 64)


def test_zero_weights_and_identity():
    dc = DeviceCase("w4a8_i8_pc_256x512", 9, N=256, K=256, seed_base=4, with_bias=True)
    dc.case.w_logical = workloads.store_nibbles(torch.eye(256, dtype=torch.int16))
    dc.case.w_scales = torch.ones(256, dtype=torch.float32)
    dc.w_logical = dc.case.w_logical.to(DEV)
    dc.w_scales = dc.case.w_scales.to(DEV)
    dc.case.bias = None
    dc.bias = None
    out, aq, sa, _ = run_w4a8(dc)
    deq = (aq.float() * sa[:, None]).to(torch.float16)
    assert torch.equal(out, deq)                      # identity weights reproduce the quantised A
    dc.w_logical = torch.zeros_like(dc.w_logical)
    out, *_ = run_w4a8(dc)
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("wl", ["w4a8_i8_pc_256x512", "w4a8_fp8_g128_28672x8192", "w4a8_i8_g128_down"])
@pytest.mark.parametrize("path,split,bm", [(1, 1, 0), (1, 8, 0), (2, 1, 64), (2, 5, 64), (2, 3, 128)])
@pytest.mark.parametrize("sparse", [False, True])
def test_w4a8_within_rounding_bound(wl, path, split, bm, sparse):
    """Every output within the rounding bound of its own terms (the strict
    clause alone), on both kernels, with dense weights and with 15 of 16
    weights zero (small outputs, where the absolute 1e-3 of the tolerance
    would hide errors)."""
    M = 16 if path == 1 else (48 if bm == 64 else 150)
    dc = DeviceCase(wl, M, N=272, K=1024, seed_base=78)
    if sparse:
        keep = torch.Generator().manual_seed(79)
        mask = torch.rand(dc.N, dc.K, generator=keep) < 1 / 16
        vals = O.weight_values(dc.case.w_logical.numpy(), dc.K, dc.wtype)
        vals = torch.from_numpy(vals).to(torch.int16) * mask
        dc.case.w_logical = workloads.store_nibbles(vals)
        dc.w_logical = dc.case.w_logical.to(DEV)
    with options(path, split, bm):
        out, *_ = run_w4a8(dc)
    codes, sa = dc.oracle_quant()
    assert_w4a8(out, dc.oracle_w4a8(codes, sa), dc.wl.out_dtype, dc.wl.q_dtype, dc.G, strict=True,
                label=f"{wl} path={path} split={split} bm={bm} sparse={sparse}")


@pytest.mark.parametrize("path", [1, 2])
def test_fp8_grouped_zero_weights_identity_and_extremes(path):
    """Grouped fp8 on both kernels with unit scales: identity weights give the
    dequantised codes, zero weights give zero, weights of -8 give -8 times the
    dequantised codes, bit for bit.  Each output then has one nonzero product
    per group, which the MFMA's fp8 accumulation keeps exactly.  (An int4 ->
    e4m3 expansion as two operands, 8 + l and -8 (1 + s), failed this: next to
    the large 8a terms the accumulation dropped low-order bits of the small
    ones, errors of 1e-3 on outputs of 5e-3.)"""
    dc = DeviceCase("w4a8_fp8_g128_28672x8192", 9, N=256, K=256, seed_base=5)
    dc.case.w_scales = torch.ones((256, 2), dtype=torch.float32)
    dc.w_scales = dc.case.w_scales.to(DEV)
    dc.case.bias = None
    dc.bias = None
    eye = torch.eye(256, dtype=torch.int16)
    for mult in (1, 0, -8):
        dc.w_logical = workloads.store_nibbles(mult * eye).to(DEV)
        with options(path):
            out, aq, sa, _ = run_w4a8(dc)
        deq = aq.cpu().view(torch.float8_e4m3fn).float() * sa.cpu()[:, None]
        assert torch.equal(out.cpu(), (mult * deq).to(torch.bfloat16)), f"weights {mult} * I"


# ---------------------------------------------------------------------------
# Full-size workloads on sampled outputs.
# ---------------------------------------------------------------------------
def _sample(n, k, rng, must=()):
    idx = set(must) | set(rng.choice(n, size=min(k, n), replace=False).tolist())
    return np.array(sorted(i for i in idx if 0 <= i < n))


FULL_W4A8 = ["w4a8_i8_pc_8192x21760", "w4a8_i8_g128_qkv", "w4a8_i8_g128_o", "w4a8_i8_g128_gateup",
             "w4a8_i8_g128_down", "w4a8_fp8_g128_28672x8192", "w4a8_i8_pc_256x512"]


@pytest.mark.parametrize("wl_name", FULL_W4A8)
def test_w4a8_full_size_sampled(wl_name):
    wl = workloads.WORKLOADS[wl_name]
    Mmax = max(wl.Ms)
    case = workloads.make_case(wl, Mmax, seed_base=123)
    packed = w4.prepack_B(case.w_logical.to(DEV), "i8")
    s_dev = case.w_scales.to(DEV)
    a_dev = case.a.to(DEV)
    out_dt = torch.float16 if wl.out_dtype == "f16" else torch.bfloat16
    gs = -1 if wl.group_size == wl.K else wl.group_size
    G = 1 if gs == -1 else wl.K // gs
    rng = np.random.default_rng(len(wl_name))
    # small problems are compared whole, the others on sampled rows x columns
    whole = wl.N * Mmax <= 65536
    cols = np.arange(wl.N) if whole else _sample(wl.N, 192, rng, must=(0, 15, 16, wl.N - 1))
    sd = "f32" if wl.s_dtype == "f32" else wl.s_dtype
    s_np = case.w_scales.numpy() if sd == "f32" else bits16(case.w_scales)
    for M in wl.Ms:
        aq, sa = w4.quant_act_per_token(a_dev[:M].contiguous(), wl.q_dtype)
        out = w4.w4a8_gemm(aq, sa, packed, s_dev, gs, out_dt)
        rows = np.arange(M) if whole else _sample(M, 12, rng, must=(0, M - 1))
        codes, sa_o = O.quant_act_per_token(bits16(case.a[rows]), wl.a_dtype, wl.q_dtype)
        ref = O.w4a8_gemm(codes, wl.q_dtype, sa_o, case.w_logical.numpy(), wl.K, wl.wtype, s_np, sd,
                          wl.K if gs == -1 else gs, wl.out_dtype, cols=cols)
        sub = out[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
        assert_w4a8(sub, ref, wl.out_dtype, wl.q_dtype, G, label=f"{wl_name} M={M}")


def test_w4a16_full_size():
    wl = workloads.WORKLOADS["w4a16_bf16_g128_4096x4096"]
    case = workloads.make_case(wl, max(wl.Ms), seed_base=321)
    packed = w4.prepack_B(case.w_logical.to(DEV), "f16")
    s, z, a = case.w_scales.to(DEV), case.zeros.to(DEV), case.a.to(DEV)
    for M in wl.Ms:
        out = w4.w4a16_gemm(a[:M].contiguous(), packed, s, z, 128)
        ref = O.w4a16_gemm(bits16(case.a[:M]), "bf16", case.w_logical.numpy(), wl.K, "uint4",
                           bits16(case.w_scales), bits16(case.zeros), 128)
        assert_w4a16(out, ref, "bf16", label=f"W4A16 full M={M}")
