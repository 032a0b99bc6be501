"""Guard bands around every buffer the GEMMs write.

Outputs, split-K workspaces and partials buffers are placed between two
4 KiB bands of canary bytes; after each call the bands must be intact and the
result must pass the oracle.  Cases cover ragged M and N on every kernel and
tile shape (small-M with one and two strips; tiled 64 x 256, 128 x 256,
128 x 128 and 64 x 128 (8- and 16-bit); ping-pong 256 x 256 and 128 x 256; streaming 32 x 256, 64 x 128 and 128 x 128), with
and without K splits.  The W4A16
zero-points of the per-channel fp16 case are followed by NaN bytes: columns
past N must not read them into any stored output.
"""
import ctypes
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, DeviceCase, assert_w4a8, assert_w4a16, bits16

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


class Guarded:
    """nbytes of device memory between two guard bands of canary bytes; the
    body starts filled with `fill`."""

    def __init__(self, nbytes: int, fill: int = 0x7F):
        self.nbytes = nbytes
        body = (nbytes + 15) // 16 * 16
        self.buf = torch.full((GUARD + body + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        self.buf[GUARD:GUARD + nbytes] = fill   # the pad to 16 bytes keeps the canary
        self.body = self.buf[GUARD:GUARD + nbytes]

    def tensor(self, dtype, shape):
        return self.body.view(dtype).view(*shape)

    def check(self, what: str):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        lo = b[:GUARD]
        hi = b[GUARD + self.nbytes:]
        assert np.all(lo == CANARY), f"{what}: {int(np.sum(lo != CANARY))} bytes before the buffer overwritten"
        assert np.all(hi == CANARY), f"{what}: {int(np.sum(hi != CANARY))} bytes after the buffer overwritten"


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


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# (path, M, N, K splits, tile rows, strips): small-M with one strip (N = 272
# is not a multiple of 32) and two; tiled with ragged M and N on 64- and
# 128-row tiles, with and without K splits
SHAPES = [
    (1, 1, 272, 0, 0, 1), (1, 13, 288, 0, 0, 2), (1, 16, 272, 3, 0, 1),
    (2, 17, 272, 1, 64, 0), (2, 70, 272, 3, 64, 0), (2, 130, 272, 1, 128, 0), (2, 200, 272, 2, 128, 0),
    (3, 20, 272, 2, 32, 4), (3, 50, 272, 1, 64, 2), (3, 100, 272, 3, 128, 0), (2, 70, 272, 2, 64, 2),
    (4, 300, 272, 2, 256, 0), (4, 130, 272, 1, 128, 0),
]

W4A8 = ["w4a8_i8_pc_256x512", "w4a8_i8_g128_o", "w4a8_fp8_g128_28672x8192"]


# the ping-pong kernel (path 4) is for int8 per channel only
W4A8_CASES = [(wl,) + shape for wl in W4A8 for shape in SHAPES
              if shape[0] != 4 or wl == "w4a8_i8_pc_256x512"]


@pytest.mark.parametrize("wl,path,M,N,split,bm,strips", W4A8_CASES)
def test_w4a8_output_and_workspace_guard_bands(wl, path, M, N, split, bm, strips):
    print(f"guard w4a8 {wl} path={path} M={M} N={N} split={split} bm={bm} strips={strips}", flush=True)
    dc = DeviceCase(wl, M, N=N, K=640, with_bias=True, seed_base=M + N)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, sa = w4.quant_act_per_token(dc.a, dc.wl.q_dtype)
    out_dt = torch.float16 if dc.wl.out_dtype == "f16" else torch.bfloat16
    gs = -1 if dc.gs == dc.K else dc.gs
    a_dt = w4.I8 if dc.wl.q_dtype == "i8" else w4.FP8_E4M3
    with options(path, split, bm, strips):
        need = w4.gemm_workspace_bytes(M, N, dc.K, gs, a_dt)
        out_g = Guarded(M * N * 2)
        ws_g = Guarded(max(need, 16))
        w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out_dt, bias=dc.bias, out=out_g.tensor(out_dt, (M, N)),
                     workspace=ws_g.body)
    out_g.check("output")
    ws_g.check("workspace")
    codes, sa_o = dc.oracle_quant()
    assert_w4a8(out_g.tensor(out_dt, (M, N)), dc.oracle_w4a8(codes, sa_o), dc.wl.out_dtype, dc.wl.q_dtype, dc.G,
                label=f"guarded {wl} M={M}")


@pytest.mark.parametrize("wl,path,M,N,split,bm,strips",
                         [(wl,) + SHAPES[i] for wl in ("w4a8_i8_pc_256x512", "w4a8_i8_g128_o") for i in (0, 2, 4, 6, 7)]
                         + [("w4a8_i8_pc_256x512",) + SHAPES[-2]])
def test_w4a8_partials_guard_bands(wl, path, M, N, split, bm, strips):
    dc = DeviceCase(wl, M, N=N, K=640, seed_base=M * 3 + N)
    packed = w4.prepack_B(dc.w_logical, "i8")
    aq, _ = w4.quant_act_per_token(dc.a, "i8")
    gs = -1 if dc.gs == dc.K else dc.gs
    win = (min(1, M - 1), M, 16, N - 16)
    m0, m1, n0, n1 = win
    with options(path, split, bm, strips):
        need = w4.gemm_workspace_bytes(M, N, dc.K, gs, w4.I8)
        part_g = Guarded(dc.G * (m1 - m0) * (n1 - n0) * 4, fill=0)
        ws_g = Guarded(max(need, 16))
        st = w4.lib().w4a8_gemm_partials(_ptr(aq), w4.I8, _ptr(packed), 0, gs, M, N, dc.K, m0, m1, n0, n1,
                                         _ptr(part_g.body), _ptr(ws_g.body), ws_g.nbytes, _stream())
        assert st == 0, w4.lib().w4_last_error()
    part_g.check("partials")
    ws_g.check("workspace")
    want = O.w4a8_group_partials(aq.cpu().numpy(), "i8", dc.case.w_logical.numpy(), dc.K, "int4", dc.gs,
                                 rows=np.arange(m0, m1), cols=np.arange(n0, n1))
    got = part_g.tensor(torch.int32, (dc.G, m1 - m0, n1 - n0)).cpu().numpy().astype(np.int64)
    assert np.array_equal(got, want)


def test_w4a8_zero_point_guard_bands():
    dc = DeviceCase("w4a8_i8_pc_256x512", 150, N=272, K=640, seed_base=8)
    g = torch.Generator().manual_seed(3)
    u = torch.randint(0, 16, (272, 640), generator=g, dtype=torch.int16)
    dc.case.w_logical = workloads.store_nibbles(u)
    zeros = torch.randint(0, 16, (272,), generator=g).to(torch.float16)
    packed = w4.prepack_B(dc.case.w_logical.to(DEV), "i8")
    aq, sa = w4.quant_act_per_token(dc.a, "i8")
    for split, bm in ((1, 128), (2, 64)):
        with options(2, split, bm):
            need = w4.gemm_workspace_bytes(150, 272, 640, -1, w4.I8)
            out_g = Guarded(150 * 272 * 2)
            ws_g = Guarded(max(need, 16))
            w4.w4a8_gemm_zp(aq, sa, packed, dc.w_scales, zeros.to(DEV), -1, torch.float16,
                            out=out_g.tensor(torch.float16, (150, 272)), workspace=ws_g.body)
        out_g.check("zp output")
        ws_g.check("zp workspace")
        codes, sa_o = dc.oracle_quant()
        ref = O.w4a8_gemm(codes, "i8", sa_o, dc.case.w_logical.numpy(), 640, "uint4", dc.case.w_scales.numpy(), "f32",
                          640, "f16", zeros=zeros.numpy().astype(np.int64).reshape(-1, 1))
        assert_w4a8(out_g.tensor(torch.float16, (150, 272)), ref, "f16", "i8", 1, label=f"zp split={split}")


W4A16_SHAPES = [(1, 1, 272, 0, 1), (1, 9, 288, 2, 2), (2, 33, 272, 1, 0), (2, 100, 272, 3, 0)]


@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("gs", [-1, 128, 32])
@pytest.mark.parametrize("path,M,N,split,strips", W4A16_SHAPES)
def test_w4a16_output_and_workspace_guard_bands(a_dtype, gs, path, M, N, split, strips):
    print(f"guard w4a16 {a_dtype} gs={gs} path={path} M={M} N={N} split={split}", flush=True)
    K = 512
    dc = DeviceCase("w4a16_bf16_g128_4096x4096", M, N=N, K=K, with_bias=True, seed_base=M + 2 * N)
    dt = torch.bfloat16 if a_dtype == "bf16" else torch.float16
    G = 1 if gs == -1 else K // gs
    g = torch.Generator().manual_seed(M)
    s = (torch.rand((N, G), generator=g) * 0.015 + 0.005).to(dt)
    z = torch.randint(0, 16, (N, G), generator=g).to(dt)
    # zero-points followed by NaN: nothing past column N may reach an output
    zbuf = torch.full((N * G + 256,), float("nan"), dtype=dt)
    zbuf[:N * G] = z.reshape(-1)
    z_dev = zbuf.to(DEV)[:N * G].view(N, G)
    a = dc.case.a.float().to(dt)
    bias = dc.case.bias.float().to(dt)
    packed = w4.prepack_B(dc.w_logical, "f16")
    a_code = w4.BF16 if a_dtype == "bf16" else w4.F16
    with options(path, split, 0, strips):
        need = w4.gemm_workspace_bytes(M, N, K, gs, a_code)
        out_g = Guarded(M * N * 2)
        ws_g = Guarded(max(need, 16))
        w4.w4a16_gemm(a.to(DEV), packed, s.to(DEV), z_dev, gs, bias=bias.to(DEV), out=out_g.tensor(dt, (M, N)),
                      workspace=ws_g.body)
    out_g.check("output")
    ws_g.check("workspace")
    gsz = K if gs == -1 else gs
    ref = O.w4a16_gemm(bits16(a), a_dtype, dc.case.w_logical.numpy(), K, "uint4", bits16(s), bits16(z), gsz,
                       bits16(bias))
    assert_w4a16(out_g.tensor(dt, (M, N)), ref, a_dtype, label=f"guarded w4a16 {a_dtype} gs={gs} M={M}")


@pytest.mark.parametrize("path,M,split", [(1, 7, 2), (2, 70, 2)])
def test_w4a16_partials_guard_bands(path, M, split):
    K, N = 512, 272
    dc = DeviceCase("w4a16_bf16_g128_4096x4096", M, N=N, K=K, seed_base=M)
    packed = w4.prepack_B(dc.w_logical, "f16")
    m0, m1, n0, n1 = 0, M, 0, N
    with options(path, split):
        need = w4.gemm_workspace_bytes(M, N, K, 128, w4.BF16)
        part_g = Guarded(4 * (m1 - m0) * (n1 - n0) * 4, fill=0)
        ws_g = Guarded(max(need, 16))
        st = w4.lib().w4a16_gemm_partials(_ptr(dc.a), w4.BF16, _ptr(packed), 1, _ptr(dc.zeros), 128, M, N, K,
                                          m0, m1, n0, n1, _ptr(part_g.body), _ptr(ws_g.body), ws_g.nbytes,
                                          _stream())
        assert st == 0, w4.lib().w4_last_error()
    part_g.check("w4a16 partials")
    ws_g.check("w4a16 workspace")
    D = O.w4a16_group_partials(bits16(dc.case.a), "bf16", dc.case.w_logical.numpy(), K, "uint4",
                               bits16(dc.case.zeros), 128)
    got = part_g.tensor(torch.float32, (4, M, N)).cpu().numpy().astype(np.float64)
    scale = np.abs(D).max() + 1.0
    assert np.max(np.abs(got - D)) <= 1e-3 * scale
