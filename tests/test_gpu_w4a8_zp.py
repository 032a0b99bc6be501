"""GPU parity: asymmetric (zero-point) W4A8 against the oracle, and against
the symmetric uint4b8 path when every zero-point is 8."""
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, assert_w4a8, bits16

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@contextlib.contextmanager
def options(path=0, splitk=0, bm=0):
    w4.set_option("force_path", path)
    w4.set_option("splitk", splitk)
    w4.set_option("tiled_bm", bm)
    try:
        yield
    finally:
        w4.set_option("force_path", 0)
        w4.set_option("splitk", 0)
        w4.set_option("tiled_bm", 0)


class ZpCase:
    def __init__(self, M, N, K, gs, seed, s_dtype="f16", z_dtype="f16", out_dtype="f16", bias=False, z=None):
        g = torch.Generator().manual_seed(seed)
        self.M, self.N, self.K = M, N, K
        self.gs = K if gs == -1 else gs
        self.G = K // self.gs
        self.u = workloads.int4_codes(N, K, "uint4", seed=seed)
        self.wl = workloads.store_nibbles(self.u)
        zz = torch.randint(0, 16, (N, self.G), generator=g) if z is None else torch.full((N, self.G), z)
        self.z_np = zz.numpy()
        shape = (N,) if gs == -1 else (N, self.G)
        self.z = zz.reshape(shape).to(TD[z_dtype])
        self.s = (torch.rand(shape, generator=g) * 0.015 + 0.005).to(TD[s_dtype])
        self.s_dtype, self.out_dtype = s_dtype, out_dtype
        self.bias = (torch.randn((N,), generator=g) * 0.1).to(TD[out_dtype]) if bias else None
        self.x = workloads.activations(M, K, "f16", seed=seed + 1)
        self.packed = w4.prepack_B(self.wl.to(DEV), "i8")

    def run(self, flag_gs=None):
        aq, sa = w4.quant_act_per_token(self.x.to(DEV), "i8")
        gs = -1 if self.gs == self.K else self.gs
        out = w4.w4a8_gemm_zp(aq, sa, self.packed, self.s.to(DEV), self.z.to(DEV), gs, TD[self.out_dtype],
                              bias=None if self.bias is None else self.bias.to(DEV))
        return out, aq, sa

    def oracle(self, aq, sa, rows=None, cols=None):
        codes = aq.cpu().numpy()
        sa_np = sa.cpu().numpy()
        if rows is not None:
            codes, sa_np = codes[rows], sa_np[rows]
        s_np = self.s.numpy() if self.s_dtype == "f32" else bits16(self.s)
        bias = None if self.bias is None else bits16(self.bias)
        return O.w4a8_gemm(codes, "i8", sa_np, self.wl.numpy(), self.K, "uint4", s_np, self.s_dtype, self.gs,
                           self.out_dtype, bias, cols=cols, zeros=self.z_np)


@pytest.mark.parametrize("gs", [128, -1])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 64, 200])
def test_zp_matches_oracle(M, gs):
    c = ZpCase(M, 256, 1024, gs, seed=M * 7 + (gs > 0), bias=True)
    out, aq, sa = c.run()
    assert_w4a8(out, c.oracle(aq, sa), c.out_dtype, "i8", c.G, label=f"zp M={M} gs={gs}")


@pytest.mark.parametrize("s_dtype,z_dtype,out_dtype", [("f32", "f32", "bf16"), ("bf16", "bf16", "f16"),
                                                       ("f16", "bf16", "bf16")])
def test_zp_dtypes(s_dtype, z_dtype, out_dtype):
    for gs in (128, -1):
        c = ZpCase(24, 128, 640, gs, seed=3, s_dtype=s_dtype, z_dtype=z_dtype, out_dtype=out_dtype)
        out, aq, sa = c.run()
        assert_w4a8(out, c.oracle(aq, sa), out_dtype, "i8", c.G, label=f"zp {s_dtype}/{z_dtype}/{out_dtype}")


@pytest.mark.parametrize("path,splitk,bm", [(1, 1, 0), (1, 4, 0), (2, 1, 64), (2, 3, 64), (2, 1, 128),
                                            (2, 2, 128)])
@pytest.mark.parametrize("gs", [128, -1])
def test_zp_forced_paths(path, splitk, bm, gs):
    M = 16 if path == 1 else 150
    c = ZpCase(M, 528, 1536, gs, seed=11 + splitk)
    with options(path, splitk, bm):
        out, aq, sa = c.run()
    assert_w4a8(out, c.oracle(aq, sa), c.out_dtype, "i8", c.G, label=f"zp path={path} split={splitk} bm={bm}")


@pytest.mark.parametrize("gs", [128, -1])
@pytest.mark.parametrize("M", [1, 16, 100, 300])
def test_zero_points_of_eight_equal_uint4b8(M, gs):
    """With every zero-point 8 the asymmetric GEMM is the symmetric uint4b8
    GEMM of the same codes: identical bits."""
    c = ZpCase(M, 512, 2048, gs, seed=M + 5, z=8, bias=True)
    out, aq, sa = c.run()
    g = -1 if gs == -1 else gs
    ref = w4.w4a8_gemm(aq, sa, c.packed, c.s.to(DEV), g, torch.float16, wtype="uint4b8", bias=c.bias.to(DEV))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("N,K,gs,Ms", [(8192, 21760, -1, (1, 16, 256, 4096)), (22016, 4096, 128, (1, 16, 1024))])
def test_zp_full_size_sampled(N, K, gs, Ms):
    c = ZpCase(max(Ms), N, K, gs, seed=77, s_dtype="f32" if gs == -1 else "f16")
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([[0, 15, 16, N - 1], rng.choice(N, 96, replace=False)]))
    aq_all, sa_all = w4.quant_act_per_token(c.x.to(DEV), "i8")
    for M in Ms:
        aq, sa = aq_all[:M].contiguous(), sa_all[:M].contiguous()
        out = w4.w4a8_gemm_zp(aq, sa, c.packed, c.s.to(DEV), c.z.to(DEV), gs, torch.float16)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 10), replace=False)]))
        ref = c.oracle(aq, sa, rows=rows, cols=cols)
        sub = out.cpu()[torch.as_tensor(rows)][:, torch.as_tensor(cols)]
        assert_w4a8(sub, ref, "f16", "i8", c.G, label=f"zp full N={N} K={K} M={M}")
