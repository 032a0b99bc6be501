"""GPU parity: W4A16 with groups of 64 and 32 (2 or 4 groups per 128-deep
block) against the oracle: outputs on both kernels, forced K splits,
per-group partials within the fp32 evaluation bound, full size on sampled
outputs."""
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import formats as F
from oracle import w4_oracle as O
from tests.parity import DEV, assert_w4a16, bits16

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}


@contextlib.contextmanager
def options(path=0, splitk=0):
    w4.set_option("force_path", path)
    w4.set_option("splitk", splitk)
    try:
        yield
    finally:
        w4.set_option("force_path", 0)
        w4.set_option("splitk", 0)


class Case:
    def __init__(self, M, N, K, gs, a_dtype, seed, zeros=True, bias=False):
        g = torch.Generator().manual_seed(seed)
        self.M, self.N, self.K, self.gs, self.a_dtype = M, N, K, gs, a_dtype
        G = K // gs
        self.u = workloads.int4_codes(N, K, "uint4", seed=seed)
        self.wl = workloads.store_nibbles(self.u)
        self.a = workloads.activations(M, K, a_dtype, seed=seed + 1)
        self.s = (torch.rand((N, G), generator=g) * 0.015 + 0.005).to(TD[a_dtype])
        self.z = torch.randint(0, 16, (N, G), generator=g).to(TD[a_dtype]) if zeros else None
        self.bias = (torch.randn((N,), generator=g) * 0.1).to(TD[a_dtype]) if bias else None
        self.packed = w4.prepack_B(self.wl.to(DEV), "f16")

    def run(self):
        return w4.w4a16_gemm(self.a.to(DEV), self.packed, self.s.to(DEV),
                             None if self.z is None else self.z.to(DEV), self.gs,
                             bias=None if self.bias is None else self.bias.to(DEV))

    def oracle(self, rows=None, cols=None):
        return O.w4a16_gemm(bits16(self.a), self.a_dtype, self.wl.numpy(), self.K, "uint4", bits16(self.s),
                            None if self.z is None else bits16(self.z), self.gs,
                            None if self.bias is None else bits16(self.bias), rows=rows, cols=cols)


@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("M", [1, 4, 16, 17, 64, 150])
def test_small_group_outputs(a_dtype, gs, M):
    c = Case(M, 272, 640, gs, a_dtype, seed=M * 3 + gs, bias=M % 2 == 1)
    assert_w4a16(c.run(), c.oracle(), a_dtype, label=f"W4A16 {a_dtype} g{gs} M={M}")


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("M", [3, 40])
def test_small_group_single_block(gs, M):
    """K = 128: one block holding 2 or 4 groups, on both kernels."""
    c = Case(M, 64, 128, gs, "f16", seed=M + gs, bias=True)
    assert_w4a16(c.run(), c.oracle(), "f16", label=f"W4A16 K=128 g{gs} M={M}")


@pytest.mark.parametrize("gs", [64, 32])
def test_small_group_without_zero_points(gs):
    c = Case(8, 256, 512, gs, "bf16", seed=gs, zeros=False)
    assert_w4a16(c.run(), c.oracle(), "bf16", label=f"W4A16 g{gs} z=8")


@pytest.mark.parametrize("path,split", [(1, 1), (1, 2), (1, 4), (2, 1), (2, 3)])
@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
def test_small_group_forced_paths(path, split, gs, a_dtype):
    M = 12 if path == 1 else 80
    c = Case(M, 288, 1024, gs, a_dtype, seed=split * 7 + gs)
    with options(path, split):
        out = c.run()
    assert_w4a16(out, c.oracle(), a_dtype, label=f"W4A16 g{gs} path={path} split={split}")


@pytest.mark.parametrize("path,M,split", [(1, 4, 2), (2, 40, 1), (2, 100, 3)])
@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
def test_small_group_partials_within_bound(path, M, split, gs, a_dtype):
    c = Case(M, 144, 384, gs, a_dtype, seed=M + gs)
    with options(path, split):
        part = w4.w4a16_gemm_partials(c.a.to(DEV), c.packed, c.N, gs, zeros=c.z.to(DEV))
    part = part.cpu().numpy().astype(np.float64)
    assert part.shape == (c.K // gs, M, c.N)
    ab, zb = bits16(c.a), bits16(c.z)
    D = O.w4a16_group_partials(ab, a_dtype, c.wl.numpy(), c.K, "uint4", zb, gs)
    av = np.abs(F.decode(ab, a_dtype))
    # the bf16 path multiplies by (128 + c) and subtracts (128 + z) * sum(a)
    big = 300.0 if a_dtype == "bf16" else 16.0
    bound = np.stack([np.repeat(av[:, g * gs:(g + 1) * gs].sum(axis=1, keepdims=True), c.N, axis=1)
                      for g in range(c.K // gs)]) * big * 140 * 2.0 ** -24
    assert np.all(np.abs(part - D) <= bound)


@pytest.mark.parametrize("gs", [64, 32])
def test_small_group_full_size_sampled(gs):
    c = Case(1024, 4096, 4096, gs, "bf16", seed=gs + 1)
    rng = np.random.default_rng(gs)
    cols = np.unique(np.concatenate([[0, 15, 16, 4095], rng.choice(4096, 96, replace=False)]))
    a_dev, s_dev, z_dev = c.a.to(DEV), c.s.to(DEV), c.z.to(DEV)
    for M in (1, 16, 1024):
        out = w4.w4a16_gemm(a_dev[:M].contiguous(), c.packed, s_dev, z_dev, gs)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 12), replace=False)]))
        ref = c.oracle(rows=rows, cols=cols)
        sub = out.cpu()[torch.as_tensor(rows)][:, torch.as_tensor(cols)]
        assert_w4a16(sub, ref, "bf16", label=f"W4A16 full g{gs} M={M}")
