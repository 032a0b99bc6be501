"""GPU parity: W4A16 with pre-scaled zero-points (weight c * s - zs) against
the oracle, on both kernels, forced K splits, and full size on sampled
outputs."""
import contextlib

import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
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
    def __init__(self, M, N, K, a_dtype, seed, bias=False):
        g = torch.Generator().manual_seed(seed)
        G = K // 128
        self.K, self.a_dtype = K, a_dtype
        self.wl = workloads.store_nibbles(workloads.int4_codes(N, K, "uint4", seed=seed))
        self.a = workloads.activations(M, K, a_dtype, seed=seed + 1)
        self.s = (torch.rand((N, G), generator=g) * 0.015 + 0.005).to(TD[a_dtype])
        # zs around z * s for integer z in [0, 15], not exactly
        z = torch.randint(0, 16, (N, G), generator=g).float()
        self.zs = (z * self.s.float() * (1 + 0.01 * torch.randn((N, G), generator=g))).to(TD[a_dtype])
        self.bias = (torch.randn((N,), generator=g) * 0.1).to(TD[a_dtype]) if bias else None
        self.packed = w4.prepack_B(self.wl.to(DEV), "f16")

    def run(self, M=None):
        a = self.a if M is None else self.a[:M].contiguous()
        return w4.w4a16_gemm_prescaled_zeros(a.to(DEV), self.packed, self.s.to(DEV), self.zs.to(DEV), 128,
                                             bias=None if self.bias is None else self.bias.to(DEV))

    def oracle(self, rows=None, cols=None, M=None):
        a = self.a if M is None else self.a[:M]
        return O.w4a16_gemm_prescaled_zeros(bits16(a), self.a_dtype, self.wl.numpy(), self.K, bits16(self.s),
                                            bits16(self.zs), 128,
                                            None if self.bias is None else bits16(self.bias), rows=rows, cols=cols)


@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 4, 16, 17, 64, 200])
def test_prescaled_outputs(a_dtype, M):
    c = Case(M, 272, 640, a_dtype, seed=M + 17, bias=M % 2 == 0)
    assert_w4a16(c.run(), c.oracle(), a_dtype, label=f"prescaled {a_dtype} M={M}")


@pytest.mark.parametrize("path,split", [(1, 1), (1, 2), (1, 4), (2, 1), (2, 3)])
@pytest.mark.parametrize("a_dtype", ["f16", "bf16"])
def test_prescaled_forced_paths(path, split, a_dtype):
    M = 12 if path == 1 else 80
    c = Case(M, 288, 1024, a_dtype, seed=split * 5 + path)
    with options(path, split):
        out = c.run()
    assert_w4a16(out, c.oracle(), a_dtype, label=f"prescaled path={path} split={split}")


def test_prescaled_full_size_sampled():
    c = Case(1024, 4096, 4096, "bf16", seed=91)
    rng = np.random.default_rng(4)
    cols = np.unique(np.concatenate([[0, 15, 16, 4095], rng.choice(4096, 96, replace=False)]))
    for M in (1, 16, 1024):
        out = c.run(M)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 12), replace=False)]))
        ref = c.oracle(rows=rows, cols=cols, M=M)
        sub = out.cpu()[torch.as_tensor(rows)][:, torch.as_tensor(cols)]
        assert_w4a16(sub, ref, "bf16", label=f"prescaled full M={M}")
