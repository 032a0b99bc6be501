"""Seeded synthetic inputs for the 4-bit-weight GEMM path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only draws random numbers and stores them in the dtypes the
library consumes; it holds none of the method's arithmetic (no unpacking, no
quantisation, no dot products, no scaling).

Every tensor returned is a CPU tensor.  The callers copy what they need to the
device or view it as numpy for the oracle.

Storage formats
---------------
* activations ``a``   : [M, K] float16 or bfloat16, row-major.
* weights ``w_logical``: [N, K/2] uint8; byte (n, j) holds the 4-bit code of
  k = 2j in bits 0..3 and of k = 2j + 1 in bits 4..7.  For INT4 the code is the
  two's-complement nibble of a value in [-8, 7]; for UINT4 it is the value in
  [0, 15].
* W4A8 weight scales  : [N] (per channel) or [N, K/G] (grouped), row-major.
* W4A16 scales/zeros  : [N, K/G] in the activation dtype.

Workloads
---------
The distributions follow the method's published workloads: ~N(0, 1)
activations, uniform int4 codes, scales ~U(0.005, 0.02), integer zero-points
uniform in [0, 15].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# ----------------------------------------------------------------------------
# Workload table (shapes and dtypes only).
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "w4a8" or "w4a16"
    N: int
    K: int
    Ms: tuple
    group_size: int      # K means per-channel
    a_dtype: str         # "f16" | "bf16"   (activation input dtype)
    q_dtype: Optional[str]  # "i8" | "fp8" for W4A8, None for W4A16
    s_dtype: str         # weight-scale storage dtype: "f32" | "f16" | "bf16"
    out_dtype: str       # "f16" | "bf16"
    wtype: str           # "int4" | "uint4"
    has_zeros: bool = False


WORKLOADS = {
    # W4A8 per-channel symmetric, small correctness case.
    "w4a8_i8_pc_256x512": Workload("w4a8_i8_pc_256x512", "w4a8", 256, 512, (16,), 512,
                                   "f16", "i8", "f32", "f16", "int4"),
    # W4A16 group-128 asymmetric decode GEMM.
    "w4a16_bf16_g128_4096x4096": Workload("w4a16_bf16_g128_4096x4096", "w4a16", 4096, 4096,
                                          (1, 4, 16), 128, "bf16", None, "bf16", "bf16",
                                          "uint4", has_zeros=True),
    # W4A8 per-channel at the method's GEMM benchmark shape.
    "w4a8_i8_pc_8192x21760": Workload("w4a8_i8_pc_8192x21760", "w4a8", 8192, 21760,
                                      (1, 16, 64, 256, 1024, 4096), 21760,
                                      "f16", "i8", "f32", "f16", "int4"),
    # W4A8 group-128 over 7B-style decoder-layer shapes.
    "w4a8_i8_g128_qkv": Workload("w4a8_i8_g128_qkv", "w4a8", 12288, 4096, (1, 16, 128, 1024),
                                 128, "f16", "i8", "f16", "f16", "int4"),
    "w4a8_i8_g128_o": Workload("w4a8_i8_g128_o", "w4a8", 4096, 4096, (1, 16, 128, 1024),
                               128, "f16", "i8", "f16", "f16", "int4"),
    "w4a8_i8_g128_gateup": Workload("w4a8_i8_g128_gateup", "w4a8", 22016, 4096,
                                    (1, 16, 128, 1024), 128, "f16", "i8", "f16", "f16", "int4"),
    "w4a8_i8_g128_down": Workload("w4a8_i8_g128_down", "w4a8", 4096, 11008, (1, 16, 128, 1024),
                                  128, "f16", "i8", "f16", "f16", "int4"),
    # W4A8 with fp8-e4m3 per-token activations, group-128 fp32 scales.
    "w4a8_fp8_g128_28672x8192": Workload("w4a8_fp8_g128_28672x8192", "w4a8", 28672, 8192,
                                         (1, 32, 512, 8192), 128, "bf16", "fp8", "f32",
                                         "bf16", "int4"),
}

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


# ----------------------------------------------------------------------------
# Random draws.
# ----------------------------------------------------------------------------

def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def activations(M: int, K: int, dtype: str, seed: int, dist: str = "normal") -> torch.Tensor:
    """[M, K] activations drawn ~N(0, 1) in fp32 and stored in ``dtype``."""
    g = _gen(seed)
    if dist == "normal":
        x = torch.randn((M, K), generator=g, dtype=torch.float32)
    elif dist == "wide":
        # log-uniform magnitudes over ~24 binades with random signs: exercises
        # small, subnormal-adjacent and large codes in the quantiser.
        mag = torch.exp2(torch.rand((M, K), generator=g) * 24.0 - 16.0)
        sign = torch.randint(0, 2, (M, K), generator=g).float() * 2 - 1
        x = mag * sign
    else:
        raise ValueError(dist)
    return x.to(TORCH_DTYPES[dtype]).contiguous()


def norm_weight(K: int, dtype: str, seed: int) -> torch.Tensor:
    """[K] RMSNorm weight ~U(0.25, 1.75) stored in ``dtype``."""
    g = _gen(seed)
    return (torch.rand((K,), generator=g, dtype=torch.float32) * 1.5 + 0.25).to(TORCH_DTYPES[dtype]).contiguous()


def int4_codes(N: int, K: int, wtype: str, seed: int, lo: Optional[int] = None,
               hi: Optional[int] = None) -> torch.Tensor:
    """Logical 4-bit weight values as an int16 tensor [N, K].

    INT4 values are uniform in [-8, 7]; UINT4 values uniform in [0, 15].
    ``lo``/``hi`` (inclusive) narrow the range when a test needs it.
    """
    g = _gen(seed)
    if wtype == "int4":
        lo = -8 if lo is None else lo
        hi = 7 if hi is None else hi
    elif wtype in ("uint4", "uint4b8"):
        lo = 0 if lo is None else lo
        hi = 15 if hi is None else hi
    else:
        raise ValueError(wtype)
    return torch.randint(lo, hi + 1, (N, K), generator=g, dtype=torch.int16)


def store_nibbles(values: torch.Tensor) -> torch.Tensor:
    """Store logical 4-bit values [N, K] as the [N, K/2] byte array.

    Storage only: the low 4 bits of each value are kept (two's complement for
    negative INT4 values); even k goes to the low nibble.
    """
    N, K = values.shape
    if K % 2:
        raise ValueError("K must be even")
    nib = (values.to(torch.int32) & 0xF).to(torch.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()


def scales(shape, dtype: str, seed: int, lo: float = 0.005, hi: float = 0.02) -> torch.Tensor:
    """Scales ~U(lo, hi) drawn in fp32 and stored in ``dtype``."""
    g = _gen(seed)
    s = torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo
    return s.to(TORCH_DTYPES[dtype]).contiguous()


def zero_points(shape, dtype: str, seed: int) -> torch.Tensor:
    """Integer zero-points uniform in [0, 15] stored in ``dtype``."""
    g = _gen(seed)
    z = torch.randint(0, 16, shape, generator=g, dtype=torch.int32).to(torch.float32)
    return z.to(TORCH_DTYPES[dtype]).contiguous()


def bias(N: int, dtype: str, seed: int) -> torch.Tensor:
    g = _gen(seed)
    return (torch.randn((N,), generator=g) * 0.5).to(TORCH_DTYPES[dtype]).contiguous()


@dataclasses.dataclass
class Case:
    """One GEMM problem instance (CPU tensors)."""
    wl: Workload
    M: int
    a: torch.Tensor              # [M, K] activations (f16/bf16)
    w_values: torch.Tensor       # [N, K] int16 logical values (for reference only)
    w_logical: torch.Tensor      # [N, K/2] uint8
    w_scales: torch.Tensor       # [N] or [N, K/G]
    zeros: Optional[torch.Tensor]
    bias: Optional[torch.Tensor]


def seed_for(name: str, M: int, part: int) -> int:
    """Deterministic seed per (workload, M, input part)."""
    h = 0
    for ch in name:
        h = (h * 131 + ord(ch)) % 1_000_003
    return h * 100_000 + M * 10 + part


def make_case(wl: Workload, M: int, with_bias: bool = False, seed_base: Optional[int] = None,
              N: Optional[int] = None, K: Optional[int] = None, a_dist: str = "normal") -> Case:
    """Build the seeded inputs of ``wl`` at row count ``M``.

    ``N``/``K`` override the workload's shape (used for reduced test sizes
    that keep the workload's dtypes and distributions).
    """
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    gs = K if wl.group_size == wl.K else wl.group_size

    def sd(part):
        return seed_for(wl.name, M, part) if seed_base is None else seed_base * 10 + part

    a = activations(M, K, wl.a_dtype, sd(0), dist=a_dist)
    wv = int4_codes(N, K, wl.wtype, sd(1))
    wlog = store_nibbles(wv)
    if wl.kind == "w4a8" and gs == K:
        ws = scales((N,), wl.s_dtype, sd(2))
    else:
        ws = scales((N, K // gs), wl.s_dtype, sd(2))
    zp = zero_points((N, K // gs), wl.a_dtype, sd(3)) if wl.has_zeros else None
    b = bias(N, wl.out_dtype, sd(4)) if with_bias else None
    return Case(wl, M, a, wv, wlog, ws, zp, b)


def weight_copy(w_logical: torch.Tensor, i: int) -> torch.Tensor:
    """A distinct weight with the same distribution: every stored byte XOR-ed
    with a per-copy constant (a bijection on each 4-bit code).  Used to rotate
    several resident weight copies through a benchmark so that no launch finds
    its weight in a cache.  Works on CPU or device tensors."""
    if i == 0:
        return w_logical
    return w_logical ^ ((i * 0x37 + 0x5A) & 0xFF)
