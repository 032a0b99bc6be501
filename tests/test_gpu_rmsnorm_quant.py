"""GPU parity: fused RMSNorm + per-token quantisation, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, bits16

pytestmark = pytest.mark.gpu


def _check(x, gamma, eps, x_dtype, q_dtype, rows=None):
    q, s = w4.rmsnorm_quant_per_token(x.to(DEV), gamma.to(DEV), eps, q_dtype)
    q, s = q.cpu().numpy().view(np.uint8), s.cpu().numpy()
    if rows is not None:                  # rows are independent: check a sample
        x, q, s = x[rows], q[rows], s[rows]
    qo, so, _ = O.rmsnorm_quant_per_token(bits16(x), x_dtype, bits16(gamma), eps, q_dtype)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q, qo.view(np.uint8))


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
@pytest.mark.parametrize("M,K,dist,eps", [
    (1, 128, "normal", 1e-6), (3, 4096, "normal", 1e-5), (16, 512, "wide", 1e-6), (5, 8, "normal", 0.5),
    (37, 21760, "normal", 1e-6),          # 1024-thread rows, all in registers
    (600, 4096, "wide", 1e-5),            # 256-thread rows
    (7, 40000, "normal", 1e-6),           # 1024 threads, tail re-read
    (520, 30000, "normal", 1e-6),         # 256 threads, 12 chunks per thread, tail re-read
    (2, 100000, "wide", 1e-6)])
def test_rmsnorm_quant_bit_exact(x_dtype, q_dtype, M, K, dist, eps):
    x = workloads.activations(M, K, x_dtype, seed=M * 17 + K, dist=dist)
    if M >= 3:
        x[1] = 0                          # a zero row: scale 0, codes 0
        x[2, :K // 2] = 0
    gamma = workloads.norm_weight(K, x_dtype, seed=K)
    _check(x, gamma, eps, x_dtype, q_dtype)


@pytest.mark.parametrize("x_dtype,q_dtype", [("f16", "fp8"), ("bf16", "i8")])
@pytest.mark.parametrize("M,K,dist", [(16, 512, "wide"), (37, 21760, "normal"), (600, 4096, "wide"),
                                      (7, 40000, "normal"), (520, 30000, "normal")])
def test_rmsnorm_quant_exact_sum_path(x_dtype, q_dtype, M, K, dist):
    """The path that re-sums the squares exactly (taken when the fast sum
    cannot decide r), forced for every row: same results."""
    x = workloads.activations(M, K, x_dtype, seed=M * 13 + K, dist=dist)
    gamma = workloads.norm_weight(K, x_dtype, seed=K + 1)
    try:
        w4.set_option("norm_exact_sum", 1)
        _check(x, gamma, 1e-6, x_dtype, q_dtype)
    finally:
        w4.set_option("norm_exact_sum", 0)


@pytest.mark.parametrize("M,K,x_dtype,q_dtype", [(4096, 21760, "f16", "i8"), (8192, 8192, "bf16", "fp8"),
                                                 (1024, 11008, "f16", "i8")])
def test_rmsnorm_quant_full_size_sampled_rows(M, K, x_dtype, q_dtype):
    x = workloads.activations(M, K, x_dtype, seed=98)
    gamma = workloads.norm_weight(K, x_dtype, seed=3)
    rows = np.random.default_rng(M + K).choice(M, size=48, replace=False)
    rows.sort()
    _check(x, gamma, 1e-6, x_dtype, q_dtype, rows=rows)


def test_rmsnorm_quant_matches_the_unfused_pair():
    """The fused call returns what the unfused pair does: the oracle's RMSNorm
    output (in the activation dtype) quantised by the library's quantiser."""
    x = workloads.activations(64, 4096, "bf16", seed=4)
    gamma = workloads.norm_weight(4096, "bf16", seed=5)
    q, s = w4.rmsnorm_quant_per_token(x.to(DEV), gamma.to(DEV), 1e-5, "i8")
    _, _, y = O.rmsnorm_quant_per_token(bits16(x), "bf16", bits16(gamma), 1e-5, "i8")
    y_t = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16)
    q2, s2 = w4.quant_act_per_token(y_t.to(DEV), "i8")
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_rmsnorm_quant_empty_rows_is_a_no_op():
    x = torch.zeros((0, 256), dtype=torch.float16, device=DEV)
    g = torch.ones((256,), dtype=torch.float16, device=DEV)
    q, s = w4.rmsnorm_quant_per_token(x, g, 1e-6)
    assert q.shape == (0, 256) and s.shape == (0,)
