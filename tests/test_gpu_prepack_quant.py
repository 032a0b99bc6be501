"""GPU parity: weight prepack and per-token quantisation, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, bits16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("operand", ["i8", "f16"])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 640), (1024, 4096)])
def test_prepack_bit_exact(operand, N, K):
    w = workloads.store_nibbles(workloads.int4_codes(N, K, "uint4", seed=N + K))
    got = w4.prepack_B(w.to(DEV), operand).cpu().numpy()
    assert np.array_equal(got, O.prepack_B(w.numpy(), N, K, operand))


@pytest.mark.parametrize("N,K,operand", [(4096, 4096, "f16"), (8192, 21760, "i8"),
                                         (28672, 8192, "i8"), (22016, 4096, "i8")])
def test_prepack_bit_exact_full_size(N, K, operand):
    w = workloads.store_nibbles(workloads.int4_codes(N, K, "uint4", seed=7))
    got = w4.prepack_B(w.to(DEV), operand).cpu().numpy()
    assert np.array_equal(got, O.prepack_B(w.numpy(), N, K, operand))


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
@pytest.mark.parametrize("M,K,dist", [(1, 128, "normal"), (3, 4096, "normal"), (16, 512, "wide"),
                                      (5, 8, "normal"), (7, 40000, "normal"), (33, 21760, "wide"),
                                      (64, 8192, "normal"),
                                      # rows longer than the register-resident chunks: tail pass
                                      (520, 30000, "normal"), (2, 100000, "wide"),
                                      # a few long rows: several workgroups per row, chunk counts
                                      # that do not divide evenly among them
                                      (1, 21760, "normal"), (16, 21760, "wide"), (1, 8192, "normal"),
                                      (40, 8200, "normal"), (17, 9000, "wide")])
def test_quant_bit_exact(x_dtype, q_dtype, M, K, dist):
    x = workloads.activations(M, K, x_dtype, seed=M * 31 + K, dist=dist)
    if M >= 3:
        x[1] = 0                     # a zero row
        x[2, :K // 2] = 0
    q, s = w4.quant_act_per_token(x.to(DEV), q_dtype)
    qo, so = O.quant_act_per_token(bits16(x), x_dtype, q_dtype)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    qg = q.cpu().numpy()
    if q_dtype == "i8":
        assert np.array_equal(qg, qo)
    else:
        assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("M,K,x_dtype,q_dtype", [(4096, 21760, "f16", "i8"), (8192, 8192, "bf16", "fp8"),
                                                 (1024, 11008, "f16", "i8")])
def test_quant_bit_exact_full_size(M, K, x_dtype, q_dtype):
    x = workloads.activations(M, K, x_dtype, seed=99)
    q, s = w4.quant_act_per_token(x.to(DEV), q_dtype)
    qo, so = O.quant_act_per_token(bits16(x), x_dtype, q_dtype)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("M,K", [(2, 21760), (12, 8192), (48, 16392)])
def test_quant_row_maximum_in_any_part(M, K):
    """Rows split over several workgroups: the row maximum placed in the
    first, a middle and the last chunk of different rows; every workgroup
    must code with the same scale."""
    x = workloads.activations(M, K, "f16", seed=M + K)
    for m in range(M):
        pos = [0, K // 2 + 3, K - 1][m % 3]
        x[m, pos] = 60.0 if m % 2 else -60.0
    q, s = w4.quant_act_per_token(x.to(DEV), "i8")
    qo, so = O.quant_act_per_token(bits16(x), "f16", "i8")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)


def test_quant_empty_rows_is_a_no_op():
    x = torch.zeros((0, 256), dtype=torch.float16, device=DEV)
    q, s = w4.quant_act_per_token(x)
    assert q.shape == (0, 256) and s.shape == (0,)


def test_quant_exhaustive_fp16_codes():
    """Every finite fp16 bit pattern goes through the quantiser once, in rows
    whose absolute maxima span the whole range."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(b.view(np.float16))
    vals = b[fin]
    K = 512
    pad = (-vals.size) % K
    vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, K)
    rng = np.random.default_rng(5)
    vals = vals[rng.permutation(vals.shape[0])]
    x = torch.from_numpy(vals.view(np.int16)).view(torch.float16)
    for q_dtype in ("i8", "fp8"):
        q, s = w4.quant_act_per_token(x.to(DEV), q_dtype)
        qo, so = O.quant_act_per_token(vals, "f16", q_dtype)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("operand", ["i8", "f16"])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 640), (4096, 4096), (22016, 4096)])
def test_prepack_from_exllama_bit_exact(operand, N, K):
    g = torch.Generator().manual_seed(N + 3 * K)
    words = torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), generator=g, dtype=torch.int64).to(torch.int32)
    got = w4.prepack_B_from_exllama(words.to(DEV), operand).cpu().numpy()
    assert np.array_equal(got, O.prepack_B_from_exllama(words.numpy(), N, K, operand))


def test_exllama_import_feeds_the_gemm():
    """A W4A16 GEMM on imported words equals the one on the logical weight."""
    N, K, M = 256, 512, 5
    g = torch.Generator().manual_seed(9)
    words = torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), generator=g, dtype=torch.int64).to(torch.int32)
    logical = torch.from_numpy(O.exllama_to_logical(words.numpy(), N, K))
    a = torch.randn((M, K), generator=g).to(torch.bfloat16).to(DEV)
    s = (torch.rand((N, K // 128), generator=g) * 0.01 + 0.005).to(torch.bfloat16).to(DEV)
    z = torch.randint(0, 16, (N, K // 128), generator=g).to(torch.bfloat16).to(DEV)
    p1 = w4.prepack_B_from_exllama(words.to(DEV), "f16")
    p2 = w4.prepack_B(logical.to(DEV), "f16")
    assert torch.equal(p1, p2)
    o1 = w4.w4a16_gemm(a, p1, s, zeros=z, group_size=128)
    o2 = w4.w4a16_gemm(a, p2, s, zeros=z, group_size=128)
    assert torch.equal(o1, o2)
