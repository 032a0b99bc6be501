"""GPU parity: dynamic per-tensor activation quantisation, bit-exact against
the oracle (codes and the one scale, written to every row)."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, DeviceCase, assert_w4a8, bits16

pytestmark = pytest.mark.gpu


def _check(x, x_dtype, q_dtype):
    q, s = w4.quant_act_per_tensor(x.to(DEV), q_dtype)
    qo, so = O.quant_act_per_tensor(bits16(x), x_dtype, q_dtype)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("q_dtype", ["i8", "fp8"])
@pytest.mark.parametrize("M,K,dist", [(1, 128, "normal"), (3, 4096, "normal"), (16, 512, "wide"),
                                      (5, 8, "normal"), (7, 40000, "normal"), (33, 21760, "wide"),
                                      (520, 30000, "normal"), (2, 100000, "wide")])
def test_quant_per_tensor_bit_exact(x_dtype, q_dtype, M, K, dist):
    x = workloads.activations(M, K, x_dtype, seed=M * 37 + K, dist=dist)
    if M >= 3:
        x[1] = 0                     # a zero row
        x[2] *= 1e-3                 # a row far below the tensor's maximum
    _check(x, x_dtype, q_dtype)


@pytest.mark.parametrize("M", [1025, 70000])
def test_quant_per_tensor_many_rows(M):
    """More rows than the scale reduction's threads: the maximum sits in the
    last row, past the first pass of its loop."""
    x = workloads.activations(M, 64, "f16", seed=M, dist="normal")
    x[-1, 5] = -30.0
    _check(x, "f16", "i8")
    _check(x, "f16", "fp8")


def test_quant_per_tensor_all_zero_and_empty():
    _check(torch.zeros((4, 256), dtype=torch.bfloat16), "bf16", "i8")
    q, s = w4.quant_act_per_tensor(torch.zeros((0, 256), dtype=torch.float16, device=DEV))
    assert q.shape == (0, 256) and s.shape == (0,)


def test_quant_per_tensor_then_per_token_on_the_same_buffers():
    """The row maxima held in the scales between launches leave nothing
    behind: per-token after per-tensor (and back) on the same outputs."""
    x = workloads.activations(64, 1024, "f16", seed=3, dist="wide").to(DEV)
    q = torch.empty((64, 1024), dtype=torch.int8, device=DEV)
    s = torch.empty((64,), dtype=torch.float32, device=DEV)
    for per_tensor in (True, False, True):
        if per_tensor:
            w4.quant_act_per_tensor(x, "i8", out=q, scales=s)
            qo, so = O.quant_act_per_tensor(bits16(x.cpu()), "f16", "i8")
        else:
            w4.quant_act_per_token(x, "i8", out=q, scales=s)
            qo, so = O.quant_act_per_token(bits16(x.cpu()), "f16", "i8")
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("M,K,x_dtype,q_dtype", [(4096, 21760, "f16", "i8"), (2048, 8192, "bf16", "fp8")])
def test_quant_per_tensor_full_size(M, K, x_dtype, q_dtype):
    _check(workloads.activations(M, K, x_dtype, seed=101), x_dtype, q_dtype)


@pytest.mark.parametrize("wl,M", [("w4a8_i8_pc_8192x21760", 16), ("w4a8_fp8_g128_28672x8192", 40)])
def test_per_tensor_codes_feed_the_gemm(wl, M):
    """W4A8 with per-tensor activation scales: the GEMM takes them as one
    scale per row, equal across rows."""
    c = DeviceCase(wl, M)
    q_dtype = c.wl.q_dtype
    aq, sa = w4.quant_act_per_tensor(c.a, q_dtype)
    codes, so = O.quant_act_per_tensor(bits16(c.case.a), c.wl.a_dtype, q_dtype)
    assert np.array_equal(aq.cpu().numpy().view(np.uint8), codes.view(np.uint8))
    packed = w4.prepack_B(c.w_logical, "i8")
    out_dt = torch.float16 if c.wl.out_dtype == "f16" else torch.bfloat16
    gs = -1 if c.gs == c.K else c.gs
    out = w4.w4a8_gemm(aq, sa, packed, c.w_scales, gs, out_dt, wtype=c.wtype, bias=c.bias)
    cols = np.arange(0, c.N, 97)
    ref = c.oracle_w4a8(codes, so, cols=cols)
    assert_w4a8(out.cpu()[:, torch.as_tensor(cols)], ref, c.wl.out_dtype, q_dtype, c.G, label=f"{wl} M={M}")
