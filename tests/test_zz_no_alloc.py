"""GPU test of w4a8_gemm_no_alloc, the W4A8 GEMM whose split-K workspace is
the library's built-in per-GPU buffer (for callers that cannot allocate).

Through the C ABI: two calls in a row on the same GPU, the second with a
smaller problem, each against w4a8_gemm with a workspace of its own (the
same kernels and plan, so the same output bits) and against the oracle.
"""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
from tests.parity import DEV, DeviceCase, assert_w4a8, bits16

pytestmark = pytest.mark.gpu


def _run_pair(dc, aq, sa, gs):
    out_dt = torch.float16 if dc.wl.out_dtype == "f16" else torch.bfloat16
    packed = w4.prepack_B(dc.w_logical, "i8")
    ref_out = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out_dt, bias=dc.bias)
    out = torch.full((dc.M, dc.N), float("nan"), dtype=out_dt, device=DEV)
    w4.w4a8_gemm_no_alloc(aq, sa, packed, dc.w_scales, gs, out_dt, bias=dc.bias, out=out)
    torch.cuda.synchronize()
    return out, ref_out


@pytest.mark.parametrize("wl,shapes", [
    ("w4a8_i8_pc_8192x21760", [(64, 1024, 4096), (40, 512, 2048)]),
    ("w4a8_i8_g128_o", [(128, 1024, 2048), (33, 256, 1024)]),
    ("w4a8_fp8_g128_28672x8192", [(96, 512, 2048), (17, 256, 1024)]),
])
def test_no_alloc_matches_w4a8_gemm_twice(wl, shapes):
    for i, (M, N, K) in enumerate(shapes):
        print(f"no_alloc {wl} call {i} M={M} N={N} K={K}", flush=True)
        dc = DeviceCase(wl, M, N=N, K=K, with_bias=(i == 0), seed_base=300 + i)
        gs = -1 if dc.gs == dc.K else dc.gs
        a_dt = w4.I8 if dc.wl.q_dtype == "i8" else w4.FP8_E4M3
        # these shapes take a split-K plan, so the built-in workspace is used
        assert w4.gemm_workspace_bytes(M, N, K, gs, a_dt) > 0
        aq, sa = w4.quant_act_per_token(dc.a, dc.wl.q_dtype)
        out, ref_out = _run_pair(dc, aq, sa, gs)
        assert np.array_equal(bits16(out), bits16(ref_out)), f"call {i}: differs from w4a8_gemm"
        codes, sa_o = dc.oracle_quant()
        assert np.array_equal(aq.cpu().numpy().view(np.uint8), codes.view(np.uint8))
        assert_w4a8(out, dc.oracle_w4a8(codes, sa_o), dc.wl.out_dtype, dc.wl.q_dtype, dc.G,
                    label=f"no_alloc {wl} call {i}")


def test_no_alloc_without_split_and_m0():
    dc = DeviceCase("w4a8_i8_pc_8192x21760", 1, N=512, K=1024, seed_base=9)
    aq, sa = w4.quant_act_per_token(dc.a, "i8")
    out, ref_out = _run_pair(dc, aq, sa, -1)
    assert np.array_equal(bits16(out), bits16(ref_out))
    empty = torch.empty((0, 1024), dtype=torch.int8, device=DEV)
    w4.w4a8_gemm_no_alloc(empty, torch.empty((0,), dtype=torch.float32, device=DEV),
                          w4.prepack_B(dc.w_logical, "i8"), dc.w_scales, -1, torch.float16,
                          out=torch.empty((0, 512), dtype=torch.float16, device=DEV))


def test_no_alloc_refuses_oversized_workspace():
    dc = DeviceCase("w4a8_i8_pc_8192x21760", 64, N=8192, K=8192, seed_base=4)
    aq, sa = w4.quant_act_per_token(dc.a, "i8")
    packed = w4.prepack_B(dc.w_logical, "i8")
    out = torch.zeros((64, 8192), dtype=torch.float16, device=DEV)
    try:
        w4.set_option("force_path", 2)
        w4.set_option("splitk", 64)
        with pytest.raises(w4.W4Error) as ei:
            w4.w4a8_gemm_no_alloc(aq, sa, packed, dc.w_scales, -1, torch.float16, out=out)
        assert ei.value.status == 6          # W4_E_WORKSPACE
    finally:
        w4.set_option("force_path", 0)
        w4.set_option("splitk", 0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0      # nothing was enqueued
