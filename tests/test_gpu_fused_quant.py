"""GPU parity: the W4A8 GEMM with the per-token quantisation fused into the
small-M kernel returns the same bits as the quantisation kernel followed by
the GEMM (and, through them, the oracle's result)."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
from oracle import w4_oracle as O
from tests.parity import DEV, DeviceCase, assert_w4a8, bits16

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def _two_step_and_fused(dc, M, x_dtype, wtype="int4", bias=False):
    x = dc.case.a[:M].to(TD[x_dtype]).contiguous().to(DEV)
    if M > 2:
        x[1] = 0                                          # a zero row: scale 0, codes 0
    packed = w4.prepack_B(dc.w_logical, "i8")
    q_dtype = dc.wl.q_dtype
    out_dt = TD[dc.wl.out_dtype]
    gs = -1 if dc.gs == dc.K else dc.gs
    b = dc.bias if bias else None
    aq, sa = w4.quant_act_per_token(x, q_dtype)
    ref = w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out_dt, wtype=wtype, bias=b)
    s_out = torch.full((M,), -1.0, device=DEV)
    got = w4.w4a8_gemm_quant_fused(x, packed, dc.w_scales, gs, out_dt, q_dtype=q_dtype, wtype=wtype, bias=b,
                                   a_scales_out=s_out)
    return got, ref, s_out, sa, x


@pytest.mark.parametrize("wl,M,x_dtype", [("w4a8_i8_pc_8192x21760", 1, "f16"),
                                          ("w4a8_i8_pc_8192x21760", 1, "bf16"),
                                          ("w4a8_i8_g128_qkv", 1, "f16"), ("w4a8_i8_g128_qkv", 4, "f16"),
                                          ("w4a8_i8_g128_qkv", 7, "bf16"),
                                          ("w4a8_i8_g128_o", 12, "f16"),
                                          ("w4a8_fp8_g128_28672x8192", 1, "bf16"),
                                          ("w4a8_fp8_g128_28672x8192", 3, "f16"),
                                          ("w4a8_i8_pc_256x512", 16, "f16")])
def test_fused_quant_equals_two_step(wl, M, x_dtype):
    dc = DeviceCase(wl, M, with_bias=True)
    got, ref, s_out, sa, _ = _two_step_and_fused(dc, M, x_dtype, bias=True)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(s_out.view(torch.int32), sa.view(torch.int32))


def test_fused_quant_uint4b8_and_oracle():
    dc = DeviceCase("w4a8_i8_g128_o", 5, N=512, K=1024, wtype="uint4b8")
    got, ref, s_out, sa, x = _two_step_and_fused(dc, 5, "f16", wtype="uint4b8")
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    codes, so = O.quant_act_per_token(bits16(x.cpu()), "f16", "i8")
    assert np.array_equal(s_out.cpu().numpy().view(np.uint32), so.view(np.uint32))
    r = dc.oracle_w4a8(codes, so)
    assert_w4a8(got, r, dc.wl.out_dtype, "i8", dc.G, label="fused uint4b8")


def test_fused_quant_outside_its_range_is_refused():
    dc = DeviceCase("w4a8_i8_pc_8192x21760", 16)
    packed = w4.prepack_B(dc.w_logical, "i8")
    x = dc.case.a[:16].to(DEV)
    with pytest.raises(w4.W4Error) as e:      # 16 x 21760 codes do not fit the LDS
        w4.w4a8_gemm_quant_fused(x, packed, dc.w_scales, -1, torch.float16)
    assert e.value.status == 7
    dc2 = DeviceCase("w4a8_i8_g128_o", 20, N=256, K=512)
    with pytest.raises(w4.W4Error):           # M > 16: the tiled kernel
        w4.w4a8_gemm_quant_fused(dc2.a, w4.prepack_B(dc2.w_logical, "i8"), dc2.w_scales, 128, torch.float16)
    empty = torch.zeros((0, 512), dtype=torch.float16, device=DEV)
    out = w4.w4a8_gemm_quant_fused(empty, w4.prepack_B(dc2.w_logical, "i8"), dc2.w_scales, 128, torch.float16)
    assert out.shape == (0, 256)
