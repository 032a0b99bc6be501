"""GPU parity of the schedules the built-in schedule table selects: every
entry at both ends of its M range, on sampled rows and columns against the
oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
import workloads
from oracle import w4_oracle as O
from tests.parity import DEV, assert_w4a8, assert_w4a16, bits16
from tests.schedule_table import builtin_schedule_entries

pytestmark = pytest.mark.gpu

ENTRIES = builtin_schedule_entries()


def _workload(a_dtype, grouped):
    if a_dtype == w4.I8:
        return workloads.WORKLOADS["w4a8_i8_g128_o" if grouped else "w4a8_i8_pc_8192x21760"]
    if a_dtype == w4.FP8_E4M3 and grouped:
        return workloads.WORKLOADS["w4a8_fp8_g128_28672x8192"]
    if a_dtype in (w4.BF16, w4.F16):
        # the W4A16 workload's dtypes and distributions (converted to fp16 and
        # to one group per row below where the entry asks for them)
        return workloads.WORKLOADS["w4a16_bf16_g128_4096x4096"]
    raise AssertionError(f"no workload for a_dtype={a_dtype} grouped={grouped}")


def _sample(n, k, rng, must):
    extra = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([np.asarray(must), extra]))


@pytest.mark.parametrize("entry", ENTRIES, ids=lambda e: f"{e[0]}-{e[1]}-{e[2]}x{e[3]}-M{e[4]}..{e[5]}")
def test_table_schedule_parity(entry):
    a_dtype, grouped, N, K, m_lo, m_hi, path, splitk, tile_m, strips = entry
    wl = _workload(a_dtype, grouped)
    case = workloads.make_case(wl, m_hi, N=N, K=K, seed_base=N + K + m_hi)
    gs = 128 if grouped else -1
    G = K // 128 if grouped else 1
    rng = np.random.default_rng(m_hi)
    cols = _sample(N, 48, rng, must=(0, 15, 16, N - 1))
    packed = w4.prepack_B(case.w_logical.to(DEV), "i8" if wl.kind == "w4a8" else "f16")
    for M in sorted({m_lo, m_hi}):
        plan = w4.gemm_plan(M, N, K, gs, a_dtype)
        assert plan[0] == path and (splitk == 0 or plan[1] == splitk)
        rows = _sample(M, 8, rng, must=(0, M - 1))
        a = case.a[:M].contiguous()
        if wl.kind == "w4a8":
            aq, sa = w4.quant_act_per_token(a.to(DEV), wl.q_dtype)
            out_dt = torch.float16 if wl.out_dtype == "f16" else torch.bfloat16
            out = w4.w4a8_gemm(aq, sa, packed, case.w_scales.to(DEV), gs, out_dt)
            codes, sa_o = O.quant_act_per_token(bits16(a[rows]), wl.a_dtype, wl.q_dtype)
            sd = wl.s_dtype
            s_np = case.w_scales.numpy() if sd == "f32" else bits16(case.w_scales)
            ref = O.w4a8_gemm(codes, wl.q_dtype, sa_o, case.w_logical.numpy(), K, wl.wtype, s_np, sd,
                              K if gs == -1 else gs, wl.out_dtype, cols=cols)
            sub = out.cpu()[torch.as_tensor(rows)][:, torch.as_tensor(cols)]
            assert_w4a8(sub, ref, wl.out_dtype, wl.q_dtype, G, label=f"{entry} M={M}")
        else:
            dt, dname = (torch.float16, "f16") if a_dtype == w4.F16 else (torch.bfloat16, "bf16")
            gsz = 128 if grouped else K
            a16 = a.float().to(dt)
            s16 = case.w_scales.float()[:, :K // gsz].contiguous().to(dt)
            z16 = case.zeros.float()[:, :K // gsz].contiguous().to(dt)
            out = w4.w4a16_gemm(a16.to(DEV), packed, s16.to(DEV), z16.to(DEV), gsz if grouped else -1)
            ref = O.w4a16_gemm(bits16(a16), dname, case.w_logical.numpy(), K, wl.wtype,
                               bits16(s16), bits16(z16), gsz, rows=rows, cols=cols)
            sub = out.cpu()[torch.as_tensor(rows)][:, torch.as_tensor(cols)]
            assert_w4a16(sub, ref, dname, label=f"{entry} M={M}")
