"""GPU: the hot path captured in a HIP graph.

Serving loops replay a captured decode step instead of launching each kernel.
The library allocates nothing and issues no memset on its launch path (the
caller passes outputs and workspaces), so per-token quantisation plus the GEMM,
the split-K reduce launch included, can be captured on the caller's stream.
Each case runs the path eagerly, captures it once, then replays it several
times with eager work of its own and a synchronisation between replays; every
replay must return the eager call's bits.  A new input copied into the
captured input buffer must give the eager result for that input, and the last
replay is checked against the oracle as well."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_prepack_amd as w4
from tests.parity import DEV, DeviceCase, assert_w4a8, assert_w4a16, bits16

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _w4a8_step(dc, x, aq, sa, out, ws, packed, gs):
    w4.quant_act_per_token(x, dc.wl.q_dtype, out=aq, scales=sa)
    w4.w4a8_gemm(aq, sa, packed, dc.w_scales, gs, out.dtype, bias=dc.bias, out=out, workspace=ws)


def _w4a16_step(dc, x, out, ws, packed):
    w4.w4a16_gemm(x, packed, dc.w_scales, dc.zeros, dc.gs, bias=dc.bias, out=out, workspace=ws)


def _replays_match(g, out, want, eager_other):
    for r in range(REPLAYS):
        out.fill_(-1)                       # eager work between replays: poison the output
        eager_other()                       # and an eager call of the same kernels
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {r}"


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                              # warm-up on the capture stream (first-call set-up)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("wl,M,N,K,want_path,want_split", [
    ("w4a8_i8_pc_8192x21760", 1, 1024, 4096, 1, 8),       # small-M kernel, K split across waves
    ("w4a8_i8_pc_8192x21760", 12, 1024, 4096, 1, 8),      # small-M, activations staged in LDS
    ("w4a8_fp8_g128_28672x8192", 12, 1024, 2048, 1, 2),   # small-M fp8 g128, staged activations
    ("w4a8_i8_pc_8192x21760", 64, 1024, 4096, 3, 16),     # streaming kernel + split-K reduce
    ("w4a8_i8_pc_8192x21760", 300, 1024, 4096, 2, 8),     # ragged tile rows + reduce
    ("w4a8_i8_g128_o", 130, 2048, 4096, 2, 4),            # grouped int8, tiled 64 x 128 + reduce
    ("w4a8_fp8_g128_28672x8192", 40, 1024, 2048, 2, 4),   # fp8 e4m3 codes, tiled + reduce
    ("w4a8_i8_pc_8192x21760", 1024, 8192, 1024, 4, 2),    # ping-pong kernel + reduce
    ("w4a8_i8_pc_8192x21760", 500, 8192, 1024, 4, 2),     # ping-pong, halves splitting K, + reduce
])
def test_w4a8_path_in_a_graph(wl, M, N, K, want_path, want_split):
    dc = DeviceCase(wl, M, N=N, K=K, with_bias=True, seed_base=71)
    gs = -1 if dc.gs == dc.K else dc.gs
    a_dt = w4.I8 if dc.wl.q_dtype == "i8" else w4.FP8_E4M3
    plan = w4.gemm_plan(M, N, K, gs, a_dt)
    assert plan[:2] == (want_path, want_split), plan
    packed = w4.prepack_B(dc.w_logical, "i8")
    out_dt = torch.float16 if dc.wl.out_dtype == "f16" else torch.bfloat16
    x = dc.a.clone()
    code_dt = torch.int8 if dc.wl.q_dtype == "i8" else torch.uint8
    aq = torch.empty((M, K), dtype=code_dt, device=DEV)
    sa = torch.empty((M,), dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=out_dt, device=DEV)
    ws = torch.empty(max(w4.gemm_workspace_bytes(M, N, K, gs, a_dt), 1), dtype=torch.uint8, device=DEV)
    step = lambda: _w4a8_step(dc, x, aq, sa, out, ws, packed, gs)

    step()
    torch.cuda.synchronize()
    want = out.clone()
    g = _capture(step)

    # eager work between replays: the same kernels on a second input, own buffers
    x_other = torch.flip(x, dims=[1]).contiguous()
    def other():
        q2, s2 = w4.quant_act_per_token(x_other, dc.wl.q_dtype)
        w4.w4a8_gemm(q2, s2, packed, dc.w_scales, gs, out_dt, bias=dc.bias)
    _replays_match(g, out, want, other)

    # a new input in the captured buffer: the replay follows it
    x.copy_(torch.roll(dc.a, shifts=1, dims=0) * 0.5)
    q3, s3 = w4.quant_act_per_token(x, dc.wl.q_dtype)
    want2 = w4.w4a8_gemm(q3, s3, packed, dc.w_scales, gs, out_dt, bias=dc.bias)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want2.view(torch.int16))
    assert torch.equal(aq, q3) and torch.equal(sa.view(torch.int32), s3.view(torch.int32))

    # and the replay's output against the oracle, from the oracle's own codes
    codes, so = _oracle_codes(dc, x)
    assert np.array_equal(so.view(np.uint32), sa.cpu().numpy().view(np.uint32))
    ref = dc.oracle_w4a8(codes, so)
    assert_w4a8(out, ref, dc.wl.out_dtype, dc.wl.q_dtype, dc.G, label=f"graph {wl} M={M}")


def _oracle_codes(dc, x):
    from oracle import w4_oracle as O
    return O.quant_act_per_token(bits16(x.cpu()), dc.wl.a_dtype, dc.wl.q_dtype)


@pytest.mark.parametrize("M,want_path,want_split", [(4, 1, 2), (200, 2, 4)])
def test_w4a16_path_in_a_graph(M, want_path, want_split):
    dc = DeviceCase("w4a16_bf16_g128_4096x4096", M, N=1024, K=2048, with_bias=True, seed_base=72)
    plan = w4.gemm_plan(M, dc.N, dc.K, dc.gs, w4.BF16)
    assert plan[:2] == (want_path, want_split), plan
    packed = w4.prepack_B(dc.w_logical, "f16")
    x = dc.a.clone()
    out = torch.empty((M, dc.N), dtype=x.dtype, device=DEV)
    ws = torch.empty(max(w4.gemm_workspace_bytes(M, dc.N, dc.K, dc.gs, w4.BF16), 1), dtype=torch.uint8,
                     device=DEV)
    step = lambda: _w4a16_step(dc, x, out, ws, packed)

    step()
    torch.cuda.synchronize()
    want = out.clone()
    g = _capture(step)
    x_other = torch.flip(x, dims=[1]).contiguous()
    other = lambda: w4.w4a16_gemm(x_other, packed, dc.w_scales, dc.zeros, dc.gs, bias=dc.bias)
    _replays_match(g, out, want, other)
    ref = dc.oracle_w4a16()
    assert_w4a16(out, ref, dc.wl.a_dtype, label=f"graph w4a16 M={M}")
