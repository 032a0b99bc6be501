"""Properties of the host-side planner over a seeded sweep of problem shapes
(no GPU: the library plans for a 256-CU part without a device).

For every valid (M, N, K, group, activation dtype) the plan must exist and
be consistent with the kernel it names:
* small-M only for M <= 16, with N a multiple of its strip width;
* the streaming kernel only for 8-bit symmetric operands with 16 < M;
* the ping-pong kernel only for int8 per channel, 128 or 256 rows x 256
  columns;
* a K split between 1 and min(64, K / 128) (small-M: waves, at most 16);
* the workspace query covers every split plan's M x N int32 slots, and is 0
  when nothing is split across workgroups;
and, with the schedule table off, the heuristic's plan.
"""
import os
import random

import pytest

import mixed_precision_quantized_prepack_amd as w4

DTYPES = [w4.I8, w4.FP8_E4M3, w4.F16, w4.BF16]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        pytest.skip("libw4.so not built")
    return w4.lib()


def _shapes(n, seed):
    rng = random.Random(seed)
    for _ in range(n):
        M = rng.choice([0, 1, 2, 7, 16, 17, 31, 33, 64, 65, 100, 128, 200, 256, 300, 511, 640, 1000, 1024, 1280,
                        2048, 3000, 4096, 8192])
        N = 16 * rng.randint(1, 2048)
        K = 128 * rng.randint(1, 256)
        dt = rng.choice(DTYPES)
        gs = rng.choice([-1, 128] + ([64, 32] if dt in (w4.F16, w4.BF16) else []))
        if gs > 0 and K % gs:
            gs = -1
        yield M, N, K, gs, dt


@pytest.mark.parametrize("table", [1, 0])
def test_plans_are_consistent(lib, table):
    w4.set_option("schedule_table", table)
    try:
        for M, N, K, gs, dt in _shapes(1500, 7 + table):
            path, split, tm, tn = w4.gemm_plan(M, N, K, gs, dt)
            what = (M, N, K, gs, dt, (path, split, tm, tn))
            KB = K // 128
            eight_bit = dt in (w4.I8, w4.FP8_E4M3)
            grouped = gs != -1 and gs != K
            assert path in (1, 2, 3, 4), what
            if path == 1:
                assert M <= 16 and tm == 16 and tn in (16, 32) and N % tn == 0, what
                assert 1 <= split <= min(16, KB), what
            else:
                assert M > 16 or M == 0 or path == 2, what
                assert 1 <= split <= min(64, KB), what
            if path == 3:
                assert eight_bit and tm in (32, 64, 128) and tn in (128, 256), what
            if path == 4:
                assert dt == w4.I8 and not grouped and tm in (128, 256) and tn == 256, what
            if path == 2:
                assert tm in (32, 64, 128) and tn in (128, 256), what
            ws = w4.gemm_workspace_bytes(M, N, K, gs, dt)
            if path != 1 and split > 1:
                assert ws >= split * M * N * 4, what
            elif dt != w4.I8:
                # int8 also sizes for the asymmetric GEMM's plan, which may split
                assert ws == 0, what
    finally:
        w4.set_option("schedule_table", 1)


def test_plans_reject_invalid_shapes(lib):
    for bad in ((1, 8, 128, -1, w4.I8), (1, 16, 100, -1, w4.I8), (-1, 16, 128, -1, w4.I8),
                (1, 16, 256, 64, w4.I8), (1, 16, 384, 256, w4.F16)):
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(*bad)


def test_plans_reject_shapes_past_32bit_offsets(lib):
    """K above 2^22 (a 256-row tile of K bytes, or 64 rows of K fp16 values,
    must stay within a 2 GiB buffer range), and more than 2^29 - 4 scales."""
    w4.gemm_plan(300, 16, 1 << 22, 128, w4.FP8_E4M3)
    w4.gemm_plan(1, 1 << 16, 1 << 16, 128, w4.I8)            # 2^25 scales
    w4.gemm_plan(1, (1 << 29) - 16, 128, -1, w4.BF16)        # per channel: one scale per column
    for bad in ((300, 16, (1 << 22) + 128, 128, w4.FP8_E4M3), (1, 16, 1 << 23, 128, w4.BF16),
                (1, 1 << 20, 1 << 16, 128, w4.I8), (1, 1 << 18, 1 << 18, 64, w4.F16), (1, 1 << 29, 128, -1, w4.I8)):
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(*bad)
