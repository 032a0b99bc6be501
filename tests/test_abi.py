"""Host-side tests of the C ABI (CPU only: no kernel is launched).

The library must load, export every function that include/w4.h declares,
and reject invalid arguments on the host with the documented status before
enqueueing anything.
"""
import ctypes
import os
import re

import pytest

import mixed_precision_quantized_prepack_amd as w4
from tests.schedule_table import builtin_schedule_entries

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")

W4_OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_GROUP, E_WS, E_UNSUP = 0, 1, 2, 3, 4, 5, 6, 7
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced by validation
MISALIGNED = ctypes.c_void_p(0x10008)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        pytest.skip("libw4.so not built")
    return w4.lib()


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"^W4_API\s+[\w\s\*]+?\b(w4\w*)\s*\(", text, flags=re.M)


def test_header_declares_the_documented_entry_points():
    names = header_functions()
    for n in ("w4_prepack_B", "w4_quant_act_per_token", "w4_quant_act_per_tensor", "w4_rmsnorm_quant_per_token",
              "w4a8_gemm", "w4a16_gemm"):
        assert n in names
    assert sorted(names) == sorted(w4.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_only_the_abi_is_exported(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert text_syms == set(header_functions())


def test_versions_and_status_strings(lib):
    assert lib.w4_abi_version() == 1
    assert lib.w4_layout_version() == 1
    for s in range(9):
        assert lib.w4_status_string(s).decode().startswith("W4_")
    assert lib.w4_prepack_B_bytes(256, 512) == 256 * 512 // 2


def test_prepack_validation(lib):
    assert lib.w4_prepack_B(None, FAKE, 16, 128, 0, None) == E_NULL
    assert lib.w4_prepack_B(FAKE, ctypes.c_void_p(0x90000), 24, 128, 0, None) == E_SHAPE
    assert lib.w4_prepack_B(FAKE, ctypes.c_void_p(0x90000), 16, 100, 0, None) == E_SHAPE
    assert lib.w4_prepack_B(FAKE, ctypes.c_void_p(0x90000), 16, 128, 7, None) == E_DTYPE
    assert lib.w4_prepack_B(MISALIGNED, ctypes.c_void_p(0x90000), 16, 128, 0, None) == E_ALIGN
    # overlapping input and output
    assert lib.w4_prepack_B(FAKE, ctypes.c_void_p(0x10010), 16, 128, 0, None) == E_SHAPE
    assert "overlap" in lib.w4_last_error().decode()


def test_prepack_from_exllama_validation(lib):
    f = lib.w4_prepack_B_from_exllama
    assert f(None, FAKE, 16, 128, 0, None) == E_NULL
    assert f(FAKE, ctypes.c_void_p(0x90000), 24, 128, 0, None) == E_SHAPE
    assert f(FAKE, ctypes.c_void_p(0x90000), 16, 128, 9, None) == E_DTYPE
    assert f(MISALIGNED, ctypes.c_void_p(0x90000), 16, 128, 0, None) == E_ALIGN
    assert f(FAKE, ctypes.c_void_p(0x10010), 16, 128, 0, None) == E_SHAPE       # overlap
    assert f(FAKE, ctypes.c_void_p(0x90000), 1 << 22, 1 << 22, 0, None) == E_SHAPE   # 2^44 elements


def test_quant_validation(lib):
    q = lib.w4_quant_act_per_token
    assert q(FAKE, 7, FAKE, 3, FAKE, 4, 64, None) == E_DTYPE
    assert q(FAKE, 0, FAKE, 5, FAKE, 4, 64, None) == E_DTYPE
    assert q(FAKE, 0, FAKE, 3, FAKE, 4, 60, None) == E_SHAPE
    assert q(FAKE, 0, FAKE, 3, FAKE, -1, 64, None) == E_SHAPE
    assert q(None, 0, FAKE, 3, FAKE, 4, 64, None) == E_NULL
    assert q(MISALIGNED, 0, FAKE, 3, FAKE, 4, 64, None) == E_ALIGN
    assert q(None, 0, None, 3, None, 0, 64, None) == W4_OK        # M = 0: nothing to do


def test_quant_per_tensor_validation(lib):
    q = lib.w4_quant_act_per_tensor
    assert q(FAKE, 7, FAKE, 3, FAKE, 4, 64, None) == E_DTYPE
    assert q(FAKE, 0, FAKE, 5, FAKE, 4, 64, None) == E_DTYPE
    assert q(FAKE, 0, FAKE, 3, FAKE, 4, 60, None) == E_SHAPE
    assert q(FAKE, 0, FAKE, 3, FAKE, -1, 64, None) == E_SHAPE
    assert q(FAKE, 0, None, 3, FAKE, 4, 64, None) == E_NULL
    assert q(FAKE, 0, FAKE, 3, ctypes.c_void_p(0x10002), 4, 64, None) == E_ALIGN
    assert q(None, 0, None, 3, None, 0, 64, None) == W4_OK        # M = 0: nothing to do


def test_rmsnorm_quant_validation(lib):
    f = lib.w4_rmsnorm_quant_per_token
    assert f(FAKE, 7, FAKE, 1e-6, FAKE, 3, FAKE, 4, 64, None) == E_DTYPE
    assert f(FAKE, 0, FAKE, 1e-6, FAKE, 5, FAKE, 4, 64, None) == E_DTYPE
    assert f(FAKE, 0, FAKE, 1e-6, FAKE, 3, FAKE, 4, 60, None) == E_SHAPE
    assert f(FAKE, 0, FAKE, 0.0, FAKE, 3, FAKE, 4, 64, None) == E_SHAPE
    assert f(FAKE, 0, FAKE, -1.0, FAKE, 3, FAKE, 4, 64, None) == E_SHAPE
    assert f(FAKE, 0, FAKE, float("nan"), FAKE, 3, FAKE, 4, 64, None) == E_SHAPE
    assert f(FAKE, 0, FAKE, float("inf"), FAKE, 3, FAKE, 4, 64, None) == E_SHAPE
    assert f(FAKE, 0, None, 1e-6, FAKE, 3, FAKE, 4, 64, None) == E_NULL
    assert f(FAKE, 0, MISALIGNED, 1e-6, FAKE, 3, FAKE, 4, 64, None) == E_ALIGN
    assert f(None, 0, None, 1e-6, None, 3, None, 0, 64, None) == W4_OK      # M = 0: nothing to do


def _w4a8(lib, aq=FAKE, a_dtype=3, a_scales=FAKE, b=FAKE, wtype=0, bs=FAKE, s_dtype=2, gs=128,
          bias=None, out=FAKE, out_dtype=0, M=4, N=32, K=256, ws=None, wsb=0):
    return lib.w4a8_gemm(aq, a_dtype, a_scales, b, wtype, bs, s_dtype, gs, bias, out, out_dtype,
                         M, N, K, ws, wsb, None)


def test_w4a8_validation(lib):
    assert _w4a8(lib, a_dtype=0) == E_DTYPE
    assert _w4a8(lib, wtype=1) == E_DTYPE              # unsigned without zero-points
    assert _w4a8(lib, s_dtype=3) == E_DTYPE
    assert _w4a8(lib, out_dtype=2) == E_DTYPE
    assert _w4a8(lib, N=40) == E_SHAPE
    assert _w4a8(lib, K=200) == E_SHAPE
    assert _w4a8(lib, M=-2) == E_SHAPE
    assert _w4a8(lib, gs=64) == E_GROUP
    assert _w4a8(lib, K=384, gs=256) == E_GROUP
    assert _w4a8(lib, aq=None) == E_NULL
    assert _w4a8(lib, b=None) == E_NULL
    assert _w4a8(lib, out=None) == E_NULL
    assert _w4a8(lib, a_scales=None) == E_NULL
    assert _w4a8(lib, aq=MISALIGNED) == E_ALIGN
    assert _w4a8(lib, out=MISALIGNED) == E_ALIGN
    assert _w4a8(lib, K=131072 + 128, gs=-1) == E_SHAPE  # int32 range of per-channel int8
    assert _w4a8(lib, M=0) == W4_OK
    assert _w4a8(lib, gs=32) == E_GROUP                 # groups of 64 / 32: W4A16 only


def test_w4a8_no_alloc_validation(lib):
    """Invalid arguments give w4a8_gemm's status; a workspace beyond the
    built-in buffer is refused before anything is enqueued."""
    f = lib.w4a8_gemm_no_alloc

    def call(aq=FAKE, a_dtype=3, sa=FAKE, b=FAKE, wtype=0, bs=FAKE, s_dtype=2, gs=128, bias=None, out=FAKE,
             out_dtype=0, M=4, N=32, K=256):
        return f(aq, a_dtype, sa, b, wtype, bs, s_dtype, gs, bias, out, out_dtype, M, N, K, None)
    assert call(a_dtype=0) == E_DTYPE
    assert call(s_dtype=3) == E_DTYPE
    assert call(out_dtype=2) == E_DTYPE
    assert call(N=40) == E_SHAPE
    assert call(gs=64) == E_GROUP
    assert call(out=None) == E_NULL
    assert call(out=MISALIGNED) == E_ALIGN
    assert call(M=0) == W4_OK
    # the same problems with a split-K plan: validation still comes first
    try:
        w4.set_option("force_path", 2)
        w4.set_option("splitk", 64)
        assert call(s_dtype=3, M=64, N=8192, K=8192, gs=-1) == E_DTYPE
        # 64 splits x 64 x 8192 x 4 bytes = 128 MiB > the 64 MiB buffer
        assert call(M=64, N=8192, K=8192, gs=-1) == E_WS
        assert "64 MiB" in lib.w4_last_error().decode() or "67108864" in lib.w4_last_error().decode()
    finally:
        w4.set_option("force_path", 0)
        w4.set_option("splitk", 0)


def test_w4a16_validation(lib):
    def call(a=FAKE, a_dtype=1, b=FAKE, wtype=1, s=FAKE, z=FAKE, gs=128, out=FAKE, M=2, N=32, K=256):
        return lib.w4a16_gemm(a, a_dtype, b, wtype, s, z, gs, None, out, M, N, K, None, 0, None)
    assert call(a_dtype=3) == E_DTYPE
    assert call(wtype=0) == E_DTYPE
    assert call(wtype=2) == E_DTYPE                      # uint4b8 takes no zero-points
    assert call(s=None) == E_NULL
    assert call(gs=48) == E_GROUP
    assert call(gs=16) == E_GROUP
    assert call(gs=64, K=320) == E_SHAPE                 # K % 128
    assert call(N=8) == E_SHAPE
    assert call(z=ctypes.c_void_p(0x10001)) == E_ALIGN
    assert call(M=0) == W4_OK


def test_w4a8_quant_fused_validation(lib):
    f = lib.w4a8_gemm_quant_fused

    def call(x=FAKE, x_dtype=0, q_dtype=3, b=FAKE, wtype=0, bs=FAKE, s_dtype=2, gs=-1, out=FAKE, out_dtype=0,
             M=1, N=32, K=256, so=None):
        return f(x, x_dtype, q_dtype, b, wtype, bs, s_dtype, gs, None, out, out_dtype, M, N, K, so, None)
    assert call(x_dtype=3) == E_DTYPE
    assert call(q_dtype=0) == E_DTYPE
    assert call(wtype=1) == E_DTYPE
    assert call(b=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(x=MISALIGNED) == E_ALIGN
    assert call(so=ctypes.c_void_p(0x10002)) == E_ALIGN
    assert call(gs=64) == E_GROUP
    assert call(M=17) == E_UNSUP                             # the tiled kernel: no fused quantisation
    assert call(M=16, N=8192, K=21760) == E_UNSUP            # 16 x 21760 codes exceed the LDS
    assert call(M=0) == W4_OK


def test_w4a16_prescaled_validation(lib):
    f = lib.w4a16_gemm_prescaled_zeros

    def call(a=FAKE, a_dtype=1, b=FAKE, s=FAKE, z=FAKE, gs=128, out=FAKE, M=2, N=32, K=256):
        return f(a, a_dtype, b, s, z, gs, None, out, M, N, K, None, 0, None)
    assert call(a_dtype=3) == E_DTYPE
    assert call(z=None) == E_NULL
    assert call(s=None) == E_NULL
    assert call(gs=64) == E_GROUP
    assert call(gs=-1) == E_GROUP
    assert call(K=128) == E_GROUP                          # one group: per channel
    assert call(N=8) == E_SHAPE
    assert call(out=MISALIGNED) == E_ALIGN
    assert call(M=0) == W4_OK


def test_w4a8_zp_validation(lib):
    f = lib.w4a8_gemm_zp

    def call(aq=FAKE, sa=FAKE, b=FAKE, bs=FAKE, s_dtype=1, z=FAKE, z_dtype=0, gs=128, out=FAKE, out_dtype=0,
             M=4, N=32, K=256):
        return f(aq, sa, b, bs, s_dtype, z, z_dtype, gs, None, out, out_dtype, M, N, K, None, 0, None)
    assert call(z=None) == E_NULL
    assert call(sa=None) == E_NULL
    assert call(z_dtype=3) == E_DTYPE
    assert call(s_dtype=4) == E_DTYPE
    assert call(out_dtype=2) == E_DTYPE
    assert call(gs=64) == E_GROUP
    assert call(N=40) == E_SHAPE
    assert call(gs=-1, K=65536 + 128) == E_SHAPE           # per-channel int32 range
    assert call(z=ctypes.c_void_p(0x10001)) == E_ALIGN
    assert call(z=ctypes.c_void_p(0x10002), z_dtype=2) == E_ALIGN
    assert call(M=0) == W4_OK


def test_partials_window_validation(lib):
    f = lib.w4a8_gemm_partials
    assert f(FAKE, 3, FAKE, 0, 128, 4, 32, 256, 0, 5, 0, 32, FAKE, None, 0, None) == E_SHAPE
    assert f(FAKE, 3, FAKE, 0, 128, 4, 32, 256, 2, 1, 0, 32, FAKE, None, 0, None) == E_SHAPE
    assert f(FAKE, 3, FAKE, 0, 128, 4, 32, 256, 0, 4, 0, 32, None, None, 0, None) == E_NULL


@pytest.fixture
def heuristic_only(lib):
    """The heuristic alone: the schedule table switched off."""
    w4.set_option("schedule_table", 0)
    try:
        yield
    finally:
        w4.set_option("schedule_table", 1)


def test_plan_choices(lib, heuristic_only):
    """Kernel choice and K split of the heuristic for the int8 per-channel
    8192x21760 sweep on a 256-CU part (the CU count the library assumes
    without a device)."""
    plans = {M: w4.gemm_plan(M, 8192, 21760, -1, w4.I8) for M in (1, 16, 64, 128, 256, 512, 1024, 4096)}
    assert plans[1][0] == plans[16][0] == 1                      # small-M kernel
    assert plans[1][3] == 32                                     # two 16-column strips per wave
    assert plans[64] == (3, 4, 64, 128)                         # streaming kernel, 64 tiles x 4 K splits
    assert plans[128][:2] == (2, 4)                              # tiled: 32 K-split ping-pong tiles are too few
    assert plans[256] == (4, 4, 128, 256)                       # ping-pong, halves splitting K: 64 tiles x 4
    assert plans[512] == (4, 2, 128, 256)                       # ... 128 tiles x 2
    assert w4.gemm_plan(384, 8192, 21760, -1, w4.I8) == (4, 2, 128, 256)     # 96 tiles x 2 (3/4 of the CUs)
    assert w4.gemm_plan(640, 8192, 21760, -1, w4.I8) == (4, 2, 256, 256)    # 96 tiles x 2 (3/4 of the CUs)
    assert w4.gemm_plan(520, 8192, 21760, -1, w4.I8) == (4, 2, 256, 256)
    assert w4.gemm_plan(160, 8192, 21760, -1, w4.I8) == (4, 4, 128, 256)    # 64 K-split tiles x 4
    assert w4.gemm_plan(640, 8192, 8192, -1, w4.I8)[0] == 4
    assert plans[1024] == (4, 2, 256, 256)                      # ping-pong: 128 tiles x 2 K splits
    assert plans[4096] == (4, 1, 256, 256)                      # ping-pong: one 256 x 256 tile per CU
    assert w4.gemm_plan(2048, 8192, 21760, -1, w4.I8) == (4, 1, 256, 256)    # 256 tiles
    assert w4.gemm_plan(2048, 4096, 21760, -1, w4.I8) == (4, 2, 256, 256)   # 128 ping-pong tiles x 2 splits
    assert w4.gemm_plan(1024, 4096, 21760, -1, w4.I8) == (4, 2, 128, 256)   # 64 x 2 < 256: halves split K
    assert w4.gemm_plan(512, 4096, 21760, -1, w4.I8) == (4, 4, 128, 256)    # 64 K-split tiles x 4
    assert w4.gemm_plan(4096, 8192, 21760, 128, w4.I8)[:3] == (2, 1, 128)   # grouped: tiled
    assert w4.gemm_plan(4096, 8192, 21760, -1, w4.FP8_E4M3)[0] == 2
    try:
        w4.set_option("tiled_bm", 256)                               # a 256-row tile forces the ping-pong kernel
        assert w4.gemm_plan(300, 8192, 21760, -1, w4.I8) == (4, 4, 256, 256)    # 64 tiles x 4 K splits
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(300, 8192, 21760, 128, w4.I8)               # grouped: the tiled kernel has no 256 rows
        w4.set_option("force_path", 4)
        w4.set_option("tiled_bm", 128)
        assert w4.gemm_plan(300, 8192, 21760, -1, w4.I8) == (4, 2, 128, 256)    # 96 tiles x 2 K splits
        for bad in ((300, 8192, 21760, 128, w4.I8), (300, 8192, 21760, -1, w4.FP8_E4M3),
                    (300, 8192, 4096, -1, w4.BF16)):
            with pytest.raises(w4.W4Error):
                w4.gemm_plan(*bad)
        w4.set_option("skinny_strips", 2)
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(300, 8192, 21760, -1, w4.I8)
    finally:
        for k in ("tiled_bm", "skinny_strips", "force_path"):
            w4.set_option(k, 0)
    # grouped small M: two strips from M = 8 when N >= 8192, at any M when
    # N >= 16384 or (N >= 8192 and K >= 8192), else one
    assert w4.gemm_plan(1, 12288, 4096, 128, w4.I8)[3] == 16
    assert w4.gemm_plan(8, 12288, 4096, 128, w4.I8)[3] == 32
    assert w4.gemm_plan(1, 22016, 4096, 128, w4.I8)[:2] == (1, 8)  # 4 K blocks x 2 strips per wave
    assert w4.gemm_plan(1, 22016, 4096, 128, w4.I8)[3] == 32
    assert w4.gemm_plan(1, 8192, 8192, 128, w4.BF16)[:2] == (1, 8) and w4.gemm_plan(1, 8192, 8192, 128, w4.BF16)[3] == 32
    assert w4.gemm_plan(16, 22016, 4096, 128, w4.I8)[3] == 32
    assert w4.gemm_plan(16, 4096, 11008, 128, w4.I8)[3] == 16
    # 16 < M <= 64, int8 (grouped: M <= 32): the streaming kernel, 32- or
    # 64-row tiles of 128 columns, K split to one workgroup per CU
    assert w4.gemm_plan(32, 4096, 11008, 128, w4.I8) == (3, 8, 32, 128)       # 32 tiles, 86 K blocks
    assert w4.gemm_plan(32, 4096, 4096, 128, w4.I8) == (3, 8, 32, 128)
    assert w4.gemm_plan(64, 8192, 21760, -1, w4.I8) == (3, 4, 64, 128)        # 64 tiles
    assert w4.gemm_plan(48, 8192, 21760, -1, w4.I8) == (3, 4, 64, 128)
    assert w4.gemm_plan(32, 8192, 21760, -1, w4.I8) == (3, 4, 32, 128)
    # ... whose grouped K range must fit the scale table (64 groups of 128-column tiles)
    assert w4.gemm_plan(32, 28672, 16384, 128, w4.I8) == (3, 2, 32, 128)      # 224 tiles
    # more 32-row tiles than CUs: 64-row tiles; more 64-row tiles than CUs: tiled
    assert w4.gemm_plan(64, 65536, 8192, -1, w4.I8)[0] == 2
    # grouped above M = 32: the tiled kernel's 64 x 128 tiles
    assert w4.gemm_plan(64, 12288, 4096, 128, w4.I8) == (2, 2, 64, 128)       # 96 tiles
    assert w4.gemm_plan(64, 22016, 4096, 128, w4.I8) == (2, 1, 64, 128)       # 172 tiles
    assert w4.gemm_plan(64, 4096, 11008, 128, w4.I8) == (2, 8, 64, 128)       # 32 tiles, long K
    # fp8 stays on the tiled kernel
    assert w4.gemm_plan(32, 28672, 8192, 128, w4.FP8_E4M3)[0] == 2
    # grouped int8 and fp8: 128 x 128 tiles once there is one per CU, else 64 x 256;
    # grouped int8 with K <= 8192 takes 64 x 128 tiles while they number at most 3 per CU
    assert w4.gemm_plan(1024, 22016, 4096, 128, w4.I8)[2:] == (128, 128)      # 2752 narrow tiles
    assert w4.gemm_plan(128, 22016, 4096, 128, w4.I8)[2:] == (64, 128)        # 344
    assert w4.gemm_plan(512, 12288, 4096, 128, w4.I8) == (2, 1, 64, 128)      # 768
    assert w4.gemm_plan(1024, 12288, 4096, 128, w4.I8)[2:] == (128, 128)      # 1536
    assert w4.gemm_plan(256, 4096, 4096, 128, w4.I8) == (2, 2, 64, 128)       # 128: two K splits
    assert w4.gemm_plan(256, 4096, 11008, 128, w4.I8)[2:] == (64, 256)        # K > 8192
    assert w4.gemm_plan(256, 28672, 8192, 128, w4.FP8_E4M3)[2:] == (128, 128)
    assert w4.gemm_plan(8192, 28672, 8192, 128, w4.FP8_E4M3)[1:] == (1, 128, 128)
    # grouped fp8: the tall tile from M = 128 (half a workgroup per CU), the
    # most K splits that fit two workgroups per CU
    assert w4.gemm_plan(128, 28672, 8192, 128, w4.FP8_E4M3)[1:] == (2, 128, 128)
    assert w4.gemm_plan(256, 28672, 8192, 128, w4.FP8_E4M3)[1:] == (1, 128, 128)
    # the tiled kernel's K splits at M <= 64 (forced): grouped int8 takes the
    # most that keep one workgroup per CU (at least 4 K blocks each)
    try:
        w4.set_option("force_path", 2)
        assert w4.gemm_plan(64, 12288, 4096, 128, w4.I8) == (2, 2, 64, 128)   # 96 tiles
        assert w4.gemm_plan(32, 4096, 11008, 128, w4.I8) == (2, 8, 64, 128)   # 32 tiles, 86 K blocks
        assert w4.gemm_plan(32, 28672, 8192, 128, w4.FP8_E4M3)[2:] == (64, 256)
        assert w4.gemm_plan(64, 28672, 8192, 128, w4.FP8_E4M3)[1:] == (4, 64, 256)
        assert w4.gemm_plan(64, 8192, 21760, -1, w4.I8)[1] == 8
    finally:
        w4.set_option("force_path", 0)
    assert w4.gemm_plan(128, 22016, 4096, 128, w4.I8)[1] == 1         # 172 tiles
    # int8 workspace: large enough for the asymmetric GEMM's (tiled) plan too
    assert w4.gemm_workspace_bytes(64, 8192, 21760, -1, w4.I8) >= 8 * 64 * 8192 * 4
    # a grouped K whose LDS scale table would not fit the small-M kernel: tiled
    assert w4.gemm_plan(1, 8192, 131072, 128, w4.I8)[0] == 2
    try:
        w4.set_option("force_path", 1)
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(1, 8192, 131072, 128, w4.I8)
    finally:
        w4.set_option("force_path", 0)


def test_options_and_plans(lib, heuristic_only):
    try:
        assert lib.w4_set_option(b"nonsense", 1) == E_UNSUP
        assert lib.w4_set_option(b"force_path", 5) == E_SHAPE
        assert lib.w4_set_option(b"force_path", 4) == W4_OK
        w4.set_option("force_path", 0)
        assert w4.gemm_plan(1, 8192, 21760, -1, w4.I8)[0] == 1     # small M -> skinny
        assert w4.gemm_plan(100, 8192, 21760, -1, w4.I8)[0] == 2   # larger M -> tiled
        assert w4.gemm_plan(4096, 8192, 21760, -1, w4.I8)[0] == 4  # ... ping-pong once its tiles fill 3/4 of the CUs
        assert lib.w4_set_option(b"norm_exact_sum", 2) == E_SHAPE
        w4.set_option("norm_exact_sum", 1)
        assert w4.get_option("norm_exact_sum") == 1
        w4.set_option("norm_exact_sum", 0)
        w4.set_option("force_path", 1)
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(64, 8192, 21760, -1, w4.I8)               # skinny handles M <= 16
        w4.set_option("force_path", 2)
        assert w4.gemm_plan(1, 8192, 21760, -1, w4.I8)[0] == 2
        w4.set_option("splitk", 4)
        assert w4.gemm_plan(1, 8192, 21760, -1, w4.I8)[:2] == (2, 4)
        assert w4.gemm_workspace_bytes(1, 8192, 21760, -1, w4.I8) == 4 * 1 * 8192 * 4
        # a split-K tiled plan needs its workspace
        assert _w4a8(lib, M=1, N=8192, K=21760, gs=-1, s_dtype=2) == E_WS
        # tiled column blocks per wave: 2 (128 columns) or 4 (256); 128 x 256
        # tiles for symmetric int8 per channel only; 16-bit tiles are 64 x 128
        w4.set_option("skinny_strips", 2)
        w4.set_option("tiled_bm", 64)
        assert w4.gemm_plan(100, 8192, 21760, -1, w4.I8) == (2, 4, 64, 128)
        assert w4.gemm_plan(100, 4096, 4096, 128, w4.FP8_E4M3) == (2, 4, 64, 128)
        assert w4.gemm_plan(100, 4096, 4096, 128, w4.BF16)[2:] == (64, 128)
        w4.set_option("skinny_strips", 4)
        assert w4.gemm_plan(100, 4096, 4096, 128, w4.I8)[2:] == (64, 256)
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(100, 4096, 4096, 128, w4.BF16)
        w4.set_option("tiled_bm", 128)
        assert w4.gemm_plan(200, 8192, 21760, -1, w4.I8)[2:] == (128, 256)
        with pytest.raises(w4.W4Error):
            w4.gemm_plan(200, 4096, 4096, 128, w4.I8)
    finally:
        for k in ("force_path", "splitk", "skinny_strips", "tiled_bm"):
            w4.set_option(k, 0)
    assert w4.get_option("force_path") == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        w4.quant_act_per_token(x)


def test_schedule_add_validation(lib):
    f = lib.w4_schedule_add
    assert f(9, 0, 8192, 21760, 1, 16, 1, 2, 0, 0) == E_DTYPE
    assert f(3, 2, 8192, 21760, 1, 16, 1, 2, 0, 0) == E_SHAPE         # group mode
    assert f(3, 0, 8192, 21760, 17, 16, 2, 2, 0, 0) == E_SHAPE        # m_hi < m_lo
    assert f(3, 0, 8192, 21760, 1, 64, 1, 2, 0, 0) == E_SHAPE         # small-M kernel above M = 16
    assert f(3, 0, 8192, 21760, 1, 16, 5, 2, 0, 0) == E_SHAPE         # paths 0..4
    assert f(3, 0, 8192, 21760, 1, 16, 2, 65, 0, 0) == E_SHAPE
    assert f(3, 0, 8192, 21760, 1, 16, 2, 2, 96, 0) == E_SHAPE
    assert f(3, 0, 8192, 21760, 1, 16, 1, 2, 0, 3) == E_SHAPE


def test_schedule_table_lookup(lib):
    try:
        w4.schedule_clear()
        base = {M: w4.gemm_plan(M, 8192, 21760, -1, w4.I8) for M in (8, 16, 17, 64)}
        w4.schedule_add(w4.I8, False, 8192, 21760, 9, 16, path=2, splitk=4, tile_m=64)
        assert w4.gemm_plan(16, 8192, 21760, -1, w4.I8) == (2, 4, 64, 256)
        assert w4.gemm_plan(9, 8192, 21760, -1, w4.I8)[:2] == (2, 4)
        assert w4.gemm_workspace_bytes(16, 8192, 21760, -1, w4.I8) == 4 * 16 * 8192 * 4
        # outside the M range, another N or grouping, or another dtype: unchanged
        assert w4.gemm_plan(8, 8192, 21760, -1, w4.I8) == base[8]
        assert w4.gemm_plan(17, 8192, 21760, -1, w4.I8) == base[17]
        assert w4.gemm_plan(16, 8192, 21760, -1, w4.FP8_E4M3)[0] == 1
        # a newer entry for the same problems wins; fields left at 0 go to the heuristic
        w4.schedule_add(w4.I8, False, 8192, 21760, 16, 16, path=1, splitk=0, strips=1)
        p16 = w4.gemm_plan(16, 8192, 21760, -1, w4.I8)
        assert p16[0] == 1 and p16[3] == 16
        # the options force their fields and skip the table
        w4.set_option("splitk", 2)
        assert w4.gemm_plan(9, 8192, 21760, -1, w4.I8)[:2] == (1, 2)
        w4.set_option("splitk", 0)
        # schedule_table = 0: heuristic alone
        w4.set_option("schedule_table", 0)
        assert w4.gemm_plan(16, 8192, 21760, -1, w4.I8) == base[16]
        w4.set_option("schedule_table", 1)
        # an entry that does not fit the problem (K split above K/128) is passed over
        w4.schedule_add(w4.I8, False, 8192, 21760, 64, 64, path=2, splitk=64)
        assert w4.gemm_plan(64, 8192, 21760, -1, w4.I8)[1] <= 21760 // 128
        w4.schedule_add(w4.I8, True, 4096, 256, 64, 64, path=2, splitk=8)
        assert w4.gemm_plan(64, 4096, 256, 128, w4.I8)[1] <= 2
        w4.schedule_clear()
        assert {M: w4.gemm_plan(M, 8192, 21760, -1, w4.I8) for M in (8, 16, 17, 64)} == base
    finally:
        w4.set_option("splitk", 0)
        w4.set_option("schedule_table", 1)
        w4.schedule_clear()


def test_builtin_schedule_entries_fit_their_problems(lib):
    """Every built-in entry is taken at both ends of its M range (none is
    passed over for not fitting)."""
    w4.schedule_clear()
    for a_dtype, grouped, N, K, m_lo, m_hi, path, splitk, tile_m, strips in builtin_schedule_entries():
        gs = 128 if grouped else -1
        for M in (m_lo, m_hi):
            p = w4.gemm_plan(M, N, K, gs, a_dtype)
            assert p[0] == path and (splitk == 0 or p[1] == splitk), (N, K, M)
            if path in (2, 3) and tile_m:
                assert p[2] == tile_m, (N, K, M)
            if path == 1 and strips:
                assert p[3] == 16 * strips, (N, K, M)
            if path in (2, 3) and strips:
                assert p[3] == 64 * strips, (N, K, M)
