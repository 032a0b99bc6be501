"""Python binding of libw4.so, the gfx950 4-bit-weight mixed-precision GEMM library.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/w4.h``.  PyTorch provides device
memory (outputs and workspaces are allocated as torch tensors) and the
current HIP stream.  There is no fallback: if ``libw4.so`` is missing or a
tensor is not on the GPU, the call raises.

Names follow the C ABI:

    prepack_B(w_logical, operand="i8")                      -> packed weight bytes
    quant_act_per_token(x, q_dtype="i8")                    -> (codes, scales)
    w4a8_gemm(aq, a_scales, b_packed, b_scales, group_size, out_dtype, ...)
    w4a16_gemm(a, b_packed, scales, zeros, group_size, ...)
    w4a8_gemm_partials(...), w4a16_gemm_partials(...)      (verification)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "LIB_PATH", "lib", "W4Error", "prepack_B", "prepack_B_from_exllama", "prepack_B_bytes", "quant_act_per_token",
    "quant_act_per_tensor", "rmsnorm_quant_per_token",
    "w4a8_gemm", "w4a8_gemm_no_alloc", "w4a8_gemm_quant_fused", "w4a8_gemm_zp", "w4a16_gemm", "w4a16_gemm_prescaled_zeros", "w4a8_gemm_partials", "w4a16_gemm_partials",
    "gemm_workspace_bytes", "gemm_plan", "set_option", "get_option", "schedule_add", "schedule_clear",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4.so")

# status codes (w4_status)
W4_OK = 0
# dtypes (w4_dtype)
F16, BF16, F32, I8, FP8_E4M3, I32 = 0, 1, 2, 3, 4, 5
# weight types (w4_wtype)
WTYPES = {"int4": 0, "uint4": 1, "uint4b8": 2}
# operand classes (w4_operand)
OPERANDS = {"i8": 0, "f16": 1}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# (name, restype, argtypes) of every exported function in include/w4.h
_SIGNATURES = [
    ("w4_abi_version", _int, []),
    ("w4_layout_version", _int, []),
    ("w4_status_string", ctypes.c_char_p, [_int]),
    ("w4_last_error", ctypes.c_char_p, []),
    ("w4_prepack_B_bytes", _sz, [_i64, _i64]),
    ("w4_prepack_B", _int, [_vp, _vp, _i64, _i64, _int, _vp]),
    ("w4_prepack_B_from_exllama", _int, [_vp, _vp, _i64, _i64, _int, _vp]),
    ("w4_quant_act_per_token", _int, [_vp, _int, _vp, _int, _vp, _i64, _i64, _vp]),
    ("w4_quant_act_per_tensor", _int, [_vp, _int, _vp, _int, _vp, _i64, _i64, _vp]),
    ("w4_rmsnorm_quant_per_token", _int, [_vp, _int, _vp, ctypes.c_float, _vp, _int, _vp, _i64, _i64, _vp]),
    ("w4_gemm_workspace_bytes", _sz, [_i64, _i64, _i64, _i64, _int]),
    ("w4a8_gemm", _int, [_vp, _int, _vp, _vp, _int, _vp, _int, _i64, _vp, _vp, _int,
                         _i64, _i64, _i64, _vp, _sz, _vp]),
    ("w4a8_gemm_no_alloc", _int, [_vp, _int, _vp, _vp, _int, _vp, _int, _i64, _vp, _vp, _int,
                                  _i64, _i64, _i64, _vp]),
    ("w4a8_gemm_quant_fused", _int, [_vp, _int, _int, _vp, _int, _vp, _int, _i64, _vp, _vp, _int,
                                     _i64, _i64, _i64, _vp, _vp]),
    ("w4a16_gemm_prescaled_zeros", _int, [_vp, _int, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64,
                                          _vp, _sz, _vp]),
    ("w4a8_gemm_zp", _int, [_vp, _vp, _vp, _vp, _int, _vp, _int, _i64, _vp, _vp, _int,
                            _i64, _i64, _i64, _vp, _sz, _vp]),
    ("w4a16_gemm", _int, [_vp, _int, _vp, _int, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64,
                          _vp, _sz, _vp]),
    ("w4a8_gemm_partials", _int, [_vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _i64, _i64, _vp, _vp, _sz, _vp]),
    ("w4a16_gemm_partials", _int, [_vp, _int, _vp, _int, _vp, _i64, _i64, _i64, _i64, _i64,
                                   _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    ("w4_set_option", _int, [ctypes.c_char_p, _i64]),
    ("w4_get_option", _i64, [ctypes.c_char_p]),
    ("w4_schedule_add", _int, [_int, _int, _i64, _i64, _i64, _i64, _int, _int, _int, _int]),
    ("w4_schedule_clear", _int, []),
    ("w4_gemm_plan", _int, [_i64, _i64, _i64, _i64, _int, ctypes.POINTER(_int),
                            ctypes.POINTER(_int), ctypes.POINTER(_int), ctypes.POINTER(_int)]),
]
EXPORTED_SYMBOLS = tuple(n for n, _, _ in _SIGNATURES)

_LIB: Optional[ctypes.CDLL] = None


class W4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status
        self.detail = detail


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libw4.so (once).  Raises if it has not been built.  ``path``
    binds another build of the same ABI instead (tuning experiments), as does
    the W4_LIBRARY environment variable (the host-sanitized build)."""
    global _LIB
    if _LIB is None or path is not None:
        path = path or os.environ.get("W4_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m mixed_precision_quantized_prepack_amd.build`")
        h = ctypes.CDLL(path)
        for name, res, args in _SIGNATURES:
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def _check(fn: str, status: int):
    if status != W4_OK:
        raise W4Error(fn, status, lib().w4_last_error().decode())


def _torch():
    import torch
    return torch


def _dev_ptr(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(dt) -> int:
    torch = _torch()
    m = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32, torch.int8: I8,
         torch.uint8: FP8_E4M3, torch.float8_e4m3fn: FP8_E4M3, torch.int32: I32}
    if dt not in m:
        raise ValueError(f"unsupported dtype {dt}")
    return m[dt]


def _workspace(ws, nbytes: int, device):
    """(pointer, size, tensor) of the split-K workspace.  The caller keeps the
    returned tensor alive until the C call has queued its kernels; after that
    the caching allocator hands the block only to work queued later on the
    same stream, which runs after them."""
    if nbytes == 0:
        return None, 0, None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return _dev_ptr(ws, "workspace"), ws.numel() * ws.element_size(), ws
    t = _torch().empty(nbytes, dtype=_torch().uint8, device=device)
    return _dev_ptr(t, "workspace"), nbytes, t


def prepack_B_bytes(N: int, K: int) -> int:
    return lib().w4_prepack_B_bytes(N, K)


def prepack_B(w_logical, operand: str = "i8", out=None):
    """PB-v1 prepack of a logical [N, K/2] uint8 weight (see include/w4.h)."""
    torch = _torch()
    N, half = w_logical.shape
    K = 2 * half
    if w_logical.dtype != torch.uint8:
        raise ValueError("w_logical must be uint8 [N, K/2]")
    if out is None:
        out = torch.empty(N * K // 2, dtype=torch.uint8, device=w_logical.device)
    _check("w4_prepack_B", lib().w4_prepack_B(_dev_ptr(w_logical, "w_logical"), _dev_ptr(out, "out"),
                                              N, K, OPERANDS[operand], _stream(w_logical)))
    return out


def prepack_B_from_exllama(w_words, operand: str = "f16", out=None):
    """PB-v1 prepack of a weight given as ExLlama-shuffled int32 words
    [N, K/8] (see include/w4.h)."""
    torch = _torch()
    N, k8 = w_words.shape
    K = 8 * k8
    if w_words.dtype not in (torch.int32, torch.uint32):
        raise ValueError("w_words must be int32 [N, K/8]")
    if out is None:
        out = torch.empty(N * K // 2, dtype=torch.uint8, device=w_words.device)
    _check("w4_prepack_B_from_exllama",
           lib().w4_prepack_B_from_exllama(_dev_ptr(w_words, "w_words"), _dev_ptr(out, "out"), N, K,
                                           OPERANDS[operand], _stream(w_words)))
    return out


def quant_act_per_token(x, q_dtype: str = "i8", out=None, scales=None):
    """Per-token int8 / fp8-e4m3 quantisation -> (codes [M, K], scales [M] fp32).

    fp8 codes are returned as raw uint8 bytes (OCP e4m3fn)."""
    torch = _torch()
    M, K = x.shape
    qd = I8 if q_dtype == "i8" else FP8_E4M3
    if out is None:
        out = torch.empty((M, K), dtype=torch.int8 if qd == I8 else torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("w4_quant_act_per_token",
           lib().w4_quant_act_per_token(_dev_ptr(x, "x"), _dtype_code(x.dtype), _dev_ptr(out, "out"),
                                        qd, _dev_ptr(scales, "scales"), M, K, _stream(x)))
    return out, scales


def quant_act_per_tensor(x, q_dtype: str = "i8", out=None, scales=None):
    """Dynamic per-tensor int8 / fp8-e4m3 quantisation -> (codes [M, K],
    scales [M] fp32, every entry the tensor's one scale)."""
    torch = _torch()
    M, K = x.shape
    qd = I8 if q_dtype == "i8" else FP8_E4M3
    if out is None:
        out = torch.empty((M, K), dtype=torch.int8 if qd == I8 else torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("w4_quant_act_per_tensor",
           lib().w4_quant_act_per_tensor(_dev_ptr(x, "x"), _dtype_code(x.dtype), _dev_ptr(out, "out"),
                                         qd, _dev_ptr(scales, "scales"), M, K, _stream(x)))
    return out, scales


def rmsnorm_quant_per_token(x, gamma, eps: float, q_dtype: str = "i8", out=None, scales=None):
    """Fused RMSNorm (weight ``gamma`` [K], output in x's dtype) + per-token
    int8 / fp8-e4m3 quantisation -> (codes [M, K], scales [M] fp32)."""
    torch = _torch()
    M, K = x.shape
    if gamma.dtype != x.dtype or tuple(gamma.shape) != (K,):
        raise ValueError("gamma must be [K] in x's dtype")
    qd = I8 if q_dtype == "i8" else FP8_E4M3
    if out is None:
        out = torch.empty((M, K), dtype=torch.int8 if qd == I8 else torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("w4_rmsnorm_quant_per_token",
           lib().w4_rmsnorm_quant_per_token(_dev_ptr(x, "x"), _dtype_code(x.dtype), _dev_ptr(gamma, "gamma"),
                                            float(eps), _dev_ptr(out, "out"), qd, _dev_ptr(scales, "scales"),
                                            M, K, _stream(x)))
    return out, scales


def gemm_workspace_bytes(M: int, N: int, K: int, group_size: int, a_dtype: int) -> int:
    return lib().w4_gemm_workspace_bytes(M, N, K, group_size, a_dtype)


def gemm_plan(M: int, N: int, K: int, group_size: int, a_dtype: int):
    """(path, k_split, tile_m, tile_n) the GEMM would use; path 1 = small-M, 2 = tiled."""
    p, s, tm, tn = _int(0), _int(0), _int(0), _int(0)
    _check("w4_gemm_plan", lib().w4_gemm_plan(M, N, K, group_size, a_dtype, ctypes.byref(p), ctypes.byref(s),
                                              ctypes.byref(tm), ctypes.byref(tn)))
    return p.value, s.value, tm.value, tn.value


def schedule_add(a_dtype: int, grouped: bool, N: int, K: int, m_lo: int, m_hi: int, path: int = 0,
                 splitk: int = 0, tile_m: int = 0, strips: int = 0) -> None:
    """Register a schedule-table entry (include/w4.h): problems of this
    activation dtype code, grouping, N, K and m_lo <= M <= m_hi take this
    (path, splitk, tile_m, strips); 0 leaves a field to the heuristic."""
    _check("w4_schedule_add", lib().w4_schedule_add(a_dtype, int(bool(grouped)), N, K, m_lo, m_hi, path, splitk,
                                                    tile_m, strips))


def schedule_clear() -> None:
    _check("w4_schedule_clear", lib().w4_schedule_clear())


def set_option(key: str, value: int):
    _check("w4_set_option", lib().w4_set_option(key.encode(), int(value)))


def get_option(key: str) -> int:
    return lib().w4_get_option(key.encode())


def w4a8_gemm(aq, a_scales, b_packed, b_scales, group_size: int, out_dtype, wtype: str = "int4",
              bias=None, out=None, workspace=None):
    """W4A8 GEMM (include/w4.h): aq [M, K] int8 / e4m3 bytes, a_scales [M] fp32,
    b_packed PB-v1 (I8 operand), b_scales [N] or [N, K/G]."""
    torch = _torch()
    M, K = aq.shape
    N = b_scales.shape[0]
    a_dt = I8 if aq.dtype == torch.int8 else FP8_E4M3
    o_dt = _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, a_dt), aq.device)
    _check("w4a8_gemm", lib().w4a8_gemm(
        _dev_ptr(aq, "aq"), a_dt, _dev_ptr(a_scales, "a_scales"), _dev_ptr(b_packed, "b_packed"),
        WTYPES[wtype], _dev_ptr(b_scales, "b_scales"), _dtype_code(b_scales.dtype), group_size,
        _dev_ptr(bias, "bias"), _dev_ptr(out, "out"), o_dt, M, N, K, wsp, wsb, _stream(aq)))
    return out


def w4a8_gemm_no_alloc(aq, a_scales, b_packed, b_scales, group_size: int, out_dtype, wtype: str = "int4",
                       bias=None, out=None):
    """w4a8_gemm whose split-K workspace is the library's built-in per-GPU
    buffer (include/w4.h); ``out`` must be given by callers that cannot
    allocate."""
    torch = _torch()
    M, K = aq.shape
    N = b_scales.shape[0]
    a_dt = I8 if aq.dtype == torch.int8 else FP8_E4M3
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    _check("w4a8_gemm_no_alloc", lib().w4a8_gemm_no_alloc(
        _dev_ptr(aq, "aq"), a_dt, _dev_ptr(a_scales, "a_scales"), _dev_ptr(b_packed, "b_packed"),
        WTYPES[wtype], _dev_ptr(b_scales, "b_scales"), _dtype_code(b_scales.dtype), group_size,
        _dev_ptr(bias, "bias"), _dev_ptr(out, "out"), _dtype_code(out_dtype), M, N, K, _stream(aq)))
    return out


def w4a8_gemm_quant_fused(x, b_packed, b_scales, group_size: int, out_dtype, q_dtype: str = "i8",
                          wtype: str = "int4", bias=None, out=None, a_scales_out=None):
    """W4A8 GEMM of fp16 / bf16 activations with the per-token quantisation
    fused into the small-M kernel (include/w4.h)."""
    torch = _torch()
    M, K = x.shape
    N = b_scales.shape[0]
    qd = I8 if q_dtype == "i8" else FP8_E4M3
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _check("w4a8_gemm_quant_fused", lib().w4a8_gemm_quant_fused(
        _dev_ptr(x, "x"), _dtype_code(x.dtype), qd, _dev_ptr(b_packed, "b_packed"), WTYPES[wtype],
        _dev_ptr(b_scales, "b_scales"), _dtype_code(b_scales.dtype), group_size, _dev_ptr(bias, "bias"),
        _dev_ptr(out, "out"), _dtype_code(out_dtype), M, N, K, _dev_ptr(a_scales_out, "a_scales_out"),
        _stream(x)))
    return out


def w4a8_gemm_zp(aq, a_scales, b_packed, b_scales, zeros, group_size: int, out_dtype, bias=None, out=None,
                 workspace=None):
    """Asymmetric W4A8 GEMM (include/w4.h): aq [M, K] int8, a_scales [M] fp32,
    b_packed PB-v1 (I8 operand) of raw uint4 codes, b_scales and zeros
    [N] or [N, K/G] (zeros: integers 0..15 in fp16 / bf16 / fp32)."""
    torch = _torch()
    M, K = aq.shape
    N = b_scales.shape[0]
    if aq.dtype != torch.int8:
        raise ValueError("aq must be int8 codes")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, I8), aq.device)
    _check("w4a8_gemm_zp", lib().w4a8_gemm_zp(
        _dev_ptr(aq, "aq"), _dev_ptr(a_scales, "a_scales"), _dev_ptr(b_packed, "b_packed"),
        _dev_ptr(b_scales, "b_scales"), _dtype_code(b_scales.dtype), _dev_ptr(zeros, "zeros"),
        _dtype_code(zeros.dtype), group_size, _dev_ptr(bias, "bias"), _dev_ptr(out, "out"),
        _dtype_code(out_dtype), M, N, K, wsp, wsb, _stream(aq)))
    return out


def w4a16_gemm_prescaled_zeros(a, b_packed, scales, zeros_scaled, group_size: int = 128, bias=None, out=None,
                               workspace=None):
    """W4A16 GEMM with pre-scaled zero-points (include/w4.h): weight value
    c * s - zs per group of 128; scales / zeros_scaled [N, K/128] in a's dtype."""
    torch = _torch()
    M, K = a.shape
    N = scales.shape[0]
    a_dt = _dtype_code(a.dtype)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, a_dt), a.device)
    _check("w4a16_gemm_prescaled_zeros", lib().w4a16_gemm_prescaled_zeros(
        _dev_ptr(a, "a"), a_dt, _dev_ptr(b_packed, "b_packed"), _dev_ptr(scales, "scales"),
        _dev_ptr(zeros_scaled, "zeros_scaled"), group_size, _dev_ptr(bias, "bias"), _dev_ptr(out, "out"),
        M, N, K, wsp, wsb, _stream(a)))
    return out


def w4a16_gemm(a, b_packed, scales, zeros=None, group_size: int = 128, wtype: str = "uint4",
               bias=None, out=None, workspace=None):
    """W4A16 GEMM (include/w4.h): a [M, K] fp16/bf16, b_packed PB-v1 (F16 operand),
    scales / zeros [N, K/G] in a's dtype (zeros None -> 8)."""
    torch = _torch()
    M, K = a.shape
    N = scales.shape[0]
    a_dt = _dtype_code(a.dtype)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, a_dt), a.device)
    _check("w4a16_gemm", lib().w4a16_gemm(
        _dev_ptr(a, "a"), a_dt, _dev_ptr(b_packed, "b_packed"), WTYPES[wtype], _dev_ptr(scales, "scales"),
        _dev_ptr(zeros, "zeros"), group_size, _dev_ptr(bias, "bias"), _dev_ptr(out, "out"), M, N, K,
        wsp, wsb, _stream(a)))
    return out


def _window(M, N, window):
    return (0, M, 0, N) if window is None else window


def w4a8_gemm_partials(aq, b_packed, N: int, group_size: int, wtype: str = "int4", window=None,
                       workspace=None):
    """Per-group dot products of the W4A8 main loop for a window (m0, m1, n0, n1):
    int32 for int8 activations, fp32 for fp8.  Shape [G, m1-m0, n1-n0]."""
    torch = _torch()
    M, K = aq.shape
    a_dt = I8 if aq.dtype == torch.int8 else FP8_E4M3
    m0, m1, n0, n1 = _window(M, N, window)
    gs = K if group_size == -1 else group_size
    part = torch.zeros((K // gs, m1 - m0, n1 - n0), dtype=torch.int32 if a_dt == I8 else torch.float32,
                       device=aq.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, a_dt), aq.device)
    _check("w4a8_gemm_partials", lib().w4a8_gemm_partials(
        _dev_ptr(aq, "aq"), a_dt, _dev_ptr(b_packed, "b_packed"), WTYPES[wtype], group_size, M, N, K,
        m0, m1, n0, n1, _dev_ptr(part, "partials"), wsp, wsb, _stream(aq)))
    return part


def w4a16_gemm_partials(a, b_packed, N: int, group_size: int, zeros=None, wtype: str = "uint4",
                        window=None, workspace=None):
    """Per-group sums of a * (c - z) of the W4A16 main loop (fp32) for a window."""
    torch = _torch()
    M, K = a.shape
    a_dt = _dtype_code(a.dtype)
    m0, m1, n0, n1 = _window(M, N, window)
    gs = K if group_size == -1 else group_size
    part = torch.zeros((K // gs, m1 - m0, n1 - n0), dtype=torch.float32, device=a.device)
    wsp, wsb, ws_keep = _workspace(workspace, gemm_workspace_bytes(M, N, K, group_size, a_dt), a.device)
    _check("w4a16_gemm_partials", lib().w4a16_gemm_partials(
        _dev_ptr(a, "a"), a_dt, _dev_ptr(b_packed, "b_packed"), WTYPES[wtype], _dev_ptr(zeros, "zeros"),
        group_size, M, N, K, m0, m1, n0, n1, _dev_ptr(part, "partials"), wsp, wsb, _stream(a)))
    return part
