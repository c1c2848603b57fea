"""micro_scaled_fp4_amd -- NVFP4 / MXFP4 micro-scaled FP4 on AMD MI355X (gfx950).

Thin Python binding over the C ABI of libfp4.so (include/fp4.h).  This module
only marshals arguments: torch allocates outputs and workspaces and supplies
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback: the functions raise if the library is
missing, if a tensor is not on a GPU, or if the call returns an error status.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FP4_LIBRARY may name another build of the same library (A/B timing of kernel variants).
LIB_PATH = os.environ.get("FP4_LIBRARY") or os.path.join(_PKG, "libfp4.so")

# enums of include/fp4.h
FP4_OK = 0
FP4_F32, FP4_BF16, FP4_E4M3 = 0, 1, 2
FP4_NVFP4, FP4_MXFP4 = 0, 1
FP4_RNE, FP4_SR = 0, 1
AMAX_WORKSPACE_BYTES = 4096

NV_BLOCK, MX_BLOCK = 16, 32

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p

# name -> (restype, argtypes)
SIGNATURES = {
    "nvfp4_quantize": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                      ctypes.c_int, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "nvfp4_quantize_no_workspace": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, _c_p, _c_p,
                                                   _c_p, ctypes.c_int, _c_p, _c_p]),
    "nvfp4_quantize_ex": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, ctypes.c_int,
                                         ctypes.c_int, _c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_p,
                                         ctypes.c_size_t, _c_p]),
    "nvfp4_dequantize_ex": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, ctypes.c_int, _c_p,
                                           ctypes.c_int, _c_p]),
    "mxfp4_quantize": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "fp4_dequantize": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p,
                                      ctypes.c_int, _c_p]),
    "fp4_scaled_gemm": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                       ctypes.c_float, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_int,
                                       _c_p]),
    "fp4_scaled_gemm_nvfp4_out": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                 ctypes.c_float, _c_i64, _c_i64, _c_i64, _c_p,
                                                 _c_p, _c_p, _c_p, _c_p]),
    "fp4_grouped_gemm": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                        ctypes.c_float, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_p,
                                        ctypes.c_int, _c_p]),
    "fp4_gemv_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fp4_gemv_batched": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_p, _c_p, _c_p, _c_i64,
                                        _c_i64, ctypes.c_float, _c_p, ctypes.c_int, _c_p,
                                        ctypes.c_size_t, _c_p]),
    "hadamard_quantize": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_uint64, _c_p, _c_p, _c_p,
                                         ctypes.c_int, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "hadamard_quantize_mx": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_uint64, _c_p, _c_p, _c_p]),
    "hadamard_rotate": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_i64, ctypes.c_int, _c_p,
                                       ctypes.c_int, _c_p]),
    "fp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp4_last_hip_error": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp4.so and attach the C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m micro_scaled_fp4_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


class FP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load_library()
        msg = lib.fp4_status_string(status).decode()
        extra = lib.fp4_last_hip_error().decode() if status == 7 else ""
        super().__init__(f"{where}: status {status} ({msg}) {extra}".strip())
        self.status = status


def _check(status: int, where: str):
    if status != FP4_OK:
        raise FP4Error(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return FP4_BF16
    if dt == torch.float32:
        return FP4_F32
    if dt == torch.float8_e4m3fn:   # accepted by the library as a GEMM output only
        return FP4_E4M3
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _gpu_2d(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return t.contiguous()


def _amax_arg(amax, device):
    """Static amax as a 1-element float32 device tensor, or None (dynamic)."""
    if amax is None:
        return None
    if isinstance(amax, torch.Tensor):
        return amax.to(device=device, dtype=torch.float32).reshape(1).contiguous()
    return torch.tensor([float(amax)], dtype=torch.float32, device=device)


# ------------------------------------------------------------------ API ----
def nvfp4_quantize(x: torch.Tensor, amax=None, workspace: Optional[torch.Tensor] = None):
    """x [rows, cols] bf16/f32 -> (codes u8 [rows, ceil(cols/2)], scales u8
    [rows, ceil(cols/16)] (E4M3 bytes), amax f32[1], s_global f32[1])."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, (cols + NV_BLOCK - 1) // NV_BLOCK), dtype=torch.uint8, device=dev)
    g_scale = torch.empty(1, dtype=torch.float32, device=dev)
    a = _amax_arg(amax, dev)
    given = a is not None
    if not given:
        a = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(AMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    lib = load_library()
    st = lib.nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(q), _ptr(sc), _ptr(a),
                            int(given), _ptr(g_scale), _ptr(workspace),
                            0 if workspace is None else workspace.numel() * workspace.element_size(),
                            _stream(dev))
    _check(st, "nvfp4_quantize")
    return q, sc, a, g_scale


def nvfp4_quantize_no_workspace(x: torch.Tensor, amax=None, out=None):
    """nvfp4_quantize through the allocation-free entry point: the dynamic amax
    pass uses the library's own device array, so the C call allocates nothing.
    out: optional (codes, scales, amax f32[1], s_global f32[1]) tensors to write
    into (then this function allocates nothing either; with amax given, out[2]
    is read as the static amax).  Returns the four tensors."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows, (cols + NV_BLOCK - 1) // NV_BLOCK), dtype=torch.uint8, device=dev)
        a = _amax_arg(amax, dev)
        if a is None:
            a = torch.empty(1, dtype=torch.float32, device=dev)
        g_scale = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        q, sc, a, g_scale = out
    given = amax is not None
    st = load_library().nvfp4_quantize_no_workspace(
        _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(q), _ptr(sc), _ptr(a), int(given),
        _ptr(g_scale), _stream(dev))
    _check(st, "nvfp4_quantize_no_workspace")
    return q, sc, a, g_scale


def nvfp4_quantize_ex(x: torch.Tensor, block: int = NV_BLOCK, scale_search: int = 0, amax=None,
                      workspace: Optional[torch.Tensor] = None):
    """nvfp4_quantize with `block` (8, 16, 32) values per E4M3 scale and an
    optional least-squared-error search over +-scale_search scale bytes.
    Returns (codes, scales [rows, ceil(cols/block)], amax f32[1], s_global f32[1])."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, (cols + block - 1) // block), dtype=torch.uint8, device=dev)
    g_scale = torch.empty(1, dtype=torch.float32, device=dev)
    a = _amax_arg(amax, dev)
    given = a is not None
    if not given:
        a = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(AMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    st = load_library().nvfp4_quantize_ex(
        _ptr(x), _dtype_code(x.dtype), rows, cols, int(block), int(scale_search), _ptr(q), _ptr(sc),
        _ptr(a), int(given), _ptr(g_scale), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "nvfp4_quantize_ex")
    return q, sc, a, g_scale


def mxfp4_quantize(x: torch.Tensor):
    """x [rows, cols] -> (codes u8 [rows, ceil(cols/2)], scales u8 [rows, ceil(cols/32)] E8M0)."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, (cols + MX_BLOCK - 1) // MX_BLOCK), dtype=torch.uint8, device=dev)
    st = load_library().mxfp4_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(q), _ptr(sc),
                                       _stream(dev))
    _check(st, "mxfp4_quantize")
    return q, sc


def fp4_dequantize(fmt: int, q: torch.Tensor, scales: torch.Tensor, global_scale, cols: int,
                   out_dtype: torch.dtype = torch.float32):
    """Packed codes + scales (+ NVFP4 s_global) -> [rows, cols] out_dtype."""
    q = _gpu_2d(q, "q")
    scales = _gpu_2d(scales, "scales")
    dev = q.device
    rows = q.shape[0]
    y = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    gs = None if global_scale is None else global_scale.reshape(1).contiguous()
    st = load_library().fp4_dequantize(fmt, _ptr(q), _ptr(scales), _ptr(gs), rows, cols, _ptr(y),
                                       _dtype_code(out_dtype), _stream(dev))
    _check(st, "fp4_dequantize")
    return y


def nvfp4_dequantize_ex(q: torch.Tensor, scales: torch.Tensor, global_scale, cols: int,
                        block: int = NV_BLOCK, out_dtype: torch.dtype = torch.float32):
    """fp4_dequantize of NVFP4 data with `block` values per scale."""
    q = _gpu_2d(q, "q")
    scales = _gpu_2d(scales, "scales")
    dev = q.device
    rows = q.shape[0]
    y = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    gs = global_scale.reshape(1).contiguous()
    st = load_library().nvfp4_dequantize_ex(_ptr(q), _ptr(scales), _ptr(gs), rows, cols, int(block),
                                            _ptr(y), _dtype_code(out_dtype), _stream(dev))
    _check(st, "nvfp4_dequantize_ex")
    return y


def fp4_scaled_gemm(fmt: int, A: torch.Tensor, a_scales: torch.Tensor, g_a, W: torch.Tensor,
                    w_scales: torch.Tensor, g_b, K: int, g_d: float = 1.0,
                    out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """D [M, N] = g_d * ((g_a s_a . A) @ (g_b s_b . W)^T); A [M, K/2], W [N, K/2] packed.

    out_dtype float32, bfloat16 or float8_e4m3fn (E4M3 of the float32 result,
    nearest with ties to even, saturating at 448)."""
    A = _gpu_2d(A, "A")
    W = _gpu_2d(W, "W")
    a_scales = _gpu_2d(a_scales, "a_scales")
    w_scales = _gpu_2d(w_scales, "w_scales")
    dev = A.device
    M, N = A.shape[0], W.shape[0]
    if A.shape[1] != K // 2 or W.shape[1] != K // 2:
        raise ValueError("A and W must be [rows, K/2] packed codes")
    D = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    ga = None if g_a is None else g_a.reshape(1).contiguous()
    gb = None if g_b is None else g_b.reshape(1).contiguous()
    st = load_library().fp4_scaled_gemm(fmt, _ptr(A), _ptr(a_scales), _ptr(ga), _ptr(W),
                                        _ptr(w_scales), _ptr(gb), float(g_d), M, N, K, _ptr(D),
                                        _dtype_code(D.dtype), _stream(dev))
    _check(st, "fp4_scaled_gemm")
    return D


def fp4_scaled_gemm_nvfp4_out(fmt: int, A: torch.Tensor, a_scales: torch.Tensor, g_a,
                              W: torch.Tensor, w_scales: torch.Tensor, g_b, K: int,
                              d_amax: torch.Tensor, g_d: float = 1.0):
    """The scaled GEMM with its output quantized to NVFP4 at the given tensor
    amax d_amax (device float): returns (codes [M, ceil(N/2)], scale bytes
    [M, ceil(N/16)], s_global of D [1])."""
    A = _gpu_2d(A, "A")
    W = _gpu_2d(W, "W")
    a_scales = _gpu_2d(a_scales, "a_scales")
    w_scales = _gpu_2d(w_scales, "w_scales")
    dev = A.device
    M, N = A.shape[0], W.shape[0]
    if A.shape[1] != K // 2 or W.shape[1] != K // 2:
        raise ValueError("A and W must be [rows, K/2] packed codes")
    if d_amax.dtype != torch.float32 or d_amax.device != dev:
        raise TypeError("d_amax must be a float32 tensor on the operands' device")
    q = torch.empty((M, (N + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((M, (N + 15) // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty(1, dtype=torch.float32, device=dev)
    ga = None if g_a is None else g_a.reshape(1).contiguous()
    gb = None if g_b is None else g_b.reshape(1).contiguous()
    am = d_amax.reshape(1).contiguous()
    st = load_library().fp4_scaled_gemm_nvfp4_out(fmt, _ptr(A), _ptr(a_scales), _ptr(ga), _ptr(W),
                                                  _ptr(w_scales), _ptr(gb), float(g_d), M, N, K,
                                                  _ptr(q), _ptr(sc), _ptr(am), _ptr(gs), _stream(dev))
    _check(st, "fp4_scaled_gemm_nvfp4_out")
    return q, sc, gs


def gemv_workspace_bytes(B: int, K: int) -> int:
    return int(load_library().fp4_gemv_workspace_bytes(B, K))


def fp4_gemv_batched(x: torch.Tensor, W: torch.Tensor, w_scales: torch.Tensor, g_w, K: int,
                     g_d: float = 1.0, out_dtype: torch.dtype = torch.bfloat16,
                     workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """y [B, N] = g_d * NVFP4(x) @ W_hat^T; x [B, K] bf16/f32 quantized on the fly."""
    x = _gpu_2d(x, "x")
    W = _gpu_2d(W, "W")
    w_scales = _gpu_2d(w_scales, "w_scales")
    dev = x.device
    B = x.shape[0]
    N = W.shape[0]
    if x.shape[1] != K or W.shape[1] != K // 2:
        raise ValueError("x must be [B, K] and W [N, K/2]")
    y = out if out is not None else torch.empty((B, N), dtype=out_dtype, device=dev)
    need = gemv_workspace_bytes(B, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load_library().fp4_gemv_batched(_ptr(x), _dtype_code(x.dtype), B, _ptr(W), _ptr(w_scales),
                                         _ptr(g_w.reshape(1).contiguous()), N, K, float(g_d),
                                         _ptr(y), _dtype_code(y.dtype), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "fp4_gemv_batched")
    return y


def hadamard_quantize(x: torch.Tensor, group: int = 128, mode: int = FP4_RNE, seed: int = 0,
                      amax=None, workspace: Optional[torch.Tensor] = None):
    """FWHT over 128-channel groups fused with NVFP4 quantization (RNE or SR).
    Returns what nvfp4_quantize returns."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, (cols + NV_BLOCK - 1) // NV_BLOCK), dtype=torch.uint8, device=dev)
    g_scale = torch.empty(1, dtype=torch.float32, device=dev)
    a = _amax_arg(amax, dev)
    given = a is not None
    if not given:
        a = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(AMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    st = load_library().hadamard_quantize(
        _ptr(x), _dtype_code(x.dtype), rows, cols, group, mode, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(q), _ptr(sc), _ptr(a), int(given), _ptr(g_scale), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "hadamard_quantize")
    return q, sc, a, g_scale


def hadamard_quantize_mx(x: torch.Tensor, group: int = 128, mode: int = FP4_RNE, seed: int = 0):
    """FWHT over 128-channel groups fused with MXFP4 quantization (RNE or SR).
    Returns (codes u8 [rows, cols/2], E8M0 bytes u8 [rows, cols/32])."""
    x = _gpu_2d(x, "x")
    dev = x.device
    rows, cols = x.shape
    q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, (cols + MX_BLOCK - 1) // MX_BLOCK), dtype=torch.uint8, device=dev)
    st = load_library().hadamard_quantize_mx(_ptr(x), _dtype_code(x.dtype), rows, cols, group, mode,
                                             ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(q), _ptr(sc),
                                             _stream(dev))
    _check(st, "hadamard_quantize_mx")
    return q, sc


def hadamard_rotate(x: torch.Tensor, group: int = 128, out_dtype: torch.dtype = torch.float32):
    """y = x H over 128-channel groups (orthonormal FWHT), float32 or bf16."""
    x = _gpu_2d(x, "x")
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    st = load_library().hadamard_rotate(_ptr(x), _dtype_code(x.dtype), x.shape[0], x.shape[1], group,
                                        _ptr(y), _dtype_code(out_dtype), _stream(x.device))
    _check(st, "hadamard_rotate")
    return y


def fp4_grouped_gemm(fmt: int, A: torch.Tensor, a_scales: torch.Tensor, g_a, W: torch.Tensor,
                     w_scales: torch.Tensor, g_b, offsets: torch.Tensor, K: int, g_d: float = 1.0,
                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """One launch over E GEMMs: rows offsets[e] .. offsets[e+1] of A times W[e]^T.
    A [M_total, K/2], W [E, N, K/2] (or [E*N, K/2]), w_scales [E, N, K/bs],
    g_b [E] (NVFP4) or None, offsets int32 [E+1] on the device."""
    A = _gpu_2d(A, "A")
    a_scales = _gpu_2d(a_scales, "a_scales")
    dev = A.device
    if W.dim() != 3 or not W.is_cuda:
        raise ValueError("W must be a [E, N, K/2] GPU tensor")
    E, N = W.shape[0], W.shape[1]
    if A.shape[1] != K // 2 or W.shape[2] != K // 2:
        raise ValueError("A and W must hold K/2 packed bytes per row")
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or offsets.device != dev:
        raise ValueError("offsets must be int32 [E+1] on the operands' device")
    W = W.contiguous()
    w_scales = w_scales.contiguous()
    M = A.shape[0]
    D = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    ga = None if g_a is None else g_a.reshape(1).contiguous()
    gb = None if g_b is None else g_b.reshape(E).contiguous()
    st = load_library().fp4_grouped_gemm(fmt, _ptr(A), _ptr(a_scales), _ptr(ga), _ptr(W),
                                         _ptr(w_scales), _ptr(gb), float(g_d), E,
                                         _ptr(offsets.contiguous()), M, N, K, _ptr(D),
                                         _dtype_code(D.dtype), _stream(dev))
    _check(st, "fp4_grouped_gemm")
    return D
