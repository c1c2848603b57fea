"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point that include/fp4.h declares,
and reject bad arguments on the host (before any HIP call) with the documented
status codes.
"""
import ctypes
import os
import re

import pytest

import micro_scaled_fp4_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(m.LIB_PATH), reason="libfp4.so not built")

OK, NULL, SHAPE, DTYPE, ALIGN, ARCH, WORKSPACE, HIP, ALIAS = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:fp4_status|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_six_calls():
    names = declared_functions()
    for fn in ("nvfp4_quantize", "mxfp4_quantize", "fp4_dequantize", "fp4_scaled_gemm",
               "fp4_gemv_batched", "hadamard_quantize"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(m.SIGNATURES)


def test_status_strings():
    lib = m.load_library()
    for s in range(9):
        assert lib.fp4_status_string(s)
    assert b"gfx950" in lib.fp4_status_string(ARCH)


P = ctypes.c_void_p(4096)       # a non-NULL, aligned stand-in pointer (never dereferenced)


def test_quantize_argument_errors():
    lib = m.load_library()
    q = lib.nvfp4_quantize
    assert q(P, 9, 4, 16, P, P, P, 0, P, P, 4096, None) == DTYPE
    assert q(P, 1, -1, 16, P, P, P, 0, P, P, 4096, None) == SHAPE
    assert q(P, 1, 4, 16, P, P, P, 0, None, P, 4096, None) == NULL
    assert q(None, 1, 4, 16, P, P, P, 0, P, P, 4096, None) == NULL
    assert q(P, 1, 4, 16, P, P, None, 1, P, None, 0, None) == NULL      # static amax missing
    assert q(P, 1, 4, 16, P, P, P, 0, P, None, 0, None) == WORKSPACE
    assert q(P, 1, 4, 16, P, P, P, 0, P, P, 100, None) == WORKSPACE
    assert q(ctypes.c_void_p(4097), 1, 4, 16, P, P, P, 0, P, P, 4096, None) == ALIGN
    mx = lib.mxfp4_quantize
    assert mx(P, 3, 4, 32, P, P, None) == DTYPE
    assert mx(None, 1, 4, 32, P, P, None) == NULL
    assert mx(P, 0, 4, -2, P, P, None) == SHAPE


def test_dequant_gemm_gemv_hadamard_argument_errors():
    lib = m.load_library()
    assert lib.fp4_dequantize(7, P, P, P, 4, 16, P, 0, None) == DTYPE
    assert lib.fp4_dequantize(1, P, P, P, 4, 32, P, 0, None) == DTYPE     # MX takes no tensor scale
    assert lib.fp4_dequantize(0, P, P, None, 4, 16, P, 0, None) == NULL
    g = lib.fp4_scaled_gemm
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 48, P, 1, None) == SHAPE     # K % 32
    assert g(1, P, P, P, P, P, P, 1.0, 8, 8, 64, P, 1, None) == DTYPE     # MX: g_a/g_b must be NULL
    assert g(0, P, P, None, P, P, P, 1.0, 8, 8, 64, P, 1, None) == NULL
    assert g(0, ctypes.c_void_p(4104), P, P, P, P, P, 1.0, 8, 8, 64, P, 1, None) == ALIGN
    v = lib.fp4_gemv_batched
    need = lib.fp4_gemv_workspace_bytes(4, 512)
    assert need >= 4 * 256 + 4 * 32
    assert v(P, 1, 0, P, P, P, 8, 512, 1.0, P, 1, P, need, None) == SHAPE   # B < 1
    assert v(P, 1, 17, P, P, P, 8, 512, 1.0, P, 1, P, 1 << 20, None) == SHAPE
    assert v(P, 1, 4, P, P, P, 8, 500, 1.0, P, 1, P, need, None) == SHAPE   # K % 32
    assert v(P, 1, 4, P, P, P, 8, 512, 1.0, P, 1, P, need - 1, None) == WORKSPACE
    # K = 0 needs only y; a missing or misaligned y is reported before any HIP call
    assert v(None, 1, 4, None, None, None, 8, 0, 1.0, None, 1, None, 0, None) == NULL
    assert v(None, 1, 4, None, None, None, 8, 0, 1.0, ctypes.c_void_p(4099), 1, None, 0, None) == ALIGN
    assert g(0, None, None, None, None, None, None, 1.0, 8, 8, 0, None, 1, None) == NULL
    h = lib.hadamard_quantize
    assert h(P, 1, 4, 256, 64, 0, 0, P, P, P, 0, P, P, 4096, None) == SHAPE
    assert h(P, 1, 4, 200, 128, 0, 0, P, P, P, 0, P, P, 4096, None) == SHAPE
    assert h(P, 1, 4, 256, 128, 5, 0, P, P, P, 0, P, P, 4096, None) == DTYPE


def test_e4m3_dtype_is_a_gemm_output_only():
    """FP4_E4M3 (2) passes the GEMM's dtype check (the next check decides) and is
    rejected as input or output dtype by every other call."""
    lib = m.load_library()
    E4M3 = 2
    g = lib.fp4_scaled_gemm
    assert g(0, ctypes.c_void_p(4104), P, P, P, P, P, 1.0, 8, 8, 64, P, E4M3, None) == ALIGN
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 48, P, E4M3, None) == SHAPE
    assert g(0, None, None, None, None, None, None, 1.0, 8, 8, 0, None, E4M3, None) == NULL
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, 3, None) == DTYPE
    assert lib.fp4_dequantize(0, P, P, P, 4, 16, P, E4M3, None) == DTYPE
    assert lib.nvfp4_quantize(P, E4M3, 4, 16, P, P, P, 0, P, P, 4096, None) == DTYPE
    assert lib.mxfp4_quantize(P, E4M3, 4, 32, P, P, None) == DTYPE
    need = lib.fp4_gemv_workspace_bytes(4, 512)
    assert lib.fp4_gemv_batched(P, 1, 4, P, P, P, 8, 512, 1.0, P, E4M3, P, need, None) == DTYPE
    assert lib.fp4_gemv_batched(P, E4M3, 4, P, P, P, 8, 512, 1.0, P, 1, P, need, None) == DTYPE
    assert lib.hadamard_quantize(P, E4M3, 4, 256, 128, 0, 0, P, P, P, 0, P, P, 4096, None) == DTYPE


def test_gemm_nvfp4_out_argument_errors():
    lib = m.load_library()
    g = lib.fp4_scaled_gemm_nvfp4_out
    S = ctypes.c_void_p(8192)    # d_global_scale, distinct from d_amax (P)
    assert g(2, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, P, S, None) == DTYPE
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 48, P, P, P, S, None) == SHAPE      # K % 32
    assert g(0, P, P, P, P, P, P, 1.0, -1, 8, 64, P, P, P, S, None) == SHAPE
    assert g(1, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, P, S, None) == DTYPE      # MX: no g_a/g_b
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, None, S, None) == NULL    # d_amax
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, None, P, S, None) == NULL    # d_scales
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, P, None, None) == NULL    # d_global_scale
    assert g(0, P, P, None, P, P, P, 1.0, 8, 8, 64, P, P, P, S, None) == NULL    # g_a
    assert g(0, ctypes.c_void_p(4104), P, P, P, P, P, 1.0, 8, 8, 64, P, P, P, S, None) == ALIGN
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, ctypes.c_void_p(4098), S, None) == ALIGN
    # d_amax aliasing d_global_scale: workgroup 0 would overwrite the amax others read
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 64, P, P, P, P, None) == ALIAS
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, 0, P, P, S, S, None) == ALIAS       # K = 0 too
    assert g(0, None, None, None, None, None, None, 1.0, 0, 8, 64, None, None, None, None, None) == OK


def test_no_workspace_quantize_argument_errors():
    """nvfp4_quantize_no_workspace takes nvfp4_quantize's arguments minus the
    workspace and rejects the same bad ones on the host."""
    lib = m.load_library()
    q = lib.nvfp4_quantize_no_workspace
    assert q(P, 9, 4, 16, P, P, P, 0, P, None) == DTYPE
    assert q(P, 1, -1, 16, P, P, P, 0, P, None) == SHAPE
    assert q(P, 1, 4, 16, P, P, P, 0, None, None) == NULL
    assert q(None, 1, 4, 16, P, P, P, 0, P, None) == NULL
    assert q(P, 1, 4, 16, P, P, None, 1, P, None) == NULL      # static amax missing
    assert q(ctypes.c_void_p(4097), 1, 4, 16, P, P, P, 0, P, None) == ALIGN
    assert q(P, 1, 4, 16, P, P, P, 0, ctypes.c_void_p(4098), None) == ALIGN


def test_variant_grouped_and_rotation_argument_errors():
    """nvfp4_quantize_ex / nvfp4_dequantize_ex, fp4_grouped_gemm,
    hadamard_quantize_mx and hadamard_rotate reject bad arguments on the host.
    Every call here fails a host check, so none reaches a device."""
    lib = m.load_library()
    qx = lib.nvfp4_quantize_ex
    assert qx(P, 1, 4, 64, 12, 0, P, P, P, 0, P, P, 4096, None) == SHAPE       # block 8/16/32 only
    assert qx(P, 1, 4, 64, 16, -1, P, P, P, 0, P, P, 4096, None) == SHAPE
    assert qx(P, 1, 4, 64, 16, 127, P, P, P, 0, P, P, 4096, None) == SHAPE     # search > 126
    assert qx(P, 1, 4, 64, 8, 126, P, P, P, 0, None, P, 4096, None) == NULL    # global_scale
    assert qx(P, 1, 4, 64, 32, 5, P, P, P, 0, P, P, 4095, None) == WORKSPACE
    assert qx(P, 2, 4, 64, 32, 5, P, P, P, 0, P, P, 4096, None) == DTYPE      # E4M3 is no input
    dx = lib.nvfp4_dequantize_ex
    assert dx(P, P, P, 4, 64, 4, P, 0, None) == SHAPE
    assert dx(P, P, P, 4, 64, 8, P, 2, None) == DTYPE                        # E4M3 is no output
    assert dx(None, P, P, 4, 64, 8, P, 0, None) == NULL
    gg = lib.fp4_grouped_gemm
    assert gg(0, P, P, P, P, P, P, 1.0, 0, P, 8, 8, 64, P, 1, None) == SHAPE   # no groups
    assert gg(0, P, P, P, P, P, P, 1.0, 2, P, 8, 8, 48, P, 1, None) == SHAPE   # K % 32
    assert gg(1, P, P, P, P, P, P, 1.0, 2, P, 8, 8, 64, P, 1, None) == DTYPE   # MX: no g_a / g_b
    assert gg(0, P, P, P, P, P, P, 1.0, 2, P, 8, 8, 64, P, 9, None) == DTYPE
    assert gg(0, P, P, P, P, P, P, 1.0, 2, None, 8, 8, 64, P, 1, None) == NULL
    assert gg(0, P, P, P, P, P, None, 1.0, 2, P, 8, 8, 64, P, 1, None) == NULL
    assert gg(0, P, P, P, P, P, P, 1.0, 2, ctypes.c_void_p(4098), 8, 8, 64, P, 1, None) == ALIGN
    assert gg(0, P, P, P, P, P, P, 1.0, 2, P, 0, 8, 64, P, 1, None) == OK       # no rows: no-op
    hm = lib.hadamard_quantize_mx
    assert hm(P, 1, 4, 256, 64, 0, 0, P, P, None) == SHAPE                     # group must be 128
    assert hm(P, 1, 4, 200, 128, 0, 0, P, P, None) == SHAPE
    assert hm(P, 1, 4, 256, 128, 2, 0, P, P, None) == DTYPE                    # rounding mode
    assert hm(P, 2, 4, 256, 128, 0, 0, P, P, None) == DTYPE
    assert hm(P, 1, 4, 256, 128, 1, 0, P, None, None) == NULL
    assert hm(ctypes.c_void_p(4104), 1, 4, 256, 128, 1, 0, P, P, None) == ALIGN
    assert hm(None, 1, 0, 256, 128, 1, 0, None, None, None) == OK             # no rows: no-op
    hr = lib.hadamard_rotate
    assert hr(P, 1, 4, 256, 256, P, 0, None) == SHAPE
    assert hr(P, 1, 4, 256, 128, P, 2, None) == DTYPE
    assert hr(P, 1, 4, 256, 128, None, 0, None) == NULL
    assert hr(P, 1, 4, 256, 128, ctypes.c_void_p(4104), 0, None) == ALIGN


def header_limit(name):
    """Value of one of the header's size-limit macros."""
    text = open(HEADER).read()
    expr = re.search(rf"#define {name} (.+?)(?:/\*|$)", text, flags=re.M).group(1)
    return int(eval(expr.replace("LL", "")))


def test_contraction_size_limits_are_shape_errors():
    """Shapes past the documented limits of the GEMMs and the GEMV return
    FP4_ERR_SHAPE before any launch; the limits themselves pass the host checks
    (shown by a later check failing instead)."""
    lib = m.load_library()
    mn, kmax = header_limit("FP4_GEMM_MAX_MN"), header_limit("FP4_GEMM_MAX_K")
    assert mn == 1 << 30 and kmax == (1 << 23) - 32 and kmax % 32 == 0
    g = lib.fp4_scaled_gemm
    assert g(0, P, P, P, P, P, P, 1.0, mn + 1, 8, 64, P, 1, None) == SHAPE
    assert g(0, P, P, P, P, P, P, 1.0, 8, mn + 1, 64, P, 1, None) == SHAPE
    assert g(0, P, P, P, P, P, P, 1.0, 8, 8, kmax + 32, P, 1, None) == SHAPE
    assert g(0, P, P, P, P, P, P, 1.0, mn + 1, 8, 0, P, 1, None) == SHAPE       # also for K = 0
    assert g(0, P, P, None, P, P, P, 1.0, mn, mn, kmax, P, 1, None) == NULL     # at the limits
    n = lib.fp4_scaled_gemm_nvfp4_out
    assert n(0, P, P, P, P, P, P, 1.0, 8, 8, kmax + 32, P, P, P, P, None) == SHAPE
    assert n(0, P, P, P, P, P, P, 1.0, mn + 1, 8, 64, P, P, P, P, None) == SHAPE
    gg = lib.fp4_grouped_gemm
    emax = header_limit("FP4_GROUPED_MAX_GROUPS")
    assert gg(0, P, P, P, P, P, P, 1.0, 2, P, mn + 1, 8, 64, P, 1, None) == SHAPE
    assert gg(0, P, P, P, P, P, P, 1.0, 2, P, 8, 8, kmax + 32, P, 1, None) == SHAPE
    assert gg(0, P, P, P, P, P, P, 1.0, emax + 1, P, 8, 8, 64, P, 1, None) == SHAPE
    # tile bound: (ceil(M/256) + E) * ceil(N/256) < 2^31
    assert gg(0, P, P, P, P, P, P, 1.0, 1, P, mn, mn, 64, P, 1, None) == SHAPE
    assert gg(0, P, P, P, P, P, None, 1.0, emax, P, 1 << 20, 1 << 16, kmax, P, 1, None) == NULL
    v = lib.fp4_gemv_batched
    nv, kv = header_limit("FP4_GEMV_MAX_N"), header_limit("FP4_GEMV_MAX_K")
    assert v(P, 1, 4, P, P, P, nv + 1, 512, 1.0, P, 1, P, 1 << 20, None) == SHAPE
    assert v(P, 1, 4, P, P, P, 8, kv + 32, 1.0, P, 1, P, 1 << 40, None) == SHAPE
    assert v(P, 1, 4, P, P, None, nv, kv, 1.0, P, 1, P, 1 << 40, None) == NULL   # at the limits


def test_no_cpu_fallback():
    """The binding has no CPU path: host tensors are rejected, and a missing
    library is an error at the first call, not a silent fallback."""
    import subprocess
    import sys
    import torch
    with pytest.raises(ValueError):
        m.nvfp4_quantize(torch.zeros(4, 16))
    with pytest.raises(ValueError):
        m.mxfp4_quantize(torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(RuntimeError):
        m.load_library("/nonexistent/libfp4.so")
    code = ("import micro_scaled_fp4_amd as m\n"
            "try:\n    m.load_library()\nexcept RuntimeError as e:\n    print('raised', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120,
                       env={**os.environ, "FP4_LIBRARY": "/nonexistent/libfp4.so"})
    assert r.returncode == 0 and r.stdout.startswith("raised"), (r.stdout, r.stderr)
