"""GPU parity: batched NVFP4 GEMV against the float64 oracle.

y = g_d * NVFP4(x) @ W_hat^T.  Pass rule: |y - y_ref| <= 1e-5 * |g_d| *
sum_k |x_hat_k * W_hat_nk| (float32 output), plus one bf16 rounding of y_ref
for bf16 output.  W operands come from the oracle's quantizer (small cases)
or are uniformly random valid NVFP4 codes and scales (full decode shape).
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, to_gpu_bf16, to_gpu_f32, to_gpu_u8

pytestmark = pytest.mark.gpu


def _run_and_check(xbits_or_f32, x_is_bf16, Wq, Ws, g_w, N, K, g_d, out_dtype):
    xf = o.bf16_bits_to_f32(xbits_or_f32) if x_is_bf16 else xbits_or_f32
    xg = to_gpu_bf16(xbits_or_f32) if x_is_bf16 else to_gpu_f32(xbits_or_f32)
    gw = torch.tensor([g_w], dtype=torch.float32, device="cuda:0")
    y = fp4.fp4_gemv_batched(xg, to_gpu_u8(Wq), to_gpu_u8(Ws), gw, K, g_d, out_dtype)
    y_ref, mag = o.gemv_ref(xf, Wq, Ws, np.float32(g_w), g_d, K)
    ok, err, bound = o.gemm_within_tolerance(y.float().cpu().numpy(), y_ref, mag,
                                             out_bf16=out_dtype == torch.bfloat16)
    assert ok, f"max err/bound = {np.max(err / np.maximum(bound, 1e-300))}"


@pytest.mark.parametrize("B", [1, 2, 4, 7, 16])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 512), (256, 1056), (300, 5120)])
def test_gemv_small_matches_oracle(B, N, K):
    announce(f"gemv B={B} N={N} K={K}")
    Wb = workloads.gemv_weight(N, K, seed=40 + N)
    Wq, Ws, _, g_w = o.nvfp4_quantize(o.bf16_bits_to_f32(Wb))
    x = workloads.gemv_x(B, K, seed=50 + K)
    _run_and_check(x, True, Wq, Ws, float(g_w), N, K, 1.0, torch.float32)
    _run_and_check(x, True, Wq, Ws, float(g_w), N, K, 0.5, torch.bfloat16)
    _run_and_check(o.bf16_bits_to_f32(x), False, Wq, Ws, float(g_w), N, K, 2.0, torch.float32)


@pytest.mark.parametrize("B,N,K", [(16, 64, 20480), (2, 100, 32768), (12, 70, 5120), (9, 33, 4096),
                                   (16, 33, 1 << 20)])
def test_gemv_long_k_and_wide_batch(B, N, K):
    """Shapes that take the other kernel paths: x kept in LDS as codes + scales
    (wide batch or long K) and the split-K path for K too long for LDS, up to
    K = 2^20 at B = 16 (x's global amax computed once, by the amax pass, and
    read by the prep launch)."""
    announce(f"gemv path B={B} N={N} K={K}")
    Wq = workloads.random_codes((N, K // 2), seed=K + 1)
    Ws = workloads.random_bytes((N, K // 16), 0x18, 0x58, seed=K + 2)
    x = workloads.gemv_x(B, K, seed=K + 3)
    _run_and_check(x, True, Wq, Ws, 0.02, N, K, 1.0, torch.float32)
    _run_and_check(o.bf16_bits_to_f32(x), False, Wq, Ws, 0.02, N, K, 0.5, torch.bfloat16)


@pytest.mark.parametrize("B,N,K", [(2, 40000, 2048), (3, 33000, 1056), (1, 36000, 4096),
                                   (5, 2100, 1024)])
def test_gemv_several_rounds(B, N, K):
    """More 16-row strips than one pass of the workgroups takes (2048 per round
    on 256 CUs), so strips come in rounds; covers the per-round exchange of the
    two K halves, per-pair scale loads (K = 1056) and scale groups that reach
    past a K half (K = 2048: 4 pairs per half, groups of 8)."""
    announce(f"gemv rounds B={B} N={N} K={K}")
    Wq = workloads.random_codes((N, K // 2), seed=N + 1)
    Ws = workloads.random_bytes((N, K // 16), 0x18, 0x58, seed=N + 2)
    x = workloads.gemv_x(B, K, seed=N + 3)
    _run_and_check(x, True, Wq, Ws, 0.02, N, K, 1.0, torch.float32)


@pytest.mark.parametrize("B,N,K", [(16, 17, 2304), (16, 300, 2560), (8, 40000, 5120), (12, 1, 5120),
                                   (9, 4099, 4864), (16, 70, 3328)])
def test_gemv_x_in_registers(B, N, K):
    """Batches whose fp16 x' does not fit LDS (8 to 16 rows, K a multiple of
    256 up to 5120): x dequantized once per wave into registers, a quarter of K
    per wave.  Covers a quarter with no pairs (K = 2304: 3, 3, 3, 0 pairs),
    uneven quarters (K = 2560, 3328, 4864), many rounds of two strips per
    workgroup (N = 40000), a single strip of one row, ragged last strips, and
    float32 x."""
    announce(f"gemv x' in registers B={B} N={N} K={K}")
    Wq = workloads.random_codes((N, K // 2), seed=N + K)
    Ws = workloads.random_bytes((N, K // 16), 0x18, 0x58, seed=N + K + 1)
    x = workloads.gemv_x(B, K, seed=N + K + 2)
    _run_and_check(x, True, Wq, Ws, 0.02, N, K, 1.0, torch.float32)
    _run_and_check(x, True, Wq, Ws, 0.02, N, K, 0.5, torch.bfloat16)
    _run_and_check(o.bf16_bits_to_f32(x), False, Wq, Ws, 0.02, N, K, 2.0, torch.float32)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_gemv_decode_shape_all_outputs(B):
    """W 27648x5120 (the decode GEMV shape) with random valid NVFP4 codes and
    E4M3 scale bytes in [0x18, 0x58]; every one of the B x 27648 outputs checked."""
    announce(f"gemv decode shape B={B}")
    N, K = 27648, 5120
    Wq = workloads.random_codes((N, K // 2), seed=61)
    Ws = workloads.random_bytes((N, K // 16), 0x18, 0x58, seed=62)
    x = workloads.gemv_x(B, K)
    _run_and_check(x, True, Wq, Ws, 0.013, N, K, 1.0, torch.float32)
    _run_and_check(x, True, Wq, Ws, 0.013, N, K, 1.0, torch.bfloat16)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemv_empty_k_writes_zeros(out_dtype):
    """K = 0: every output is an empty sum, so y = 0 exactly; N = 0 is a no-op."""
    announce(f"gemv K=0 {out_dtype}")
    x = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda:0")
    W = torch.empty((40, 0), dtype=torch.uint8, device="cuda:0")
    Ws = torch.empty((40, 0), dtype=torch.uint8, device="cuda:0")
    gw = torch.ones(1, dtype=torch.float32, device="cuda:0")
    y = torch.full((3, 40), 7.0, dtype=out_dtype, device="cuda:0")
    fp4.fp4_gemv_batched(x, W, Ws, gw, 0, 1.0, out_dtype, out=y)
    assert torch.count_nonzero(y).item() == 0
    y0 = fp4.fp4_gemv_batched(torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda:0"),
                              torch.empty((0, 32), dtype=torch.uint8, device="cuda:0"),
                              torch.empty((0, 4), dtype=torch.uint8, device="cuda:0"), gw, 64)
    assert y0.shape == (2, 0)
