"""GPU parity past 32-bit offsets: a bf16 tensor of more than 2^31 values
through the quantizers, the dequantizer and the rotations, and GEMM / GEMV
operands of more than 4 GiB.

The inputs are 64 seeded rows repeated down the tensor on the device, so the
oracle evaluates only those 64 rows (the repeated tensor has the same amax).
Sampled rows, among them the rows on either side of each 2^31- and 2^32-byte
or -element boundary and the last rows, must equal the oracle's result for the
row they repeat: bit for bit for quantized bytes, within the GEMM tolerance for
products.
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, bf16_bits, f32_bits, np_u8, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu

BASE = 64          # distinct seeded rows, repeated


def _tiled_rows(base: torch.Tensor, rows: int) -> torch.Tensor:
    idx = torch.arange(rows, device=base.device) % base.shape[0]
    return base.index_select(0, idx)


def _sample_rows(rows: int, boundaries, seed: int) -> np.ndarray:
    """Rows 0 and 1, the rows on either side of each boundary row, the last two
    rows and 8 random rows."""
    picks = {0, 1, rows - 2, rows - 1}
    for b in boundaries:
        picks |= {b - 1, b, b + 1}
    picks |= set(np.random.default_rng(seed).choice(rows, 8, replace=False).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < rows), dtype=np.int64)


@pytest.fixture(scope="module")
def big_activation():
    rows, cols = (1 << 18) + 3, 8192           # 2,147,508,224 values (4.3 GB of bf16)
    assert rows * cols > 1 << 31
    bits = workloads.activation(BASE, cols)
    xg = _tiled_rows(to_gpu_bf16(bits), rows)
    pick = _sample_rows(rows, [(1 << 31) // cols], 1100)   # element 2^31 (byte 2^32 of x)
    yield rows, cols, bits, xg, pick
    del xg
    torch.cuda.empty_cache()


def test_quantize_dequantize_past_2_31_values(big_activation):
    rows, cols, bits, xg, pick = big_activation
    announce(f"nvfp4 / mxfp4 / dequant {rows}x{cols}")
    xf = o.bf16_bits_to_f32(bits)
    src = pick % BASE
    ridx = torch.from_numpy(pick).cuda()
    q, s, G, sg = fp4.nvfp4_quantize(xg)
    rq, rs, rG, rsg = o.nvfp4_quantize(xf)
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    assert np.array_equal(np_u8(q[ridx]), rq[src]) and np.array_equal(np_u8(s[ridx]), rs[src])
    y = fp4.fp4_dequantize(fp4.FP4_NVFP4, q, s, sg, cols, torch.bfloat16)
    assert np.array_equal(bf16_bits(y[ridx]), o.f32_to_bf16_bits(o.nvfp4_dequantize(rq, rs, rsg, cols))[src])
    del q, s, y
    qm, sm = fp4.mxfp4_quantize(xg)
    rqm, rsm = o.mxfp4_quantize(xf)
    assert np.array_equal(np_u8(qm[ridx]), rqm[src]) and np.array_equal(np_u8(sm[ridx]), rsm[src])


def test_rotations_past_2_31_values(big_activation):
    rows, cols, bits, xg, pick = big_activation
    announce(f"hadamard_quantize / hadamard_quantize_mx {rows}x{cols}")
    xf = o.bf16_bits_to_f32(bits)
    src = pick % BASE
    ridx = torch.from_numpy(pick).cuda()
    q, s, G, sg = fp4.hadamard_quantize(xg)
    rq, rs, rG, rsg = o.hadamard_quantize(xf)
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    assert np.array_equal(np_u8(q[ridx]), rq[src]) and np.array_equal(np_u8(s[ridx]), rs[src])
    del q, s
    qm, sm = fp4.hadamard_quantize_mx(xg)
    rqm, rsm = o.hadamard_quantize_mx(xf)
    assert np.array_equal(np_u8(qm[ridx]), rqm[src]) and np.array_equal(np_u8(sm[ridx]), rsm[src])


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_operand_past_4_gib(fmt):
    """A [M, K/2] of 4.3 GB (M = 2^20 + 77, ragged last row tile), N = 272
    (ragged column tile)."""
    M, N, K = (1 << 20) + 77, 272, 8192
    announce(f"gemm {fmt} {M}x{N}x{K} (A {M * K // 2} bytes)")
    bs = 16 if fmt == "nv" else 32
    lo, hi = (0x20, 0x50) if fmt == "nv" else (120, 134)
    qa = workloads.random_codes((BASE, K // 2), 1101)
    sa = workloads.random_bytes((BASE, K // bs), lo, hi, 1102)
    qw = workloads.random_codes((N, K // 2), 1103)
    sw = workloads.random_bytes((N, K // bs), lo, hi, 1104)
    A = _tiled_rows(to_gpu_u8(qa), M)
    As = _tiled_rows(to_gpu_u8(sa), M)
    if fmt == "nv":
        ga, gb = 0.5, 0.03
        D = fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, A, As, torch.tensor([ga], device="cuda:0"), to_gpu_u8(qw),
                                to_gpu_u8(sw), torch.tensor([gb], device="cuda:0"), K, 1.0, torch.float32)
        ref, mag = o.scaled_gemm_ref(o.nv_operand_f64(qa, sa, np.float32(ga), K),
                                     o.nv_operand_f64(qw, sw, np.float32(gb), K), 1.0)
    else:
        D = fp4.fp4_scaled_gemm(fp4.FP4_MXFP4, A, As, None, to_gpu_u8(qw), to_gpu_u8(sw), None, K, 1.0,
                                torch.float32)
        ref, mag = o.scaled_gemm_ref(o.mx_operand_f64(qa, sa, K), o.mx_operand_f64(qw, sw, K), 1.0)
    del A, As
    rowb = K // 2
    pick = _sample_rows(M, [(1 << 31) // rowb, (1 << 32) // rowb], 1105)
    Dn = D[torch.from_numpy(pick).cuda()].cpu().numpy()
    ok, err, bound = o.gemm_within_tolerance(Dn, ref[pick % BASE], mag[pick % BASE])
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    del D
    torch.cuda.empty_cache()


def test_gemv_weight_past_4_gib():
    """W [N, K/2] of 4.3 GB (N = 2^20 + 5: 65,536 strips in 32 rounds, a ragged
    last strip), B = 2."""
    B, N, K = 2, (1 << 20) + 5, 8192
    announce(f"gemv B={B} N={N} K={K} (W {N * K // 2} bytes)")
    Wq = workloads.random_codes((BASE, K // 2), 1106)
    Ws = workloads.random_bytes((BASE, K // 16), 0x18, 0x58, 1107)
    W = _tiled_rows(to_gpu_u8(Wq), N)
    Wsg = _tiled_rows(to_gpu_u8(Ws), N)
    x = workloads.gemv_x(B, K, seed=1108)
    y = fp4.fp4_gemv_batched(to_gpu_bf16(x), W, Wsg, torch.tensor([0.02], device="cuda:0"), K, 1.0,
                             torch.float32)
    del W, Wsg
    ref, mag = o.gemv_ref(o.bf16_bits_to_f32(x), Wq, Ws, np.float32(0.02), 1.0, K)
    rowb = K // 2
    pick = _sample_rows(N, [(1 << 31) // rowb, (1 << 32) // rowb], 1109)
    yn = y.cpu().numpy()[:, pick]
    ok, err, bound = o.gemm_within_tolerance(yn, ref[:, pick % BASE], mag[:, pick % BASE])
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    del y
    torch.cuda.empty_cache()
