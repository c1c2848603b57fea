"""GPU parity of the contractions over the whole range of block-scale bytes.

NVFP4 operands take every finite E4M3 scale byte 0x00-0x7E: the subnormal
scales 0x01-0x07 (m * 2^-9) and 0x00 (scale 0) under non-zero codes (10100.com
data-type article, the E4M3 grid of nvFP4的针对性优化; "low-precision floats"
blog, FP8 and FP4 / MXFP4 / NVFP4).  MXFP4 operands take E8M0 bytes across
0-254 (2^-127 ... 2^127), in pairs whose products stay normal and finite in
float32.

One active block per output: row m of A has non-zero codes only in block
b(m) = m mod (K / bs), so D[m, n] = s_a[m, b] * s_w[n, b] * sum over that block
of E2M1 products.  Each output then depends on exactly one pair of scale bytes;
with g = 1 every product and partial sum is exact in float32 (at most 20
significant bits), so D must equal the float64 oracle bit for bit.  Dense
operands with wide scale ranges are checked with the tolerance rule.
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, to_gpu_bf16, to_gpu_f32, to_gpu_u8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _one_block_operands(fmt, M, N, K, a_range, w_range, seed):
    """A with one active block per row (its scale byte from a_range, inactive
    blocks' bytes anything), W dense with scale bytes from w_range."""
    bs = 16 if fmt == "nv" else 32
    nb = K // bs
    codes = o.unpack_nibbles(workloads.random_codes((M, K // 2), seed), K)
    active = np.arange(M) % nb
    mask = (np.arange(K)[None, :] // bs) == active[:, None]
    qa = o.pack_nibbles(np.where(mask, codes, 0).astype(np.uint8))
    top = 0x7E if fmt == "nv" else 254
    sa = workloads.random_bytes((M, nb), 0, top, seed + 1)
    lo, hi = a_range
    # the active blocks sweep a_range in order, so every byte in it occurs
    sa[np.arange(M), active] = (lo + np.arange(M) % (hi - lo + 1)).astype(np.uint8)
    qw = workloads.random_codes((N, K // 2), seed + 2)
    sw = workloads.random_bytes((N, nb), w_range[0], w_range[1], seed + 3)
    return qa, sa, qw, sw


def _hats(fmt, qa, sa, qw, sw, K, g_a=1.0, g_b=1.0):
    if fmt == "nv":
        return o.nv_operand_f64(qa, sa, g_a, K), o.nv_operand_f64(qw, sw, g_b, K)
    return o.mx_operand_f64(qa, sa, K), o.mx_operand_f64(qw, sw, K)


def _gemm(fmt, qa, sa, qw, sw, K, g_a, g_b, g_d, out=torch.float32):
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    ta = None if fmt == "mx" else torch.tensor([g_a], dtype=torch.float32, device=DEV)
    tb = None if fmt == "mx" else torch.tensor([g_b], dtype=torch.float32, device=DEV)
    return fp4.fp4_scaled_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), ta, to_gpu_u8(qw), to_gpu_u8(sw), tb,
                               K, g_d, out)


# (A active-block bytes, W bytes): every E4M3 byte; E8M0 pairs with sums in [130, 371]
ONE_BLOCK_CASES = [("nv", (0, 0x7E), (0, 0x7E)),
                   ("mx", (0, 127), (130, 244)),
                   ("mx", (127, 254), (3, 117)),
                   ("mx", (3, 117), (127, 254))]


@pytest.mark.parametrize("case", range(len(ONE_BLOCK_CASES)))
def test_gemm_one_block_per_output_exact(case):
    fmt, ar, wr = ONE_BLOCK_CASES[case]
    M, N, K = 508, 300, 1024
    announce(f"gemm one-block {fmt} a{ar} w{wr}")
    qa, sa, qw, sw = _one_block_operands(fmt, M, N, K, ar, wr, 500 + case)
    Ah, Wh = _hats(fmt, qa, sa, qw, sw, K)
    ref, _ = o.scaled_gemm_ref(Ah, Wh, 1.0)
    assert np.all(np.isfinite(ref)) and np.all((ref == 0) | (np.abs(ref) >= 2.0 ** -126))
    D = _gemm(fmt, qa, sa, qw, sw, K, 1.0, 1.0, 1.0).cpu().numpy()
    bad = np.argwhere(D.astype(np.float64) != ref)
    assert bad.size == 0, (f"{len(bad)} outputs differ, first {tuple(bad[0])}: {D[tuple(bad[0])]} vs "
                           f"{ref[tuple(bad[0])]} (a byte {sa[bad[0][0], bad[0][0] % sa.shape[1]]})")


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_dense_wide_scale_bytes(fmt):
    """Every block active, scale bytes spread over the whole range (NVFP4 0x00-0x7E
    with tensor scales; MXFP4 70-180 for both operands), float32 and bf16 output."""
    M, N, K = 300, 520, 2048
    announce(f"gemm dense wide scales {fmt}")
    bs = 16 if fmt == "nv" else 32
    lo, hi = (0, 0x7E) if fmt == "nv" else (70, 180)
    qa = workloads.random_codes((M, K // 2), 610)
    qw = workloads.random_codes((N, K // 2), 611)
    sa = workloads.random_bytes((M, K // bs), lo, hi, 612)
    sw = workloads.random_bytes((N, K // bs), lo, hi, 613)
    g_a, g_b = (0.75, 0.0625) if fmt == "nv" else (1.0, 1.0)
    Ah, Wh = _hats(fmt, qa, sa, qw, sw, K, g_a, g_b)
    for g_d, out in ((1.0, torch.float32), (-0.5, torch.bfloat16)):
        ref, mag = o.scaled_gemm_ref(Ah, Wh, g_d)
        D = _gemm(fmt, qa, sa, qw, sw, K, g_a, g_b, g_d, out).float().cpu().numpy()
        ok, err, bound = o.gemm_within_tolerance(D, ref, mag, out == torch.bfloat16)
        assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


@pytest.mark.parametrize("case", [0, 1])
def test_grouped_gemm_one_block_per_output_exact(case):
    fmt, ar, wr = ONE_BLOCK_CASES[case]
    sizes, N, K = [100, 0, 257, 151], 96, 512
    announce(f"grouped one-block {fmt}")
    E, M = len(sizes), sum(sizes)
    qa, sa, _, _ = _one_block_operands(fmt, M, N, K, ar, wr, 700 + case)
    ws = [_one_block_operands(fmt, 1, N, K, ar, wr, 710 + 4 * e + case)[2:] for e in range(E)]
    qw = np.stack([w[0] for w in ws])
    sw = np.stack([w[1] for w in ws])
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    ga = None if fmt == "mx" else torch.ones(1, dtype=torch.float32, device=DEV)
    gb = None if fmt == "mx" else torch.ones(E, dtype=torch.float32, device=DEV)
    D = fp4.fp4_grouped_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), ga, torch.from_numpy(qw).to(DEV),
                             torch.from_numpy(sw).to(DEV), gb, torch.from_numpy(offs).to(DEV), K, 1.0,
                             torch.float32).cpu().numpy()
    if fmt == "nv":
        A = o.nv_operand_f64(qa, sa, 1.0, K)
        W = np.stack([o.nv_operand_f64(qw[e], sw[e], 1.0, K) for e in range(E)])
    else:
        A = o.mx_operand_f64(qa, sa, K)
        W = np.stack([o.mx_operand_f64(qw[e], sw[e], K) for e in range(E)])
    ref, _ = o.grouped_gemm_ref(A, W, offs, 1.0)
    assert np.array_equal(D.astype(np.float64), ref)


def _wide_x(B, K, seed):
    """x [B, K] ~ N(0,1) with each 16-value block scaled by 2^-u (u uniform in
    0..24) and one entry x60, so x's own NVFP4 scale bytes include subnormals
    and zero."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, K)).astype(np.float32)
    x *= np.repeat(np.exp2(-rng.integers(0, 25, (B, K // 16))), 16, axis=1).astype(np.float32)
    x[0, 5] = np.float32(60.0)
    return x


@pytest.mark.parametrize("B,K", [(1, 512), (4, 1056), (16, 2048), (3, 20480)])
def test_gemv_wide_scale_bytes(B, K):
    """W with one active block per row and every E4M3 scale byte 0x00-0x7E (each
    output then depends on one W byte and one x byte), and dense W with the same
    byte range; x whose own scale bytes include subnormals and zero."""
    N = 381
    announce(f"gemv wide scales B={B} K={K}")
    x = _wide_x(B, K, 800 + K)
    xq, xs, _, _ = o.nvfp4_quantize(x)
    assert np.any((xs >= 1) & (xs <= 7)) and np.any(xs == 0), "x scales miss the subnormal range"
    qa, sa, _, _ = _one_block_operands("nv", N, 1, K, (0, 0x7E), (0, 0x7E), 820 + K)
    dense_q = workloads.random_codes((N, K // 2), 830 + K)
    dense_s = workloads.random_bytes((N, K // 16), 0, 0x7E, 831 + K)
    gw = torch.tensor([0.37], dtype=torch.float32, device=DEV)
    for Wq, Ws in ((qa, sa), (dense_q, dense_s)):
        for g_d, out in ((1.0, torch.float32), (0.25, torch.bfloat16)):
            y = fp4.fp4_gemv_batched(to_gpu_f32(x), to_gpu_u8(Wq), to_gpu_u8(Ws), gw, K, g_d, out)
            ref, mag = o.gemv_ref(x, Wq, Ws, np.float32(0.37), g_d, K)
            ok, err, bound = o.gemm_within_tolerance(y.float().cpu().numpy(), ref, mag,
                                                     out == torch.bfloat16)
            assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    # bf16 input: the same x rounded to bf16
    xb = workloads.f32_to_bf16_bits(x)
    y = fp4.fp4_gemv_batched(to_gpu_bf16(xb), to_gpu_u8(qa), to_gpu_u8(sa), gw, K, 1.0, torch.float32)
    ref, mag = o.gemv_ref(o.bf16_bits_to_f32(xb), qa, sa, np.float32(0.37), 1.0, K)
    assert o.gemm_within_tolerance(y.cpu().numpy(), ref, mag)[0]
