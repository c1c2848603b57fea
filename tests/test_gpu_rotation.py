"""GPU parity: Hadamard rotation alone, rotation + MXFP4, and the rotated FP4
linear layer (offline weight rotation): (x H)(W H)^T = x W^T through the FP4
GEMM.

Rotation outputs and quantized bytes must match the oracle bit for bit; the
rotated GEMM must match the oracle's float64 product of the oracle's rotated
operands within the GEMM tolerance (1e-5 of the magnitude sum).
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, bf16_bits, f32_bits, np_u8, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu

RSHAPES = [(1, 128), (3, 256), (64, 1024), (33, 640), (512, 2048), (257, 384)]


def _input(shape, dtype, seed, n_out=None):
    a = workloads.normal(shape, seed)
    workloads.with_outlier_channels(a, n_out or max(1, shape[1] // 200), 40.0, seed)
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(a)
        return to_gpu_bf16(bits), o.bf16_bits_to_f32(bits)
    return to_gpu_f32(a), a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", RSHAPES)
def test_hadamard_rotate_matches_oracle(shape, dtype):
    """y = x H: float32 output bit-exact against the oracle's FWHT, bf16 output
    its nearest-even rounding."""
    announce(f"hadamard_rotate {shape} {dtype}")
    xg, xf = _input(shape, dtype, 900 + shape[0] + shape[1])
    ref = o.fwht_orthonormal(xf)
    y = fp4.hadamard_rotate(xg, 128, torch.float32)
    assert np.array_equal(f32_bits(y), ref.view(np.uint32))
    yb = fp4.hadamard_rotate(xg, 128, torch.bfloat16)
    assert np.array_equal(bf16_bits(yb), o.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("mode", [fp4.FP4_RNE, fp4.FP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", RSHAPES)
def test_hadamard_quantize_mx_matches_oracle(shape, dtype, mode):
    announce(f"hadamard_quantize_mx {shape} {dtype} mode={mode}")
    xg, xf = _input(shape, dtype, 950 + shape[0] + shape[1])
    seed = 0xC0FFEE + shape[1]
    q, s = fp4.hadamard_quantize_mx(xg, 128, mode, seed)
    rq, rs = o.hadamard_quantize_mx(xf, 128, "sr" if mode else "rne", seed)
    assert np.array_equal(np_u8(s), rs)
    assert np.array_equal(np_u8(q), rq)


def test_rotation_argument_errors():
    announce("rotation argument errors")
    x = torch.zeros((4, 200), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError):
        fp4.hadamard_rotate(x)                       # cols % 128
    with pytest.raises(RuntimeError):
        fp4.hadamard_quantize_mx(x)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError):
        fp4.hadamard_quantize_mx(x, 64)              # group must be 128
    assert fp4.hadamard_rotate(torch.zeros((0, 256), dtype=torch.float32, device="cuda:0")).shape == (0, 256)


def _gemm(fmt, qa, sa, ga, qw, sw, gw, K):
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    return fp4.fp4_scaled_gemm(f, qa, sa, ga, qw, sw, gw, K, 1.0, torch.float32).cpu().numpy()


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("M,N,K", [(64, 96, 1024), (300, 257, 2048)])
def test_rotated_fp4_linear_layer(fmt, M, N, K):
    """Both operands rotated along K on the GPU (W H once, as offline), then the
    FP4 GEMM: within the GEMM tolerance of the oracle's rotated FP4 layer, and
    (MXFP4) closer to x W^T than the unrotated FP4 layer on outlier activations."""
    announce(f"rotated fp4 linear {fmt} {M}x{N}x{K}")
    xb = workloads.gemm_a(M, K, seed=960 + M)
    wb = workloads.gemm_w(N, K, seed=961 + N)
    x, W = o.bf16_bits_to_f32(xb), o.bf16_bits_to_f32(wb)
    xg, wg = to_gpu_bf16(xb), to_gpu_bf16(wb)
    D_ref, mag, rqx, rqw = o.rotated_fp4_linear(x, W, fmt=fmt)
    if fmt == "nv":
        qx, sx, _, gx = fp4.hadamard_quantize(xg)
        qw, sw, _, gw = fp4.hadamard_quantize(wg)
        assert np.array_equal(np_u8(qw), rqw[0]) and np.array_equal(np_u8(sw), rqw[1])
        D = _gemm(fmt, qx, sx, gx, qw, sw, gw, K)
    else:
        qx, sx = fp4.hadamard_quantize_mx(xg)
        qw, sw = fp4.hadamard_quantize_mx(wg)
        assert np.array_equal(np_u8(qw), rqw[0]) and np.array_equal(np_u8(sw), rqw[1])
        D = _gemm(fmt, qx, sx, None, qw, sw, None, K)
    ok, err, bound = o.gemm_within_tolerance(D, D_ref, mag)
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    if fmt == "mx":
        exact = x.astype(np.float64) @ W.astype(np.float64).T
        pq, ps = fp4.mxfp4_quantize(xg)
        pwq, pws = fp4.mxfp4_quantize(wg)
        D_plain = _gemm("mx", pq, ps, None, pwq, pws, None, K)
        e_rot = np.linalg.norm(D - exact) / np.linalg.norm(exact)
        e_plain = np.linalg.norm(D_plain - exact) / np.linalg.norm(exact)
        assert e_rot < e_plain, (e_rot, e_plain)


def test_rotation_invariant_on_gpu():
    """(x H)(W H)^T from the GPU's float32 rotations equals x W^T to float32
    rounding of the rotated values."""
    announce("rotation invariant")
    xg, xf = _input((48, 1024), "f32", 970)
    wg, wf = _input((40, 1024), "f32", 971, n_out=1)
    xr = fp4.hadamard_rotate(xg).cpu().numpy().astype(np.float64)
    wr = fp4.hadamard_rotate(wg).cpu().numpy().astype(np.float64)
    mag = np.abs(xf.astype(np.float64)) @ np.abs(wf.astype(np.float64)).T
    assert np.all(np.abs(xr @ wr.T - xf.astype(np.float64) @ wf.astype(np.float64).T) <= 1e-5 * mag)


def test_weight_rotation_full_shape_sampled_rows():
    """The 28672 x 8192 GEMM weight rotated and quantized offline: NVFP4 (with
    its computed amax) and MXFP4, 48 sampled rows bit-exact against the oracle."""
    announce("weight rotation 28672x8192")
    wb = workloads.gemm_w(28672, 8192)
    wg = to_gpu_bf16(wb)
    rows = np.sort(np.random.default_rng(972).choice(28672, 48, replace=False))
    ridx = torch.from_numpy(rows).cuda()
    wf = o.bf16_bits_to_f32(wb[rows])
    qm, sm = fp4.hadamard_quantize_mx(wg)
    rqm, rsm = o.hadamard_quantize_mx(wf)
    assert np.array_equal(np_u8(qm[ridx]), rqm) and np.array_equal(np_u8(sm[ridx]), rsm)
    q, s, G, sg = fp4.hadamard_quantize(wg)
    rG = max(float(np.max(np.abs(o.fwht_orthonormal(o.bf16_bits_to_f32(wb[r:r + 2048])))))
             for r in range(0, 28672, 2048))
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    rq, rs, _, _ = o.hadamard_quantize(wf, amax=np.float32(rG))
    assert np.array_equal(np_u8(q[ridx]), rq) and np.array_equal(np_u8(s[ridx]), rs)
