"""GPU parity: quantize, dequantize and Hadamard-quantize against the CPU oracle.

Quantized bytes, scale bytes, the global amax and s_global must match the
oracle bit for bit; dequantized outputs too.  Small cases span several
workgroups and ragged tails; the full activation (8192x8192) and rotate
(16384x8192) workloads are checked on sampled rows with the full-tensor amax.
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import (announce, bf16_bits, f32_bits, np_u8, to_gpu_bf16, to_gpu_f32, to_gpu_u8)

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256), (1, 16), (3, 48), (37, 100), (5, 33), (1, 1), (2, 7), (128, 4096), (257, 1056)]


def _input(shape, dtype, seed):
    a = workloads.normal(shape, seed)
    if shape[1] > 8:
        workloads.with_outlier_channels(a, max(1, shape[1] // 100), 40.0, seed)
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(a)
        return to_gpu_bf16(bits), o.bf16_bits_to_f32(bits)
    return to_gpu_f32(a), a


def _check_nv(xg, xf, amax=None):
    q, s, G, sg = fp4.nvfp4_quantize(xg, amax=amax)
    rq, rs, rG, rsg = o.nvfp4_quantize(xf, amax=amax)
    assert np.array_equal(np_u8(q), rq), "codes differ"
    assert np.array_equal(np_u8(s), rs), "scale bytes differ"
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    return q, s, sg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_nvfp4_quantize_matches_oracle(shape, dtype):
    announce(f"nvfp4_quantize {shape} {dtype}")
    xg, xf = _input(shape, dtype, 100 + shape[0] * 7 + shape[1])
    q, s, sg = _check_nv(xg, xf)
    # static amax (calibrated), larger than the tensor's own
    _check_nv(xg, xf, amax=float(np.max(np.abs(xf))) * 1.7 + 0.1)
    # dequantize (NV) to f32 and bf16
    for out in (torch.float32, torch.bfloat16):
        y = fp4.fp4_dequantize(fp4.FP4_NVFP4, q, s, sg, shape[1], out)
        ref = o.nvfp4_dequantize(np_u8(q), np_u8(s), np.float32(f32_bits(sg).view(np.float32)[0]), shape[1])
        if out == torch.float32:
            assert np.array_equal(f32_bits(y), ref.view(np.uint32))
        else:
            assert np.array_equal(bf16_bits(y), o.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_mxfp4_quantize_matches_oracle(shape, dtype):
    announce(f"mxfp4_quantize {shape} {dtype}")
    xg, xf = _input(shape, dtype, 300 + shape[0] * 7 + shape[1])
    q, s = fp4.mxfp4_quantize(xg)
    rq, rs = o.mxfp4_quantize(xf)
    assert np.array_equal(np_u8(q), rq)
    assert np.array_equal(np_u8(s), rs)
    for out in (torch.float32, torch.bfloat16):
        y = fp4.fp4_dequantize(fp4.FP4_MXFP4, q, s, None, shape[1], out)
        ref = o.mxfp4_dequantize(rq, rs, shape[1])
        if out == torch.float32:
            assert np.array_equal(f32_bits(y), ref.view(np.uint32))
        else:
            assert np.array_equal(bf16_bits(y), o.f32_to_bf16_bits(ref))


def test_special_values_and_empty():
    announce("special values")
    x = np.zeros((4, 64), np.float32)
    x[1] = -0.0
    x[2, :] = np.float32(1e-30)
    x[3, 5] = 7.0
    x[3, 6] = -0.2
    x[3, 40] = 3.0e5                     # one huge block: saturated E4M3 scale
    xg = to_gpu_f32(x)
    _check_nv(xg, x)
    q, s = fp4.mxfp4_quantize(xg)
    rq, rs = o.mxfp4_quantize(x)
    assert np.array_equal(np_u8(q), rq) and np.array_equal(np_u8(s), rs)
    # all-zero tensor: s_global = 1
    z = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda:0")
    q, s, G, sg = fp4.nvfp4_quantize(z)
    assert float(G) == 0.0 and float(sg) == 1.0 and int(s.sum()) == 0
    # empty tensors
    e = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda:0")
    q, s, G, sg = fp4.nvfp4_quantize(e)
    assert q.numel() == 0 and float(sg) == 1.0


def test_determinism_and_unaligned_input():
    announce("determinism/unaligned")
    bits = workloads.activation(96, 512, 2, 40.0, seed=77)
    xg = to_gpu_bf16(bits)
    a = [np_u8(t) for t in fp4.nvfp4_quantize(xg)[:2]]
    b = [np_u8(t) for t in fp4.nvfp4_quantize(xg)[:2]]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    # an input that starts 2 bytes into an allocation takes the generic path
    big = torch.zeros(96 * 512 + 1, dtype=torch.bfloat16, device="cuda:0")
    big[1:] = xg.reshape(-1)
    xo = big[1:].view(96, 512)
    assert xo.data_ptr() % 16 != 0
    q, s, G, sg = fp4.nvfp4_quantize(xo)
    assert np.array_equal(np_u8(q), a[0]) and np.array_equal(np_u8(s), a[1])
    qm, sm = fp4.mxfp4_quantize(xo)
    rq, rs = o.mxfp4_quantize(o.bf16_bits_to_f32(bits))
    assert np.array_equal(np_u8(qm), rq) and np.array_equal(np_u8(sm), rs)


def test_activation_workload_full_size_sampled_rows():
    """8192x8192 bf16 with 8 outlier channels x40 (the activation-quantization
    workload): full-tensor amax on the GPU, then 48 sampled rows byte-compared
    with the oracle run on those rows at the same amax."""
    announce("activation 8192x8192 sampled")
    bits = workloads.activation()
    xf_rows = np.random.default_rng(5).choice(8192, 48, replace=False)
    xg = to_gpu_bf16(bits)
    q, s, G, sg = fp4.nvfp4_quantize(xg)
    xf = o.bf16_bits_to_f32(bits)
    rG = o.global_amax(xf)
    assert f32_bits(G)[0] == rG.view(np.uint32)
    sub = xf[xf_rows]
    rq, rs, _, rsg = o.nvfp4_quantize(sub, amax=rG)
    assert np.array_equal(np_u8(q)[xf_rows], rq)
    assert np.array_equal(np_u8(s)[xf_rows], rs)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    y = fp4.fp4_dequantize(fp4.FP4_NVFP4, q, s, sg, 8192, torch.bfloat16)
    ref = o.nvfp4_dequantize(rq, rs, rsg, 8192)
    assert np.array_equal(bf16_bits(y)[xf_rows], o.f32_to_bf16_bits(ref))
    qm, sm = fp4.mxfp4_quantize(xg)
    rqm, rsm = o.mxfp4_quantize(sub)
    assert np.array_equal(np_u8(qm)[xf_rows], rqm) and np.array_equal(np_u8(sm)[xf_rows], rsm)
    ym = fp4.fp4_dequantize(fp4.FP4_MXFP4, qm, sm, None, 8192, torch.bfloat16)
    assert np.array_equal(bf16_bits(ym)[xf_rows], o.f32_to_bf16_bits(o.mxfp4_dequantize(rqm, rsm, 8192)))


@pytest.mark.parametrize("shape", [(2053, 4112), (1031, 8192)])
def test_nvfp4_quantize_large_matches_oracle(shape):
    """bf16 tensors of several million values (hundreds of workgroups, a ragged
    last chunk), computed amax: every byte against the oracle."""
    announce(f"nvfp4 large {shape}")
    xg, xf = _input(shape, "bf16", 900 + shape[0])
    _check_nv(xg, xf)


def test_nvfp4_full_activation_computed_amax_equals_given_amax():
    """8192x8192 activation: quantizing with the computed amax gives the same
    bytes everywhere as quantizing with that amax given (the oracle pins the
    given-amax path on sampled rows of this workload)."""
    announce("nvfp4 computed vs given amax 8192x8192")
    xg = to_gpu_bf16(workloads.activation())
    q, s, G, sg = fp4.nvfp4_quantize(xg)
    qs, ss, _, sgs = fp4.nvfp4_quantize(xg, amax=float(G.cpu()[0]))
    assert torch.equal(q, qs) and torch.equal(s, ss) and torch.equal(sg, sgs)


# ---------------------------------------------------------------- Hadamard --
HSHAPES = [(1, 128), (3, 256), (64, 1024), (33, 640), (512, 2048)]


@pytest.mark.parametrize("mode", [fp4.FP4_RNE, fp4.FP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", HSHAPES)
def test_hadamard_quantize_matches_oracle(shape, dtype, mode):
    announce(f"hadamard_quantize {shape} {dtype} mode={mode}")
    xg, xf = _input(shape, dtype, 500 + shape[0] + shape[1])
    seed = 0x5EED + shape[0]
    q, s, G, sg = fp4.hadamard_quantize(xg, mode=mode, seed=seed)
    rq, rs, rG, rsg = o.hadamard_quantize(xf, rounding="sr" if mode else "rne", seed=seed)
    assert np.array_equal(np_u8(s), rs)
    assert np.array_equal(np_u8(q), rq)
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    # static amax
    q2, s2, _, sg2 = fp4.hadamard_quantize(xg, mode=mode, seed=seed, amax=float(rG) * 2)
    rq2, rs2, _, rsg2 = o.hadamard_quantize(xf, rounding="sr" if mode else "rne", seed=seed, amax=np.float32(rG) * np.float32(2))
    assert np.array_equal(np_u8(q2), rq2) and np.array_equal(np_u8(s2), rs2)


def test_hadamard_sr_unbiased_on_gpu():
    """10^6 values of one constant inside an E2M1 interval: the fraction rounded
    up by the GPU's stochastic rounding matches the interval position."""
    announce("hadamard SR unbiasedness")
    # x such that the rotated tensor is constant: a one-hot per group gives
    # +-c values; use a constant row instead, whose rotation is (sum/sqrt(128), 0, ...)
    rows, cols = 1000, 1024
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, (rows, cols)).astype(np.float32)
    xg = to_gpu_f32(x)
    q, s, G, sg = fp4.hadamard_quantize(xg, mode=fp4.FP4_SR, seed=123)
    rq, rs, rG, rsg = o.hadamard_quantize(x, rounding="sr", seed=123)
    assert np.array_equal(np_u8(q), rq)
    # mean residual of SR over the whole tensor is ~0 (z-score), while RNE's is not a test
    y = o.fwht_orthonormal(x)
    yh = o.nvfp4_dequantize(rq, rs, rsg, cols)
    res = (yh - y).ravel().astype(np.float64)
    z = abs(res.mean()) / (res.std() / np.sqrt(res.size))
    assert z < 5


def test_rotate_workload_full_size_sampled_rows():
    """16384x8192 bf16, 16 outlier channels x60 (the rotate-then-quantize
    workload), RNE and SR: the global amax of the rotated tensor bit-exact, and
    32 sampled rows byte-compared with the oracle at that amax."""
    announce("rotate 16384x8192 sampled")
    bits = workloads.rotate_input()
    xg = to_gpu_bf16(bits)
    xf = o.bf16_bits_to_f32(bits)
    rG = np.float32(0)
    for r0 in range(0, 16384, 2048):
        rG = max(rG, np.max(np.abs(o.fwht_orthonormal(xf[r0:r0 + 2048]))))
    rows = np.sort(np.random.default_rng(6).choice(16384, 32, replace=False))
    y = o.fwht_orthonormal(xf[rows])
    for mode in (fp4.FP4_RNE, fp4.FP4_SR):
        q, s, G, sg = fp4.hadamard_quantize(xg, mode=mode, seed=workloads.SEED_SR)
        assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
        if mode == fp4.FP4_SR:
            idx = rows[:, None].astype(np.uint64) * np.uint64(8192) + np.arange(8192, dtype=np.uint64)[None, :]
            srb = o.sr_bits_at(idx, workloads.SEED_SR)
            rq, rs, _, rsg = o.nvfp4_quantize(y, amax=rG, rounding="sr", sr_bits=srb)
        else:
            rq, rs, _, rsg = o.nvfp4_quantize(y, amax=rG)
        assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
        assert np.array_equal(np_u8(s)[rows], rs)
        assert np.array_equal(np_u8(q)[rows], rq)
