"""GPU parity: NVFP4 scale variants (block sizes 8 / 16 / 32 and the E4M3 scale
search) against the CPU oracle, bit for bit: codes, scale bytes, the global
amax, s_global and the dequantized values.  Small shapes take the fast path
(cols a multiple of the block) and the generic path (ragged rows); the
8192x8192 activation workload is checked on sampled rows with the full tensor's
amax.
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, bf16_bits, f32_bits, np_u8, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu

SHAPES = [(64, 512), (37, 200), (5, 33), (1, 8), (2, 7), (129, 2048)]


def _input(shape, dtype, seed):
    a = workloads.normal(shape, seed)
    if shape[1] > 8:
        workloads.with_outlier_channels(a, max(1, shape[1] // 100), 40.0, seed)
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(a)
        return to_gpu_bf16(bits), o.bf16_bits_to_f32(bits)
    return to_gpu_f32(a), a


def _check(xg, xf, block, W, amax=None):
    q, s, G, sg = fp4.nvfp4_quantize_ex(xg, block, W, amax=amax)
    rq, rs, rG, rsg = o.nvfp4_quantize_ex(xf, block, W, amax=amax)
    bad = np.argwhere(np_u8(s) != rs)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {tuple(bad[0])}"
    bad = np.argwhere(np_u8(q) != rq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {tuple(bad[0])}"
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    return q, s, sg, rq, rs, rsg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [8, 16, 32])
@pytest.mark.parametrize("shape", SHAPES)
def test_block_sizes_match_oracle(shape, block, dtype):
    """Amax rule at every block size, dynamic and static amax, plus the
    dequantized values (float32 and bf16)."""
    announce(f"nvfp4_quantize_ex {shape} block {block} {dtype}")
    xg, xf = _input(shape, dtype, 500 + shape[0] * 3 + shape[1] + block)
    q, s, sg, rq, rs, rsg = _check(xg, xf, block, 0)
    _check(xg, xf, block, 0, amax=float(np.max(np.abs(xf))) * 1.3 + 0.1)
    for out in (torch.float32, torch.bfloat16):
        y = fp4.nvfp4_dequantize_ex(q, s, sg, shape[1], block, out)
        ref = o.nvfp4_dequantize_ex(rq, rs, rsg, shape[1], block)
        if out == torch.float32:
            assert np.array_equal(f32_bits(y), ref.view(np.uint32))
        else:
            assert np.array_equal(bf16_bits(y), o.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [8, 16, 32])
@pytest.mark.parametrize("W", [1, 2, 5, 126])
@pytest.mark.parametrize("shape", [(64, 512), (37, 200), (2, 7)])
def test_scale_search_matches_oracle(shape, W, block, dtype):
    """The least-squared-error scale search over +-W codes (126: every code)."""
    announce(f"scale search W={W} {shape} block {block} {dtype}")
    xg, xf = _input(shape, dtype, 700 + shape[0] + shape[1] + W + block)
    _check(xg, xf, block, W)


def test_default_variant_is_nvfp4_quantize():
    announce("nvfp4_quantize_ex(16, 0) == nvfp4_quantize")
    xg, _ = _input((96, 1024), "bf16", 801)
    for a, b in zip(fp4.nvfp4_quantize_ex(xg, 16, 0), fp4.nvfp4_quantize(xg)):
        assert torch.equal(a, b)


def test_scale_search_worked_block_on_gpu():
    """16 values of 5.0 at amax 2688: byte 0x35 for W < 5, 1.25 (0x3A, exact
    decode 5.0) for W >= 5 (hand-derived in the oracle pins)."""
    announce("scale search worked block")
    x = torch.full((3, 16), 5.0, dtype=torch.float32, device="cuda:0")
    for W, byte in ((0, 0x35), (4, 0x35), (5, 0x3A), (126, 0x3A)):
        q, s, _, sg = fp4.nvfp4_quantize_ex(x, 16, W, amax=2688.0)
        assert np_u8(s).ravel().tolist() == [byte] * 3
    y = fp4.nvfp4_dequantize_ex(q, s, sg, 16, 16)
    assert torch.equal(y, x)


def test_variant_argument_errors():
    announce("variant argument errors")
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0")
    for block, W in ((12, 0), (64, 0), (16, -1), (16, 127)):
        with pytest.raises(RuntimeError):
            fp4.nvfp4_quantize_ex(x, block, W)


@pytest.fixture(scope="module")
def activation():
    bits = workloads.activation(8192, 8192)
    return bits, to_gpu_bf16(bits), float(o.global_amax(o.bf16_bits_to_f32(bits)))


@pytest.mark.parametrize("block,W", [(8, 0), (32, 0), (16, 2), (8, 2)])
def test_activation_workload_sampled_rows(activation, block, W):
    """8192x8192 bf16 activation (N(0,1), 8 outlier channels x40) with the
    computed amax: 64 sampled rows bit-exact against the oracle run at the same
    amax (the timed shape and launch)."""
    announce(f"activation 8192x8192 block {block} W {W}")
    bits, xg, rG = activation
    q, s, G, sg = fp4.nvfp4_quantize_ex(xg, block, W)
    rows = np.sort(np.random.default_rng(802 + block + W).choice(8192, 64, replace=False))
    xf = o.bf16_bits_to_f32(bits[rows])
    assert f32_bits(G)[0] == np.float32(rG).view(np.uint32)
    rq, rs, _, rsg = o.nvfp4_quantize_ex(xf, block, W, amax=rG)
    assert f32_bits(sg)[0] == np.float32(rsg).view(np.uint32)
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(np_u8(s[ridx]), rs)
    assert np.array_equal(np_u8(q[ridx]), rq)
