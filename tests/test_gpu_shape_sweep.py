"""GPU parity over a seeded sweep of shapes, dtypes and modes for every entry
point, against the CPU oracle.

The fixed-shape tests pin chosen edges (one row, one column, ragged tails,
several tiles, full workloads).  This sweep draws the shapes instead, from one
seeded generator, so that odd sizes nobody picked (a column count one past a
block, a K tail inside a stage, a group of rows smaller than a tile) meet every
kernel path.  Each case is small enough for the oracle to finish in well under
a second.  Pass rules are the same as elsewhere: quantized codes, scale bytes,
the tensor amax and s_global bit-exact; dequantized and rotated values
bit-exact; GEMM, GEMV and grouped-GEMM outputs within
|D - D_ref| <= 1e-5 * |g_d| * sum_k |a_hat * w_hat| (plus one bf16 rounding of
D_ref for bf16 output).
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import (announce, bf16_bits, f32_bits, np_u8, to_gpu_bf16, to_gpu_f32, to_gpu_u8)

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20251203)


def _draw(n, fn):
    return [fn(i) for i in range(n)]


def _log_uniform(lo, hi):
    """An integer in [lo, hi]: log-uniform or uniform with equal odds, so that
    tiny sizes and sizes spanning several tiles or workgroups both occur."""
    if _RNG.uniform() < 0.5:
        return int(_RNG.integers(lo, hi + 1))
    return min(hi, int(np.floor(float(np.exp(_RNG.uniform(np.log(lo), np.log(hi + 1)))))))


QUANT_CASES = _draw(16, lambda i: (_log_uniform(1, 400), _log_uniform(1, 4100),
                                   "bf16" if i % 2 == 0 else "f32", bool(i % 3 == 0)))
EX_CASES = _draw(10, lambda i: (_log_uniform(1, 160), _log_uniform(1, 2100),
                                int(_RNG.choice([8, 16, 32])), int(_RNG.choice([0, 1, 2, 4]))))
GEMM_CASES = _draw(16, lambda i: ("nv" if i % 2 == 0 else "mx", _log_uniform(1, 700),
                                  _log_uniform(1, 700), 32 * _log_uniform(1, 48),
                                  "f32" if i % 4 < 2 else "bf16"))
GEMV_CASES = _draw(14, lambda i: (_log_uniform(1, 16), _log_uniform(1, 5000), 32 * _log_uniform(1, 200),
                                  "bf16" if i % 2 == 0 else "f32"))
HAD_CASES = _draw(10, lambda i: (_log_uniform(1, 200), 128 * _log_uniform(1, 24),
                                 ["nv_rne", "nv_sr", "mx_rne", "mx_sr", "rotate"][i % 5]))
GROUPED_CASES = _draw(8, lambda i: ("nv" if i % 2 == 0 else "mx", _log_uniform(1, 10),
                                    _log_uniform(1, 400), 32 * _log_uniform(1, 32)))


def _x(rows, cols, dtype, seed):
    a = workloads.normal((rows, cols), seed)
    if cols > 16:
        workloads.with_outlier_channels(a, max(1, cols // 128), 30.0, seed)
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(a)
        return to_gpu_bf16(bits), o.bf16_bits_to_f32(bits)
    return to_gpu_f32(a), a


def _f32_scalar_bits(v):
    return np.float32(v).view(np.uint32)


@pytest.mark.parametrize("rows,cols,dtype,static", QUANT_CASES)
def test_sweep_quantize_and_dequantize(rows, cols, dtype, static):
    announce(f"sweep quantize {rows}x{cols} {dtype} static={static}")
    xg, xf = _x(rows, cols, dtype, 7000 + rows * 31 + cols)
    amax = float(np.max(np.abs(xf))) * 1.25 + 0.5 if static else None
    q, s, G, sg = fp4.nvfp4_quantize(xg, amax=amax)
    rq, rs, rG, rsg = o.nvfp4_quantize(xf, amax=amax)
    assert np.array_equal(np_u8(q), rq) and np.array_equal(np_u8(s), rs)
    assert f32_bits(G)[0] == _f32_scalar_bits(rG) and f32_bits(sg)[0] == _f32_scalar_bits(rsg)
    y = fp4.fp4_dequantize(fp4.FP4_NVFP4, q, s, sg, cols, torch.float32)
    assert np.array_equal(f32_bits(y), o.nvfp4_dequantize(rq, rs, np.float32(rsg), cols).view(np.uint32))
    mq, ms = fp4.mxfp4_quantize(xg)
    rmq, rms = o.mxfp4_quantize(xf)
    assert np.array_equal(np_u8(mq), rmq) and np.array_equal(np_u8(ms), rms)
    my = fp4.fp4_dequantize(fp4.FP4_MXFP4, mq, ms, None, cols, torch.bfloat16)
    assert np.array_equal(bf16_bits(my), o.f32_to_bf16_bits(o.mxfp4_dequantize(rmq, rms, cols)))


@pytest.mark.parametrize("rows,cols,block,search", EX_CASES)
def test_sweep_scale_variants(rows, cols, block, search):
    announce(f"sweep nvfp4_quantize_ex {rows}x{cols} block={block} search={search}")
    xg, xf = _x(rows, cols, "bf16", 7100 + rows * 17 + cols)
    q, s, G, sg = fp4.nvfp4_quantize_ex(xg, block=block, scale_search=search)
    rq, rs, rG, rsg = o.nvfp4_quantize_ex(xf, block=block, search=search)
    assert np.array_equal(np_u8(q), rq) and np.array_equal(np_u8(s), rs)
    assert f32_bits(sg)[0] == _f32_scalar_bits(rsg)
    y = fp4.nvfp4_dequantize_ex(q, s, sg, cols, block=block)
    ref = o.nvfp4_dequantize_ex(rq, rs, np.float32(rsg), cols, block=block)
    assert np.array_equal(f32_bits(y), ref.view(np.uint32))


def _random_operand(fmt, rows, K, seed):
    q = workloads.random_codes((rows, K // 2), seed)
    if fmt == "nv":   # any finite E4M3 byte, subnormals and 0x00 included
        return q, workloads.random_bytes((rows, K // 16), 0x00, 0x7E, seed + 1)
    return q, workloads.random_bytes((rows, K // 32), 112, 140, seed + 1)


def _hat(fmt, q, s, g, K):
    return o.nv_operand_f64(q, s, g, K) if fmt == "nv" else o.mx_operand_f64(q, s, K)


@pytest.mark.parametrize("fmt,M,N,K,out", GEMM_CASES)
def test_sweep_gemm(fmt, M, N, K, out):
    announce(f"sweep gemm {fmt} M={M} N={N} K={K} {out}")
    seed = 7200 + M * 13 + N * 7 + K
    qa, sa = _random_operand(fmt, M, K, seed)
    qw, sw = _random_operand(fmt, N, K, seed + 2)
    ga, gw = (np.float32(0.5), np.float32(0.25)) if fmt == "nv" else (None, None)
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    dev = "cuda:0"
    tga = None if ga is None else torch.tensor([ga], dtype=torch.float32, device=dev)
    tgw = None if gw is None else torch.tensor([gw], dtype=torch.float32, device=dev)
    g_d = 0.75
    D = fp4.fp4_scaled_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), tga, to_gpu_u8(qw), to_gpu_u8(sw), tgw,
                            K, g_d, torch.float32 if out == "f32" else torch.bfloat16)
    ref, mag = o.scaled_gemm_ref(_hat(fmt, qa, sa, 1.0 if ga is None else ga, K),
                                 _hat(fmt, qw, sw, 1.0 if gw is None else gw, K), g_d)
    ok, err, bound = o.gemm_within_tolerance(D.float().cpu().numpy(), ref, mag, out == "bf16")
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


@pytest.mark.parametrize("B,N,K,xdtype", GEMV_CASES)
def test_sweep_gemv(B, N, K, xdtype):
    announce(f"sweep gemv B={B} N={N} K={K} x={xdtype}")
    seed = 7300 + B * 101 + N + K
    Wq = workloads.random_codes((N, K // 2), seed)
    Ws = workloads.random_bytes((N, K // 16), 0x10, 0x60, seed + 1)
    xbits = workloads.gemv_x(B, K, seed=seed + 2)
    xf = o.bf16_bits_to_f32(xbits)
    xg = to_gpu_bf16(xbits) if xdtype == "bf16" else to_gpu_f32(xf)
    gw = torch.tensor([0.03], dtype=torch.float32, device="cuda:0")
    for g_d, out in ((1.0, torch.float32), (0.5, torch.bfloat16)):
        y = fp4.fp4_gemv_batched(xg, to_gpu_u8(Wq), to_gpu_u8(Ws), gw, K, g_d, out)
        ref, mag = o.gemv_ref(xf, Wq, Ws, np.float32(0.03), g_d, K)
        ok, err, bound = o.gemm_within_tolerance(y.float().cpu().numpy(), ref, mag,
                                                 out == torch.bfloat16)
        assert ok, f"{out}: max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


@pytest.mark.parametrize("rows,cols,mode", HAD_CASES)
def test_sweep_rotation(rows, cols, mode):
    announce(f"sweep rotation {rows}x{cols} {mode}")
    xg, xf = _x(rows, cols, "bf16", 7400 + rows * 3 + cols)
    seed = 0x1234_5678_9ABC + rows
    sr = mode.endswith("_sr")
    fmode = fp4.FP4_SR if sr else fp4.FP4_RNE
    if mode.startswith("nv"):
        q, s, G, sg = fp4.hadamard_quantize(xg, mode=fmode, seed=seed)
        rq, rs, rG, rsg = o.hadamard_quantize(xf, rounding="sr" if sr else "rne", seed=seed)
        assert np.array_equal(np_u8(q), rq) and np.array_equal(np_u8(s), rs)
        assert f32_bits(G)[0] == _f32_scalar_bits(rG) and f32_bits(sg)[0] == _f32_scalar_bits(rsg)
    elif mode.startswith("mx"):
        q, s = fp4.hadamard_quantize_mx(xg, mode=fmode, seed=seed)
        rq, rs = o.hadamard_quantize_mx(xf, rounding="sr" if sr else "rne", seed=seed)
        assert np.array_equal(np_u8(q), rq) and np.array_equal(np_u8(s), rs)
    else:
        y = fp4.hadamard_rotate(xg, out_dtype=torch.float32)
        assert np.array_equal(f32_bits(y), o.fwht_orthonormal(xf).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("fmt,E,N,K", GROUPED_CASES)
def test_sweep_grouped_gemm(fmt, E, N, K):
    seed = 7500 + E * 37 + N + K
    rng = np.random.default_rng(seed)
    sizes = [int(v) for v in rng.integers(0, 300, size=E)]
    if E > 2:
        sizes[1] = 0                          # an empty group
    M = sum(sizes)
    announce(f"sweep grouped {fmt} E={E} sizes={sizes} N={N} K={K}")
    if M == 0:
        sizes[0], M = 5, 5
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    qa, sa = _random_operand(fmt, M, K, seed)
    qw, sw = _random_operand(fmt, E * N, K, seed + 2)
    bs = 16 if fmt == "nv" else 32
    dev = "cuda:0"
    if fmt == "nv":
        ga = np.float32(0.5)
        gb = (0.125 + 0.0625 * np.arange(E)).astype(np.float32)
        tga = torch.tensor([ga], dtype=torch.float32, device=dev)
        tgb = torch.from_numpy(gb).to(dev)
        f = fp4.FP4_NVFP4
    else:
        ga, gb, tga, tgb, f = None, None, None, None, fp4.FP4_MXFP4
    D = fp4.fp4_grouped_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), tga,
                             to_gpu_u8(qw).reshape(E, N, K // 2),
                             to_gpu_u8(sw).reshape(E, N, K // bs), tgb,
                             torch.from_numpy(offs).to(dev), K, 1.5, torch.float32)
    A_hat = _hat(fmt, qa, sa, 1.0 if ga is None else ga, K)
    W_hat = np.stack([_hat(fmt, qw[e * N:(e + 1) * N], sw[e * N:(e + 1) * N],
                           1.0 if gb is None else gb[e], K) for e in range(E)])
    ref, mag = o.grouped_gemm_ref(A_hat, W_hat, offs, 1.5)
    ok, err, bound = o.gemm_within_tolerance(D.cpu().numpy(), ref, mag)
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
