"""GPU parity: block-scaled FP4 GEMM (NVFP4 and MXFP4) against the float64 oracle.

Pass rule: |D - D_ref| <= 1e-5 * |g_d| * sum_k |A_hat_mk * W_hat_nk| for float32
output, plus one bf16 rounding of D_ref for bf16 output.  Small shapes span
several 256x256 tiles with ragged M/N edges and K tails; the prefill shape
(8192 x 28672 x 8192) is checked on sampled entries, two full rows, two full
columns and one 128x128 tile.

Requantized outputs (E4M3, NVFP4: codes decided by floating point) are checked
against the float64 oracle on their own: the same GEMM's float32 result must
meet the rule above, and every output byte must be one that some float32 value
within the rule of D_ref encodes to (oracle e4m3_output_range /
nvfp4_output_range).  Where the rule's interval holds no rounding point of the
encoder that admissible set is one value, so the byte is exactly the oracle's;
the fraction of outputs left open by the interval is reported and capped (the
rule's 1e-5 relative width against E4M3's 1/16-1/8 spacing, and exact dyadic
dot products that land on E4M3 midpoints, leave ~0.1-6% of E4M3 outputs open
on these shapes, ~0.3% of NVFP4 blocks).  As a second check
the bytes must equal the oracle's encoding of the kernel's own float32 result,
bit for bit (both sides encode the same float32 value).
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, to_gpu_u8
from requant_checks import check_e4m3_against_reference, check_nvfp4_against_reference

pytestmark = pytest.mark.gpu


def _operands(fmt, M, N, K, seed, quantized_from=None):
    """Oracle-made operands: NVFP4/MXFP4 quantization of seeded bf16 data, or
    (for the big shape) uniformly random valid codes and scale bytes."""
    if quantized_from is not None:
        Af, Wf = quantized_from
        if fmt == "nv":
            qa, sa, _, ga = o.nvfp4_quantize(Af)
            qw, sw, _, gw = o.nvfp4_quantize(Wf)
            return qa, sa, np.float32(ga), qw, sw, np.float32(gw)
        qa, sa = o.mxfp4_quantize(Af)
        qw, sw = o.mxfp4_quantize(Wf)
        return qa, sa, None, qw, sw, None
    qa = workloads.random_codes((M, K // 2), seed)
    qw = workloads.random_codes((N, K // 2), seed + 1)
    if fmt == "nv":
        sa = workloads.random_bytes((M, K // 16), 0x20, 0x50, seed + 2)
        sw = workloads.random_bytes((N, K // 16), 0x20, 0x50, seed + 3)
        return qa, sa, np.float32(0.75), qw, sw, np.float32(0.0625)
    sa = workloads.random_bytes((M, K // 32), 120, 134, seed + 2)
    sw = workloads.random_bytes((N, K // 32), 120, 134, seed + 3)
    return qa, sa, None, qw, sw, None


def _hat(fmt, q, s, g, K, rows=None):
    if rows is not None:
        q, s = q[rows], s[rows]
    return o.nv_operand_f64(q, s, g, K) if fmt == "nv" else o.mx_operand_f64(q, s, K)


def _gpu_gemm(fmt, ops, K, g_d, out_dtype):
    qa, sa, ga, qw, sw, gw = ops
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    tga = None if ga is None else torch.tensor([ga], dtype=torch.float32, device="cuda:0")
    tgw = None if gw is None else torch.tensor([gw], dtype=torch.float32, device="cuda:0")
    return fp4.fp4_scaled_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), tga, to_gpu_u8(qw), to_gpu_u8(sw),
                               tgw, K, g_d, out_dtype)


def _check(D, fmt, ops, K, g_d, out_bf16, rows=None, cols=None):
    qa, sa, ga, qw, sw, gw = ops
    Ah = _hat(fmt, qa, sa, 1.0 if ga is None else ga, K, rows)
    Wh = _hat(fmt, qw, sw, 1.0 if gw is None else gw, K, cols)
    ref, mag = o.scaled_gemm_ref(Ah, Wh, g_d)
    ok, err, bound = o.gemm_within_tolerance(D, ref, mag, out_bf16)
    assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_tiny_reference_config(fmt):
    """A, W fp32 64x256 ~ N(0,1) with 1% of entries x50, quantized (NVFP4 or
    MXFP4), D = A_hat @ W_hat^T (64x64)."""
    announce(f"gemm tiny {fmt}")
    A, W = workloads.tiny_pair()
    ops = _operands(fmt, 64, 64, 256, 0, quantized_from=(A, W))
    for out in (torch.float32, torch.bfloat16):
        D = _gpu_gemm(fmt, ops, 256, 1.0, out)
        _check(D.float().cpu().numpy(), fmt, ops, 256, 1.0, out == torch.bfloat16)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (17, 33, 96), (256, 256, 128), (100, 300, 384),
                                   (300, 520, 4096), (513, 257, 1056)])
def test_gemm_small_shapes(fmt, M, N, K):
    announce(f"gemm {fmt} {M}x{N}x{K}")
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=70 + M))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=71 + N))
    ops = _operands(fmt, M, N, K, 0, quantized_from=(A, W))
    D = _gpu_gemm(fmt, ops, K, 1.0, torch.float32)
    _check(D.cpu().numpy(), fmt, ops, K, 1.0, False)
    D = _gpu_gemm(fmt, ops, K, -2.5, torch.bfloat16)
    _check(D.float().cpu().numpy(), fmt, ops, K, -2.5, True)
    # the bf16 output is the nearest-even bf16 of the float32 result, bit for bit
    D32 = _gpu_gemm(fmt, ops, K, -2.5, torch.float32).cpu().numpy()
    assert np.array_equal(D.cpu().view(torch.int16).numpy().view(np.uint16), o.f32_to_bf16_bits(D32))


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("K", [1280, 1056])
def test_gemm_workgroups_take_several_tiles(fmt, K):
    """More 256 x 256 tiles than compute units (2300 x 7700: 9 x 31 = 279), so
    workgroups go on to further tiles, the load schedule running on from one
    tile into the next; ragged M and N edges; an odd number of 256-value
    stages (K = 1280: 5, so every tile ends on a padding stage; K = 1056: a
    32-value tail).  Every float32 output against the oracle; the bf16 output
    is the float32 result rounded to bf16; E4M3 and NVFP4 outputs (other
    epilogues between tiles) against the oracle's encoding of that result."""
    M, N = 2300, 7700
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert 9 * 31 > ncu, "the shape is meant to give some workgroups a second tile"
    announce(f"gemm several tiles per workgroup {fmt} {M}x{N}x{K}")
    ops = _operands(fmt, M, N, K, 120 + K)
    D32 = _gpu_gemm(fmt, ops, K, 1.0, torch.float32)
    d32 = D32.cpu().numpy()
    _check(d32, fmt, ops, K, 1.0, False)
    Db = _gpu_gemm(fmt, ops, K, 1.0, torch.bfloat16)
    assert np.array_equal(Db.cpu().view(torch.int16).numpy().view(np.uint16), o.f32_to_bf16_bits(d32))
    D8 = _gpu_gemm(fmt, ops, K, 1.0, torch.float8_e4m3fn)
    assert np.array_equal(D8.view(torch.uint8).cpu().numpy(), o.gemm_e4m3_output(d32))
    amax = float(np.max(np.abs(d32)))
    _check_nv_out(_gpu_gemm_nv_out(fmt, ops, K, 1.0, amax), d32, amax, what=f"{fmt} K={K}")


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_empty_k_writes_zeros(fmt):
    """K = 0: D is the empty sum, exactly 0; M = 0 or N = 0 writes nothing."""
    announce(f"gemm K=0 {fmt}")
    dev = "cuda:0"
    e = torch.empty((5, 0), dtype=torch.uint8, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev) if fmt == "nv" else None
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    for out in (torch.float32, torch.bfloat16, torch.float8_e4m3fn):
        D = torch.full((5, 5), 3.0, dtype=torch.float32, device=dev).to(out)
        fp4.fp4_scaled_gemm(f, e, e, g, e, e, g, 0, 1.0, out, out=D)
        assert torch.count_nonzero(D.view(torch.uint8)).item() == 0
    z = torch.empty((0, 16), dtype=torch.uint8, device=dev)
    assert fp4.fp4_scaled_gemm(f, z, z, g, z, z, g, 32).shape == (0, 0)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_unit_scales_exact(fmt):
    """All block scales 1 and g = 1: every product is a multiple of 1/4 and the
    float32 sums stay exact, so D must equal the integer matmul exactly."""
    announce(f"gemm exact {fmt}")
    M, N, K = 300, 200, 2048
    qa = workloads.random_codes((M, K // 2), 81)
    qw = workloads.random_codes((N, K // 2), 82)
    one = 0x38 if fmt == "nv" else 127
    bs = 16 if fmt == "nv" else 32
    sa = np.full((M, K // bs), one, np.uint8)
    sw = np.full((N, K // bs), one, np.uint8)
    g = np.float32(1.0) if fmt == "nv" else None
    ops = (qa, sa, g, qw, sw, g)
    D = _gpu_gemm(fmt, ops, K, 1.0, torch.float32).cpu().numpy()
    ref, _ = o.scaled_gemm_ref(_hat(fmt, qa, sa, 1.0, K), _hat(fmt, qw, sw, 1.0, K), 1.0)
    assert np.array_equal(D.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_prefill_shape_sampled(fmt):
    """8192 x 28672 x 8192 with random valid codes and scale bytes; bf16 output
    (the timed configuration) checked on 4096 random entries, 2 full rows, 2 full
    columns and one 128x128 tile."""
    announce(f"gemm prefill {fmt}")
    M, N, K = 8192, 28672, 8192
    ops = _operands(fmt, M, N, K, 91 if fmt == "nv" else 92)
    D = _gpu_gemm(fmt, ops, K, 1.0, torch.bfloat16)
    rng = np.random.default_rng(93)
    ii = rng.integers(0, M, 4096)
    jj = rng.integers(0, N, 4096)
    Dn = D[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()].float().cpu().numpy()
    qa, sa, ga, qw, sw, gw = ops
    Ah = _hat(fmt, qa, sa, 1.0 if ga is None else ga, K, ii)
    Wh = _hat(fmt, qw, sw, 1.0 if gw is None else gw, K, jj)
    ref = np.sum(Ah * Wh, axis=1)
    mag = np.sum(np.abs(Ah * Wh), axis=1)
    ok, err, bound = o.gemm_within_tolerance(Dn, ref, mag, True)
    assert ok, f"sampled entries: max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    rows = np.array([0, 5003])
    cols = np.array([7, 28671])
    _check(D[torch.from_numpy(rows).cuda()].float().cpu().numpy(), fmt, ops, K, 1.0, True, rows=rows)
    _check(D[:, torch.from_numpy(cols).cuda()].float().cpu().numpy(), fmt, ops, K, 1.0, True, cols=cols)
    r0, c0 = 4096 + 64, 20480 + 96
    tr, tc = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
    _check(D[r0:r0 + 128, c0:c0 + 128].float().cpu().numpy(), fmt, ops, K, 1.0, True, rows=tr, cols=tc)


def _check_e4m3(D8, D32, fmt, ops, K, g_d, rows=None, cols=None):
    """E4M3 bytes D8 of a GEMM against the float64 oracle (the same GEMM's
    float32 result D32 within the rule, every byte admissible) and against the
    oracle's encoding of D32 (bit-exact)."""
    codes = D8.view(torch.uint8).cpu().numpy()
    d32 = D32.cpu().numpy()
    qa, sa, ga, qw, sw, gw = ops
    Ah = _hat(fmt, qa, sa, 1.0 if ga is None else ga, K, rows)
    Wh = _hat(fmt, qw, sw, 1.0 if gw is None else gw, K, cols)
    ref, mag = o.scaled_gemm_ref(Ah, Wh, g_d)
    ok, err, bound = o.gemm_within_tolerance(d32, ref, mag)
    assert ok, f"float32 result: max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    check_e4m3_against_reference(codes, ref, mag, f"{fmt} {codes.shape} g_d={g_d:.3g}")
    exp = o.gemm_e4m3_output(d32)
    bad = np.flatnonzero(codes.ravel() != exp.ravel())
    assert bad.size == 0, (f"{bad.size} E4M3 codes differ from the oracle encoding of the float32 "
                           f"output, first at {np.unravel_index(bad[0], codes.shape)}")
    return codes


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (17, 33, 96), (100, 300, 384), (300, 520, 4096),
                                   (513, 257, 1056)])
def test_gemm_e4m3_output(fmt, M, N, K):
    """E4M3 output with g_d chosen so the results cover subnormal, normal and
    saturated (|D| > 448) codes; N = 33 and 257 take the byte-store path."""
    announce(f"gemm e4m3 out {fmt} {M}x{N}x{K}")
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=170 + M))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=171 + N))
    ops = _operands(fmt, M, N, K, 0, quantized_from=(A, W))
    D32 = _gpu_gemm(fmt, ops, K, 1.0, torch.float32)
    spread = float(torch.quantile(D32.abs().flatten()[:100000], 0.5).item()) if M * N > 1 else 1.0
    for g_d in (1.0, 300.0 / max(spread, 1e-30), -0.01 / max(spread, 1e-30)):
        D8 = _gpu_gemm(fmt, ops, K, g_d, torch.float8_e4m3fn)
        assert D8.dtype == torch.float8_e4m3fn and D8.shape == (M, N)
        D32g = _gpu_gemm(fmt, ops, K, g_d, torch.float32)
        _check_e4m3(D8, D32g, fmt, ops, K, g_d)
    if M * N >= 1000:
        codes = D8.view(torch.uint8).cpu().numpy() & 0x7F
        assert np.any(codes < 8), "no subnormal codes exercised"


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_gemm_e4m3_output_saturates(fmt):
    """A large g_d pushes most outputs past 448: they saturate to +-448 with the
    result's sign (0x7E / 0xFE), never NaN (0x7F / 0xFF)."""
    announce(f"gemm e4m3 saturation {fmt}")
    M, N, K = 64, 96, 512
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=180))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=181))
    ops = _operands(fmt, M, N, K, 0, quantized_from=(A, W))
    D8 = _gpu_gemm(fmt, ops, K, 1e6, torch.float8_e4m3fn)
    D32 = _gpu_gemm(fmt, ops, K, 1e6, torch.float32)
    codes = _check_e4m3(D8, D32, fmt, ops, K, 1e6)
    assert np.mean((codes & 0x7F) == 0x7E) > 0.9
    assert not np.any((codes & 0x7F) == 0x7F)


def test_gemm_e4m3_output_prefill_sampled():
    """NVFP4 8192 x 28672 x 8192 (the timed prefill shape) with E4M3 output:
    bit-exact against the oracle encoding of the float32 output on 2^20 sampled
    entries and one 128x128 tile, and within bound of the float64 reference on
    that tile."""
    announce("gemm prefill nv e4m3 out")
    M, N, K = 8192, 28672, 8192
    ops = _operands("nv", M, N, K, 91)
    g_d = 0.25
    D8 = _gpu_gemm("nv", ops, K, g_d, torch.float8_e4m3fn)
    D32 = _gpu_gemm("nv", ops, K, g_d, torch.float32)
    rng = np.random.default_rng(94)
    ii = torch.from_numpy(rng.integers(0, M, 1 << 20)).cuda()
    jj = torch.from_numpy(rng.integers(0, N, 1 << 20)).cuda()
    codes = D8.view(torch.uint8)[ii, jj].cpu().numpy()
    exp = o.gemm_e4m3_output(D32[ii, jj].cpu().numpy())
    assert np.array_equal(codes, exp), f"{np.count_nonzero(codes != exp)} sampled codes differ"
    # 4096 of the sampled entries against the float64 reference itself
    qa, sa, ga, qw, sw, gw = ops
    i4, j4 = ii[:4096].cpu().numpy(), jj[:4096].cpu().numpy()
    Ah, Wh = _hat("nv", qa, sa, ga, K, i4), _hat("nv", qw, sw, gw, K, j4)
    ref, mag = g_d * np.sum(Ah * Wh, axis=1), abs(g_d) * np.sum(np.abs(Ah * Wh), axis=1)
    assert o.gemm_within_tolerance(D32[ii[:4096], jj[:4096]].cpu().numpy(), ref, mag)[0]
    check_e4m3_against_reference(codes[:4096], ref, mag, "prefill sampled")
    r0, c0 = 2048 + 32, 12288 + 160
    tr, tc = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
    _check_e4m3(D8[r0:r0 + 128, c0:c0 + 128], D32[r0:r0 + 128, c0:c0 + 128], "nv", ops, K, g_d,
                rows=tr, cols=tc)


def _gpu_gemm_nv_out(fmt, ops, K, g_d, amax):
    qa, sa, ga, qw, sw, gw = ops
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    tga = None if ga is None else torch.tensor([ga], dtype=torch.float32, device="cuda:0")
    tgw = None if gw is None else torch.tensor([gw], dtype=torch.float32, device="cuda:0")
    tam = torch.tensor([amax], dtype=torch.float32, device="cuda:0")
    return fp4.fp4_scaled_gemm_nvfp4_out(f, to_gpu_u8(qa), to_gpu_u8(sa), tga, to_gpu_u8(qw),
                                         to_gpu_u8(sw), tgw, K, tam, g_d)


def _check_nv_out(got, D32, amax, rows=None, ref=None, mag=None, what=""):
    """NVFP4 output against the float64 reference (ref, mag given: every byte
    admissible under the tolerance rule) and against the oracle's NVFP4
    quantization (given amax) of the kernel's own float32 result, bit for bit."""
    q, sc, gs = got
    qe, se, _, sge = o.gemm_nvfp4_output(D32, amax)
    qn, sn = q.cpu().numpy(), sc.cpu().numpy()
    if rows is not None:
        qn, sn = qn[rows], sn[rows]
    if ref is not None:
        assert o.gemm_within_tolerance(D32, ref, mag)[0], f"{what}: float32 result outside the rule"
        check_nvfp4_against_reference(qn, sn, float(gs.item()), ref, mag, amax, what)
    bad = np.argwhere(sn != se)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {tuple(bad[0])}"
    bad = np.argwhere(qn != qe)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {tuple(bad[0])}"
    assert float(gs.item()) == float(sge)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (17, 33, 96), (100, 300, 384), (300, 520, 4096),
                                   (513, 257, 1056), (64, 301, 512)])
def test_gemm_nvfp4_output(fmt, M, N, K):
    """NVFP4 output at three given amaxes of D: its true max, 4x it (small
    block scales) and a quarter of it (scales saturate at 448, codes at 6).
    N = 33, 257, 301 take the byte-store path and partial last blocks; 300
    has N % 16 != 0 with 4-value stores."""
    announce(f"gemm nvfp4 out {fmt} {M}x{N}x{K}")
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=190 + M))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=191 + N))
    ops = _operands(fmt, M, N, K, 0, quantized_from=(A, W))
    g_d = 0.5
    D32 = _gpu_gemm(fmt, ops, K, g_d, torch.float32).cpu().numpy()
    qa, sa, ga, qw, sw, gw = ops
    ref, mag = o.scaled_gemm_ref(_hat(fmt, qa, sa, 1.0 if ga is None else ga, K),
                                 _hat(fmt, qw, sw, 1.0 if gw is None else gw, K), g_d)
    G = float(np.max(np.abs(D32)))
    for amax in (G, 4.0 * G, 0.25 * G):
        got = _gpu_gemm_nv_out(fmt, ops, K, g_d, amax)
        assert got[0].shape == (M, (N + 1) // 2) and got[1].shape == (M, (N + 15) // 16)
        _check_nv_out(got, D32, amax, ref=ref, mag=mag, what=f"{fmt} {M}x{N}x{K} amax={amax:.3g}")


def test_gemm_nvfp4_output_zero_amax_and_empty_k():
    """amax 0 gives s_global 1 (the quantizer's rule); K = 0 encodes D = 0 as
    codes 0 and scale bytes 0 without reading the operands."""
    announce("gemm nvfp4 out: amax 0, K = 0")
    M, N, K = 40, 48, 256
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=195))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=196))
    ops = _operands("nv", M, N, K, 0, quantized_from=(A, W))
    D32 = _gpu_gemm("nv", ops, K, 1.0, torch.float32).cpu().numpy()
    qa, sa, ga, qw, sw, gw = ops
    ref, mag = o.scaled_gemm_ref(_hat("nv", qa, sa, ga, K), _hat("nv", qw, sw, gw, K), 1.0)
    _check_nv_out(_gpu_gemm_nv_out("nv", ops, K, 1.0, 0.0), D32, 0.0, ref=ref, mag=mag,
                  what="amax 0")
    dev = "cuda:0"
    e = torch.empty((5, 0), dtype=torch.uint8, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev)
    am = torch.tensor([10.0], dtype=torch.float32, device=dev)
    e7 = torch.empty((7, 0), dtype=torch.uint8, device=dev)
    q, sc, gs = fp4.fp4_scaled_gemm_nvfp4_out(fp4.FP4_NVFP4, e, e, g, e7, e7, g, 0, am)
    assert q.shape == (5, 4) and sc.shape == (5, 1)
    assert torch.count_nonzero(q).item() == 0 and torch.count_nonzero(sc).item() == 0
    assert float(gs.item()) == float(o.nv_global_scale(np.float32(10.0)))


def test_gemm_nvfp4_output_prefill_sampled():
    """NVFP4 8192 x 28672 x 8192 with NVFP4 output at the float32 result's own
    amax: 48 sampled full rows bit-exact against the oracle's quantization of
    the same rows of the kernel's float32 output."""
    announce("gemm prefill nv nvfp4 out")
    M, N, K = 8192, 28672, 8192
    ops = _operands("nv", M, N, K, 91)
    D32 = _gpu_gemm("nv", ops, K, 1.0, torch.float32)
    G = float(D32.abs().max().item())
    got = _gpu_gemm_nv_out("nv", ops, K, 1.0, G)
    rows = np.sort(np.random.default_rng(95).choice(M, 48, replace=False))
    qa, sa, ga, qw, sw, gw = ops
    ref, mag = o.scaled_gemm_ref(_hat("nv", qa, sa, ga, K, rows), _hat("nv", qw, sw, gw, K), 1.0)
    _check_nv_out(got, D32[torch.from_numpy(rows).cuda()].cpu().numpy(), G, rows=rows, ref=ref,
                  mag=mag, what="prefill 48 rows")
