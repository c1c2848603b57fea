"""GPU parity: grouped FP4 GEMM (one launch over E GEMMs, the experts of an MoE
layer) against the float64 oracle.

Pass rule as for fp4_scaled_gemm: |D - D_ref| <= 1e-5 * |g_d| * sum_k |a * w|
(float32 output), plus one bf16 rounding (bf16 output); E4M3 output: every byte
admissible under that rule around the float64 reference (requant_checks), and
bit-exact against the oracle's encoding of the kernel's float32 output.  Each group's
rows must also equal fp4_scaled_gemm of those rows bit for bit.
"""
import numpy as np
import pytest
import torch

import micro_scaled_fp4_amd as fp4
import workloads
from oracle import fp4_oracle as o
from gpu_util import announce, to_gpu_u8
from requant_checks import check_e4m3_against_reference

pytestmark = pytest.mark.gpu


def _group_operands(fmt, sizes, N, K, seed):
    """Random valid codes and scale bytes: A [M, K/2] for all groups' rows,
    W [E, N, K/2] one operand per group, per-group tensor scales (NVFP4)."""
    E = len(sizes)
    M = int(sum(sizes))
    rng = np.random.default_rng(seed)
    qa = workloads.random_codes((M, K // 2), seed)
    qw = workloads.random_codes((E * N, K // 2), seed + 1).reshape(E, N, K // 2)
    if fmt == "nv":
        sa = workloads.random_bytes((M, K // 16), 0x20, 0x50, seed + 2)
        sw = workloads.random_bytes((E * N, K // 16), 0x20, 0x50, seed + 3).reshape(E, N, K // 16)
        ga = np.float32(0.75)
        gb = rng.uniform(0.01, 0.2, E).astype(np.float32)
    else:
        sa = workloads.random_bytes((M, K // 32), 120, 134, seed + 2)
        sw = workloads.random_bytes((E * N, K // 32), 120, 134, seed + 3).reshape(E, N, K // 32)
        ga, gb = None, None
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return qa, sa, ga, qw, sw, gb, offs


def _hats(fmt, ops, K):
    qa, sa, ga, qw, sw, gb, offs = ops
    if fmt == "nv":
        A = o.nv_operand_f64(qa, sa, ga, K)
        W = np.stack([o.nv_operand_f64(qw[e], sw[e], gb[e], K) for e in range(qw.shape[0])])
    else:
        A = o.mx_operand_f64(qa, sa, K)
        W = np.stack([o.mx_operand_f64(qw[e], sw[e], K) for e in range(qw.shape[0])])
    return A, W


def _gpu_grouped(fmt, ops, K, g_d, out_dtype, offsets=None):
    qa, sa, ga, qw, sw, gb, offs = ops
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    dev = "cuda:0"
    tga = None if ga is None else torch.tensor([ga], dtype=torch.float32, device=dev)
    tgb = None if gb is None else torch.from_numpy(gb).to(dev)
    W = torch.from_numpy(np.ascontiguousarray(qw)).to(dev)
    Ws = torch.from_numpy(np.ascontiguousarray(sw)).to(dev)
    to = torch.from_numpy(offs if offsets is None else offsets).to(dev)
    return fp4.fp4_grouped_gemm(f, to_gpu_u8(qa), to_gpu_u8(sa), tga, W, Ws, tgb, to, K, g_d, out_dtype)


CASES = [([300], 96, 256), ([0, 17, 256, 300], 257, 1056), ([40, 0, 1, 513, 77, 0, 255, 256], 520, 2048),
         ([3] * 70, 64, 512)]


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_grouped_gemm_matches_oracle(fmt, case):
    sizes, N, K = CASES[case]
    announce(f"grouped gemm {fmt} E={len(sizes)} N={N} K={K}")
    ops = _group_operands(fmt, sizes, N, K, 40 + case)
    A, W = _hats(fmt, ops, K)
    for g_d, out in ((1.0, torch.float32), (-0.5, torch.bfloat16)):
        D = _gpu_grouped(fmt, ops, K, g_d, out).float().cpu().numpy()
        ref, mag = o.grouped_gemm_ref(A, W, ops[6], g_d)
        ok, err, bound = o.gemm_within_tolerance(D, ref, mag, out == torch.bfloat16)
        assert ok, f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    D32 = _gpu_grouped(fmt, ops, K, 0.25, torch.float32)
    D8 = _gpu_grouped(fmt, ops, K, 0.25, torch.float8_e4m3fn)
    codes = D8.view(torch.uint8).cpu().numpy()
    ref, mag = o.grouped_gemm_ref(A, W, ops[6], 0.25)
    rows = ~np.isnan(ref[:, 0])     # rows inside some group
    assert o.gemm_within_tolerance(D32.cpu().numpy()[rows], ref[rows], mag[rows])[0]
    check_e4m3_against_reference(codes[rows], ref[rows], mag[rows], f"grouped {fmt} case {case}")
    assert np.array_equal(codes, o.gemm_e4m3_output(D32.cpu().numpy()))


@pytest.mark.parametrize("fmt", ["nv", "mx"])
def test_grouped_equals_per_group_gemm(fmt):
    """Each group's rows equal fp4_scaled_gemm of those rows, bit for bit (same
    tiles and float32 accumulation order)."""
    sizes, N, K = CASES[2]
    announce(f"grouped vs per-group {fmt}")
    ops = _group_operands(fmt, sizes, N, K, 60)
    qa, sa, ga, qw, sw, gb, offs = ops
    D = _gpu_grouped(fmt, ops, K, 1.0, torch.float32)
    f = fp4.FP4_NVFP4 if fmt == "nv" else fp4.FP4_MXFP4
    for e in range(len(sizes)):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        tga = None if ga is None else torch.tensor([ga], dtype=torch.float32, device="cuda:0")
        tgb = None if gb is None else torch.tensor([gb[e]], dtype=torch.float32, device="cuda:0")
        De = fp4.fp4_scaled_gemm(f, to_gpu_u8(qa[lo:hi]), to_gpu_u8(sa[lo:hi]), tga, to_gpu_u8(qw[e]),
                                 to_gpu_u8(sw[e]), tgb, K, 1.0, torch.float32)
        assert torch.equal(D[lo:hi], De), e


def test_grouped_offsets_clamped_and_rows_outside_untouched():
    """Offsets that end before M_total leave the remaining rows unwritten;
    offsets past M_total are clamped to it (no access outside A or D)."""
    announce("grouped offsets clamp")
    sizes, N, K = [20, 30, 14], 64, 256
    ops = _group_operands("nv", sizes, N, K, 70)
    A, W = _hats("nv", ops, K)
    qa, sa, ga, qw, sw, gb, offs = ops
    dev = "cuda:0"
    f = fp4.FP4_NVFP4
    args = (to_gpu_u8(qa), to_gpu_u8(sa), torch.tensor([ga], device=dev),
            torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev), torch.from_numpy(gb).to(dev))
    D = torch.full((64, N), 7.0, dtype=torch.float32, device=dev)
    short = np.array([0, 20, 40, 50], np.int32)
    fp4.fp4_grouped_gemm(f, *args, torch.from_numpy(short).to(dev), K, 1.0, torch.float32, out=D)
    Dn = D.cpu().numpy()
    assert np.all(Dn[50:] == 7.0)
    ref, mag = o.grouped_gemm_ref(A, W, short, 1.0)
    assert o.gemm_within_tolerance(Dn[:50], ref[:50], mag[:50])[0]
    D.fill_(7.0)
    past = np.array([0, 20, 50, 1 << 20], np.int32)
    fp4.fp4_grouped_gemm(f, *args, torch.from_numpy(past).to(dev), K, 1.0, torch.float32, out=D)
    ref, mag = o.grouped_gemm_ref(A, W, np.array([0, 20, 50, 64]), 1.0)
    assert o.gemm_within_tolerance(D.cpu().numpy(), ref, mag)[0]


def test_grouped_empty_k_and_argument_errors():
    announce("grouped K=0 and errors")
    dev = "cuda:0"
    e = torch.empty((6, 0), dtype=torch.uint8, device=dev)
    W = torch.empty((3, 8, 0), dtype=torch.uint8, device=dev)
    offs = torch.tensor([0, 2, 2, 6], dtype=torch.int32, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev)
    gb = torch.ones(3, dtype=torch.float32, device=dev)
    D = torch.full((6, 8), 3.0, dtype=torch.float32, device=dev)
    fp4.fp4_grouped_gemm(fp4.FP4_NVFP4, e, e, g, W, W, gb, offs, 0, 1.0, torch.float32, out=D)
    assert torch.count_nonzero(D).item() == 0
    with pytest.raises(ValueError):
        fp4.fp4_grouped_gemm(fp4.FP4_NVFP4, e, e, g, W, W, gb, offs[:3], 0)


def test_moe_workload_sampled_groups():
    """The timed MoE shape: 64 experts, N = 2048, K = 7168, 32768 routed rows
    (4096 tokens x top-8, skewed expert loads), NVFP4, bf16 output: 4 sampled
    experts' rows against the oracle."""
    announce("moe grouped 64 x 2048 x 7168")
    E, N, K = 64, 2048, 7168
    sizes = workloads.moe_group_sizes(E, 32768)
    ops = _group_operands("nv", sizes, N, K, 80)
    D = _gpu_grouped("nv", ops, K, 1.0, torch.bfloat16).float().cpu().numpy()
    qa, sa, ga, qw, sw, gb, offs = ops
    for e in np.random.default_rng(81).choice(E, 4, replace=False):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        Ah = o.nv_operand_f64(qa[lo:hi], sa[lo:hi], ga, K)
        Wh = o.nv_operand_f64(qw[e], sw[e], gb[e], K)
        ref, mag = o.scaled_gemm_ref(Ah, Wh, 1.0)
        ok, err, bound = o.gemm_within_tolerance(D[lo:hi], ref, mag, True)
        assert ok, (int(e), float(np.max(err / np.maximum(bound, 1e-300))))


def test_all_products_are_deterministic():
    """Every kernel with a reduction (GEMM, grouped GEMM, GEMV, rotation with a
    computed amax) gives the same bytes when run twice: no atomics, fixed
    summation orders."""
    announce("determinism of GEMM / grouped / GEMV / rotation")
    dev = "cuda:0"
    M, N, K = 300, 520, 2048
    A = o.bf16_bits_to_f32(workloads.gemm_a(M, K, seed=90))
    W = o.bf16_bits_to_f32(workloads.gemm_w(N, K, seed=91))
    Ag, Wg = torch.from_numpy(A).to(dev), torch.from_numpy(W).to(dev)
    qa, sa, _, ga = fp4.nvfp4_quantize(Ag)
    qw, sw, _, gw = fp4.nvfp4_quantize(Wg)
    runs = []
    for _ in range(2):
        out = [fp4.fp4_scaled_gemm(fp4.FP4_NVFP4, qa, sa, ga, qw, sw, gw, K, 1.0, torch.float32),
               fp4.fp4_gemv_batched(Ag[:16].contiguous(), qw, sw, gw, K, 1.0, torch.float32),
               fp4.fp4_grouped_gemm(fp4.FP4_NVFP4, qa, sa, ga, torch.stack([qw, qw]), torch.stack([sw, sw]),
                                    torch.cat([gw, gw]), torch.tensor([0, 123, M], dtype=torch.int32, device=dev),
                                    K, 1.0, torch.float32)]
        out += list(fp4.hadamard_quantize(Ag))
        runs.append(out)
    for a, b in zip(*runs):
        assert torch.equal(a, b)
