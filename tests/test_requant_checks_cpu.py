"""CPU checks of the requantized-output parity machinery.

The oracle's admissible ranges (e4m3_output_range, nvfp4_output_range) are
pinned by hand-worked values (tests/golden/requant_ranges.txt, from the E4M3
grid of the 10100.com data-type article and the two-level scale equations of
the "low-precision floats" blog).  The GPU tests' checkers (requant_checks)
must accept the oracle's own encoding of the exact result and reject a planted
mistake: one output byte moved to a neighbouring code where the range is a
single value.
"""
import numpy as np
import pytest

from oracle import fp4_oracle as o
from requant_checks import check_e4m3_against_reference, check_nvfp4_against_reference


def test_e4m3_range_hand_worked(golden):
    rows = [r for r in golden("requant_ranges.txt") if r[0] == "e4m3"]
    assert len(rows) == 6
    for _, d, tol, lo, hi in rows:
        vlo, vhi = o.e4m3_output_range(np.array([float(d)]), np.array([float(tol)]))
        assert (vlo[0], vhi[0]) == (float(lo), float(hi)), (d, tol)


def test_nvfp4_range_hand_worked(golden):
    rows = [r for r in golden("requant_ranges.txt") if r[0] == "nvfp4"]
    assert len(rows) == 2
    D = np.array([[1.0] * 15 + [0.6015625]])
    for r in rows:
        amax, tol = float(r[1]), float(r[2])
        blo, bhi = int(r[3], 16), int(r[4], 16)
        exp = [float(v) for v in r[5:]]
        s_g, b_lo, b_hi, (l0, h0), (l1, h1) = o.nvfp4_output_range(D, np.full(D.shape, tol), amax)
        assert s_g == np.float32(1.0)
        assert (int(b_lo[0, 0]), int(b_hi[0, 0])) == (blo, bhi)
        assert [l0[0, 0], h0[0, 0], l0[0, 15], h0[0, 15], l1[0, 0], h1[0, 0], l1[0, 15], h1[0, 15]] == exp


def _gemm_case(seed=3, M=40, N=70, K=512, g_d=0.75):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    qa, sa, _, ga = o.nvfp4_quantize(A)
    qw, sw, _, gw = o.nvfp4_quantize(W)
    return o.scaled_gemm_ref(o.nv_operand_f64(qa, sa, ga, K), o.nv_operand_f64(qw, sw, gw, K), g_d)


def test_e4m3_checker_accepts_oracle_and_rejects_planted_byte():
    ref, mag = _gemm_case()
    codes = o.gemm_e4m3_output(ref.astype(np.float32))
    check_e4m3_against_reference(codes, ref, mag, "oracle")
    lo, hi = o.e4m3_output_range(ref, o.GEMM_REL_TOL * mag)
    i, j = np.argwhere((lo == hi) & (codes & 0x7F > 0) & (codes & 0x7F < 0x7E))[0]
    bad = codes.copy()
    bad[i, j] += 1                       # the next code of the same sign
    with pytest.raises(AssertionError):
        check_e4m3_against_reference(bad, ref, mag, "planted")


def test_nvfp4_checker_accepts_oracle_and_rejects_planted_codes():
    ref, mag = _gemm_case(seed=4, N=72)
    G = float(np.max(np.abs(ref)))
    q, sc, _, sg = o.gemm_nvfp4_output(ref.astype(np.float32), G)
    check_nvfp4_against_reference(q, sc, float(sg), ref, mag, G, "oracle")
    # a scale byte one code above a block whose range is a single byte
    s_g, b_lo, b_hi, _, _ = o.nvfp4_output_range(ref, o.GEMM_REL_TOL * mag, G)
    i, j = np.argwhere((b_lo == b_hi) & (b_lo < 0x7E))[0]
    bad = sc.copy()
    bad[i, j] += 1
    with pytest.raises(AssertionError):
        check_nvfp4_against_reference(q, bad, float(sg), ref, mag, G, "planted scale")
    # an element code moved to its neighbour
    codes = o.unpack_nibbles(q, ref.shape[1])
    k = np.argwhere((codes & 7) == 3)[0]
    codes[tuple(k)] += 1
    with pytest.raises(AssertionError):
        check_nvfp4_against_reference(o.pack_nibbles(codes), sc, float(sg), ref, mag, G, "planted code")
    # a wrong tensor scale
    with pytest.raises(AssertionError):
        check_nvfp4_against_reference(q, sc, float(sg) * 2, ref, mag, G, "planted tensor scale")
