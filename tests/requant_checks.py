"""Checks of requantized GEMM outputs (FP8 E4M3, NVFP4) against the float64
oracle on its own: every output byte must be one that some float32 value within
the GEMM tolerance rule of the exact result encodes to (oracle
e4m3_output_range / nvfp4_output_range).  Where the rule's interval holds no
rounding point of the encoder that set is one value, so the byte is exactly the
oracle's.  The fraction of outputs the interval leaves open is reported and
capped: the rule's relative width of 1e-5 of the magnitude sum, against E4M3's
spacing of 1/16-1/8 of the value, leaves ~0.1-5% of E4M3 outputs open on the
test shapes and ~0.3% of NVFP4 blocks; with few terms (small K, MXFP4's
power-of-two scales) the exact dot products are short dyadic numbers that land
exactly on E4M3 midpoints, where any nonzero tolerance admits both neighbours
(~6% of a 17x33, K = 96 MXFP4 product).  Such outputs are still checked to be
one of the admissible bytes.  No method arithmetic lives here."""
import numpy as np

from oracle import fp4_oracle as o

MAX_OPEN_E4M3 = 0.10   # outputs whose admissible E4M3 set holds more than one value
MAX_OPEN_NV = 0.02     # NVFP4 blocks (scale bytes) or elements left open


def check_e4m3_against_reference(codes, ref, mag, what="", max_open=MAX_OPEN_E4M3):
    """Every E4M3 byte decodes to a value inside the range of encodings of the
    float32 values within the tolerance rule of the float64 reference; returns
    the fraction of outputs whose range holds more than one value."""
    lo, hi = o.e4m3_output_range(ref, o.GEMM_REL_TOL * mag)
    v = o.e4m3_decode(codes)
    bad = np.flatnonzero(~((v >= lo) & (v <= hi)).ravel())
    assert bad.size == 0, (f"{what}: {bad.size} E4M3 bytes outside the admissible range, first at "
                           f"{np.unravel_index(bad[0], codes.shape)}: {v.ravel()[bad[0]]} not in "
                           f"[{lo.ravel()[bad[0]]}, {hi.ravel()[bad[0]]}]")
    open_frac = float(np.mean(lo != hi)) if lo.size else 0.0
    print(f"[e4m3 parity] {what}: {lo.size} outputs, {open_frac:.3%} open", flush=True)
    assert open_frac <= max_open, f"{what}: {open_frac:.3%} of outputs open"
    return open_frac


def check_nvfp4_against_reference(q, sc, gs, ref, mag, amax, what="", max_open=MAX_OPEN_NV):
    """NVFP4 output (codes [M, ceil(N/2)], scale bytes [M, ceil(N/16)], tensor
    scale) against the float64 reference: the tensor scale is the oracle's, every
    scale byte lies in the admissible range of its block, and at that byte every
    element's E2M1 value lies in its admissible range.  Returns the open
    fractions (blocks, elements)."""
    M, N = ref.shape
    s_g, b_lo, b_hi, (l0, h0), (l1, h1) = o.nvfp4_output_range(ref, o.GEMM_REL_TOL * mag, amax)
    assert np.float32(gs) == s_g, f"{what}: tensor scale {gs} != {s_g}"
    bad = np.argwhere((sc < b_lo) | (sc > b_hi))
    assert bad.size == 0, f"{what}: {len(bad)} scale bytes outside the admissible range, first at {tuple(bad[0])}"
    at_lo = np.repeat(sc == b_lo, 16, axis=1)[:, :N]
    at_hi = np.repeat((sc == b_hi) & (sc != b_lo), 16, axis=1)[:, :N]
    middle = ~(at_lo | at_hi)      # a byte strictly inside a range of 3 or more: not checked
    v = o.e2m1_decode(o.unpack_nibbles(q, N))
    vlo = np.where(at_lo, l0, l1)
    vhi = np.where(at_lo, h0, h1)
    ok = middle | ((v >= vlo) & (v <= vhi))
    bad = np.argwhere(~ok)
    assert bad.size == 0, (f"{what}: {len(bad)} codes outside the admissible range, first at "
                           f"{tuple(bad[0])}: {v[tuple(bad[0])]} not in [{vlo[tuple(bad[0])]}, "
                           f"{vhi[tuple(bad[0])]}]")
    blk_open = float(np.mean(b_lo != b_hi))
    el_open = float(np.mean((vlo != vhi) | middle))
    print(f"[nvfp4 parity] {what}: {b_lo.size} blocks, {blk_open:.3%} open; {v.size} elements, "
          f"{el_open:.3%} open", flush=True)
    assert float(np.mean(middle)) <= min(1e-3, max_open), f"{what}: {np.mean(middle):.3%} elements unchecked"
    assert blk_open <= max_open and el_open <= max_open, (what, blk_open, el_open)
    return blk_open, el_open
