"""CPU oracle for the NVFP4 / MXFP4 micro-scaling hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code, table or constant with it.

Plain, slow, obviously-correct NumPy.  Every floating-point step that the
method performs in float32 is done here with numpy float32 scalars/arrays (IEEE
round-to-nearest-even, no fused multiply-add, no reassociation).  Reference
sums for the GEMM/GEMV are exact-in-float64.

Pages cited (titles as they appear on the pages):
  [MS]   "NVIDIA NVFP4 与 Micro-Scaling：Blackwell 推理 4-bit 浮点精度的深度工程实战"
         (ybb.press engineering article)
  [DT]   the 10100.com article on mxFP4/nvFP4 data types (part 1 of 2)
  [NV]   "Introducing NVFP4 for efficient and accurate low-precision inference"
         (NVIDIA developer blog, Chinese edition)
  [LPF]  the "low-precision floats" blog (july-h5kf3.github.io), section
         "FP4 / MXFP4 / NVFP4"
  [WIKI] the "FP4" wiki page (newton.com.tw), sections 技術原理 / 技術實現與量化方法

Readings where the pages are silent or disagree (each is also listed in the
design notes):
  * two-level convention: [LPF] s_global = amax/(6*448), s_block = (block_amax/6)/s_global
  * E4M3 block scale rounded to nearest, ties to even ([DT] picks 0.875 for 0.9),
    saturating at 448; subnormals kept; E4M3 bias 7
  * E8M0 scale = the smallest power of two 2^e with 6*2^e >= block amax, i.e. the
    "rounded up" choice of [LPF] (1.99 -> 2, 2.01 -> 4); bias 127, codes 0..254
  * E2M1 element rounding: nearest, ties to the even code, saturating at +-6
    ([MS] section 二: values above 6 are clipped); sign bit copied from the input
  * element step done as q = x * fl(1/fl(s_global*s_block)) (one reciprocal per
    block); for MXFP4 this is an exact power-of-two multiply
  * global amax 0 -> s_global = 1; a block scale that encodes to 0 makes every
    element code of the block (sign|0)
  * blocks run along the last (K / channel) dimension; a last partial block
    covers the remaining columns; rows are ceil(cols/2) bytes, first element in
    the low nibble ([WIKI] 技術原理, ONNX packing)
  * Hadamard: orthonormal Sylvester-order FWHT over 128 contiguous channels,
    butterfly stages h = 1, 2, 4, ..., 64 in float32, then one multiply by
    fl32(1/sqrt(128)); global amax taken over the rotated tensor
  * stochastic rounding: element rounding only; the position inside the E2M1
    interval, truncated to 22 bits, plus 64 times 16 random bits per element
    carries into the code (round up with probability floor(f 2^16) / 2^16 for
    position f); the bits come from Philox4x32-10 (Salmon et al., "Parallel
    random numbers: as easy as 1, 2, 3", SC'11) keyed by the 64-bit seed,
    counter = flat element index // 8, bits taken 16 at a time, low half first
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F64 = np.float64

# ------------------------------------------------------------------ E2M1 ----
# [WIKI] 技術原理: ONNX FLOAT4E2M1 value rule.  Exponent field E != 0:
#   (-1)^S * 2^(E-1) * (1 + M/2);  E == 0: (-1)^S * M/2.
# [DT] "nvFP4的数据结构设计" lists the 16 values in code order
# [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0, -0.5, ..., -6]; [MS] section 二 gives the
# same table (its E=0 formula is garbled; the table and the ONNX rule agree).


def e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=F64)
E2M1_MAGNITUDES = E2M1_VALUES[:8].copy()          # 0, .5, 1, 1.5, 2, 3, 4, 6
E2M1_MAX = 6.0                                     # [MS] section 二: max is 6.0


def _nearest_code(table: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Index of the entry of the strictly increasing table nearest to v (v >= 0),
    ties resolved to the even index.  Distances are compared in float64; the
    callers clip v so that every comparison near a tie is exact."""
    v = np.asarray(v, dtype=F64)
    hi = np.searchsorted(table, v, side="left")            # first entry >= v
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = np.abs(v - table[lo])
    d_hi = np.abs(table[hi] - v)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.int64)


def e2m1_encode_rne(q: np.ndarray) -> np.ndarray:
    """E2M1 code of each float32 q: nearest of the 8 magnitudes (ties to the
    even code), saturating at 6, sign bit from q ([LPF] Q_E2M1; [MS] section 二
    clipping above 6).  Returns uint8 codes 0..15."""
    q = np.asarray(q, dtype=F32)
    # Every magnitude >= 8 has 6 as its nearest value; clipping at 8 keeps the
    # float64 distances exact (|q| has at most 24 significant bits).
    m = np.minimum(np.abs(q).astype(F64), 8.0)
    code = _nearest_code(E2M1_MAGNITUDES, m)
    sign = np.signbit(q).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64) & 15]


# ------------------------------------------------------------------ E4M3 ----
# FP8 E4M3 ("fn" variant, torch.float8_e4m3fn per [DT]): bias 7, subnormals
# M/8 * 2^-6, no infinities, S.1111.111 is NaN, max 448 = 1.75 * 2^8
# ([MS] section 二 and [LPF] both give 448 as the E4M3 maximum).


def e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=F64)
E4M3_POS = E4M3_VALUES[:127].copy()                # codes 0..126, strictly increasing
E4M3_MAX = 448.0


def e4m3_encode_rne_sat(t: np.ndarray) -> np.ndarray:
    """E4M3 code of each non-negative float32 t: nearest finite value, ties to
    the even code; values above 448 saturate to 448 (code 0x7E)."""
    t = np.asarray(t, dtype=F32)
    v = np.minimum(t.astype(F64), 512.0)             # nearest finite of any t >= 448 is 448
    return _nearest_code(E4M3_POS, v).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.int64)]


def e4m3_encode_signed(x: np.ndarray) -> np.ndarray:
    """FP8 E4M3 byte of each float32 x (the GEMM's E4M3 output): sign bit of x,
    then the nearest finite magnitude, ties to the even code, saturating at 448
    ([MS] section 五: the scaled-mm example writes its output as
    torch.float8_e4m3fn after g_d; the kernel sketch there notes that the
    output is often stored as FP8).  Saturation, not NaN, above 448 is a
    reading: E4M3 "fn" has no infinity and the block-scale codec saturates."""
    x = np.asarray(x, dtype=F32)
    sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
    return (sign | e4m3_encode_rne_sat(np.abs(x))).astype(np.uint8)


# ------------------------------------------------------------------ E8M0 ----
# MXFP4 block scale: one power of two per 32 values ([DT] "mxFP4的技术局限";
# [NV] Table 1).  [LPF] "FP4 / MXFP4 / NVFP4": the ideal scale is A/6 and the
# power of two is rounded up (1.99 -> 2, 2.01 -> 4).  Bias 127 as for float32's
# exponent; codes clamped to 0..254 (255 is NaN).


def e8m0_exponent(block_amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with 6 * 2^e >= A (A > 0), tested exactly in float64.
    Returns the E8M0 code clamp(e + 127, 0, 254); A == 0 gives code 0."""
    A = np.asarray(block_amax, dtype=F32).astype(F64)
    pos = A > 0
    safe = np.where(pos, A, 1.0)
    e = np.ceil(np.log2(safe / 6.0)).astype(np.int64)
    # log2 is rounded: fix e up or down until it is the smallest exact solution.
    for _ in range(3):
        e = np.where(np.ldexp(6.0, e) < safe, e + 1, e)
        e = np.where(np.ldexp(6.0, e - 1) >= safe, e - 1, e)
    code = np.clip(e + 127, 0, 254)
    return np.where(pos, code, 0).astype(np.uint8)


def e8m0_value(codes: np.ndarray) -> np.ndarray:
    return np.ldexp(1.0, np.asarray(codes, dtype=np.int64) - 127)


# ------------------------------------------------------------- float32/bf16 --
def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact (bf16 is the top half of a float32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits by round-to-nearest-even on the dropped 16 bits
    (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_bits(x) -> int:
    """IEEE-754 single bit pattern ([LPF] "IEEE 754 标准浮点数": 1 sign, 8 exponent
    bits with bias 127, 23 fraction bits)."""
    return int(np.array(x, dtype=F32).view(np.uint32))


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=F32)


# ------------------------------------------------------------------ packing --
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R, C] codes -> [R, ceil(C/2)] bytes; element 2j in the low nibble of
    byte j, element 2j+1 in the high nibble ([WIKI] 技術原理: ONNX packs the first
    element in the low 4 bits; ceil(N/2) bytes).  An odd row's last high nibble is 0."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    nb = (C + 1) // 2
    padded = np.zeros((R, 2 * nb), dtype=np.uint8)
    padded[:, :C] = codes & 15
    return (padded[:, 0::2] | (padded[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, cols: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    R = packed.shape[0]
    out = np.empty((R, 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out[:, :cols]


def _blocks(x: np.ndarray, bs: int) -> np.ndarray:
    """[R, C] -> [R, ceil(C/bs), bs] with a zero-padded last partial block."""
    R, C = x.shape
    nb = -(-C // bs)
    out = np.zeros((R, nb * bs), dtype=x.dtype)
    out[:, :C] = x
    return out.reshape(R, nb, bs)


# ----------------------------------------------------------------- NVFP4 ----
NV_BLOCK = 16
MX_BLOCK = 32
NV_GLOBAL_DIV = F32(6.0 * 448.0)   # [LPF]: s_global = global_amax / (6 x 448)


def global_amax(x: np.ndarray) -> np.float32:
    x = np.asarray(x, dtype=F32)
    return F32(np.max(np.abs(x))) if x.size else F32(0.0)


def nv_global_scale(G) -> np.float32:
    """[LPF] "FP4 / MXFP4 / NVFP4": s_global = global_amax / (6 * 448) (float32
    division).  A zero amax gives 1 (reading: any value works, 1 is plainest)."""
    G = F32(G)
    return F32(G / NV_GLOBAL_DIV) if G != 0 else F32(1.0)


def nvfp4_quantize(x: np.ndarray, amax=None, rounding: str = "rne", sr_bits=None):
    """Two-level NVFP4 quantization of a float32 [R, C] tensor.

    [LPF] "FP4 / MXFP4 / NVFP4": s_global = amax/(6*448); s_block =
    (block_amax/6)/s_global stored as E4M3; x_hat = s_global*s_block*Q(x/(s_global*s_block)).
    [NV] "二级微块 scaling": one E4M3 scale per 16 values plus one FP32 per tensor.

    Steps (float32):
      1. G = max|x| (or the given static amax); s_global = fl(G / 2688).
      2. per 16-value block: A_b = max|x_i|; t = fl(fl(A_b / 6) / s_global);
         scale byte = E4M3(t) (nearest, ties even, saturating).
      3. s_b = fl(s_global * E4M3value(byte)); r_b = fl(1 / s_b).
      4. q_i = fl(x_i * r_b); code_i = E2M1(q_i) (or stochastic, see sr_round);
         a block whose s_b is 0 gets code (sign|0) everywhere.
    Returns (packed codes [R, ceil(C/2)] u8, scale bytes [R, ceil(C/16)] u8,
             G float32, s_global float32).
    """
    x = np.asarray(x, dtype=F32)
    R, C = x.shape
    G = global_amax(x) if amax is None else F32(amax)
    s_global = nv_global_scale(G)
    xb = _blocks(x, NV_BLOCK)
    A_b = np.max(np.abs(xb), axis=-1).astype(F32)
    t = ((A_b / F32(6.0)).astype(F32) / s_global).astype(F32)
    sbyte = e4m3_encode_rne_sat(t)
    s_b = (s_global * e4m3_decode(sbyte).astype(F32)).astype(F32)
    nz = s_b != 0
    r_b = np.where(nz, F32(1.0) / np.where(nz, s_b, F32(1.0)), F32(0.0)).astype(F32)
    q = (xb * r_b[..., None]).astype(F32)
    if rounding == "rne":
        codes = e2m1_encode_rne(q)
    elif rounding == "sr":
        codes = sr_round(q, _blocks(np.asarray(sr_bits, dtype=np.uint16), NV_BLOCK))
    else:
        raise ValueError(rounding)
    zero_blk = ~nz
    if zero_blk.any():
        codes = np.where(zero_blk[..., None], (np.signbit(xb).astype(np.uint8) << 3), codes)
    codes = codes.reshape(R, -1)[:, :C]
    return pack_nibbles(codes), sbyte, G, s_global


def nvfp4_dequantize(packed, sbytes, s_global, cols: int) -> np.ndarray:
    """x_hat = fl(s_b * v) with s_b = fl(s_global * E4M3value(byte)) ([LPF]
    x_hat = s_global * s_block * Q(.)).  Returns float32 [R, cols]."""
    codes = unpack_nibbles(packed, cols)
    R = codes.shape[0]
    v = e2m1_decode(codes).astype(F32)
    s_b = (F32(s_global) * e4m3_decode(sbytes).astype(F32)).astype(F32)
    s_el = np.repeat(s_b, NV_BLOCK, axis=1)[:, :cols]
    return (s_el * v).astype(F32).reshape(R, cols)


# ------------------------------------------------- NVFP4 scale variants ----
# [MS] section 3.1: block sizes 8, 16 and 32, finer blocks recover local
# dynamic range better at a higher scale overhead.  [NV] "高精度缩放": E4M3
# block scales can be chosen so that the block's summed squared (or absolute)
# error is as small as possible, rather than fixed by the block amax.
E4M3_MAX_CODE = 126                     # 0x7E = 448; 0x7F is NaN


def _search_order(window: int):
    """Code offsets in the order the search visits them: 0, -1, +1, -2, +2, ..."""
    out = [0]
    for d in range(1, window + 1):
        out += [-d, d]
    return out


def nv_block_sq_error(xb: np.ndarray, s_b: np.ndarray) -> np.ndarray:
    """float32 squared error of encoding blocks xb [..., n] with scale s_b [...]:
    r = fl(1/s_b) (0 when s_b == 0), v_i = E2M1 value of fl(x_i * r),
    x_hat_i = fl(s_b * v_i), E = sum_i fl(fl(x_i - x_hat_i)^2), summed in index
    order in float32 (the order and precision the search decides in)."""
    xb = np.asarray(xb, dtype=F32)
    s_b = np.asarray(s_b, dtype=F32)
    nz = s_b != 0
    r = np.where(nz, F32(1.0) / np.where(nz, s_b, F32(1.0)), F32(0.0)).astype(F32)
    v = e2m1_decode(e2m1_encode_rne((xb * r[..., None]).astype(F32))).astype(F32)
    xh = (s_b[..., None] * v).astype(F32)
    d = (xb - xh).astype(F32)
    sq = (d * d).astype(F32)
    E = np.zeros(xb.shape[:-1], dtype=F32)
    for i in range(xb.shape[-1]):
        E = (E + sq[..., i]).astype(F32)
    return E


def nvfp4_quantize_ex(x: np.ndarray, block: int = NV_BLOCK, search: int = 0, amax=None):
    """NVFP4 with blocks of `block` values (8, 16 or 32) along the last dim and
    an optional search for the E4M3 scale byte.

    search == 0: the amax rule of nvfp4_quantize (code0 = E4M3(fl(fl(A_b/6) /
    s_global)), nearest, ties even).  search = W > 0: the candidates code0 + d
    for d = 0, -1, +1, ..., -W, +W inside 0..126 are visited in that order and
    a candidate replaces the current choice only when its float32 squared
    error (nv_block_sq_error) is strictly smaller; the elements are then
    encoded with the chosen scale exactly as nvfp4_quantize does.
    Returns (packed codes [R, ceil(C/2)], scale bytes [R, ceil(C/block)], G,
    s_global)."""
    if block not in (8, 16, 32):
        raise ValueError(block)
    x = np.asarray(x, dtype=F32)
    R, C = x.shape
    G = global_amax(x) if amax is None else F32(amax)
    s_global = nv_global_scale(G)
    xb = _blocks(x, block)
    A_b = np.max(np.abs(xb), axis=-1).astype(F32)
    t = ((A_b / F32(6.0)).astype(F32) / s_global).astype(F32)
    code = e4m3_encode_rne_sat(t).astype(np.int64)
    if search > 0:
        code0 = code.copy()
        best = nv_block_sq_error(xb, (s_global * e4m3_decode(code0).astype(F32)).astype(F32))
        for d in _search_order(search)[1:]:
            c = code0 + d
            ok = (c >= 0) & (c <= E4M3_MAX_CODE)
            cc = np.clip(c, 0, E4M3_MAX_CODE)
            E = nv_block_sq_error(xb, (s_global * e4m3_decode(cc).astype(F32)).astype(F32))
            take = ok & (E < best)
            code = np.where(take, cc, code)
            best = np.where(take, E, best)
    sbyte = code.astype(np.uint8)
    s_b = (s_global * e4m3_decode(sbyte).astype(F32)).astype(F32)
    nz = s_b != 0
    r_b = np.where(nz, F32(1.0) / np.where(nz, s_b, F32(1.0)), F32(0.0)).astype(F32)
    q = (xb * r_b[..., None]).astype(F32)
    codes = e2m1_encode_rne(q)
    codes = np.where(~nz[..., None], (np.signbit(xb).astype(np.uint8) << 3), codes)
    codes = codes.reshape(R, -1)[:, :C]
    return pack_nibbles(codes), sbyte, G, s_global


def nvfp4_dequantize_ex(packed, sbytes, s_global, cols: int, block: int = NV_BLOCK) -> np.ndarray:
    """nvfp4_dequantize for blocks of `block` values."""
    codes = unpack_nibbles(packed, cols)
    R = codes.shape[0]
    v = e2m1_decode(codes).astype(F32)
    s_b = (F32(s_global) * e4m3_decode(sbytes).astype(F32)).astype(F32)
    s_el = np.repeat(s_b, block, axis=1)[:, :cols]
    return (s_el * v).astype(F32).reshape(R, cols)


# ----------------------------------------------------------------- MXFP4 ----
def mxfp4_quantize(x: np.ndarray):
    """MXFP4: E2M1 values with one E8M0 power-of-two scale per 32 values and no
    tensor scale ([DT] "mxFP4的技术局限"; [NV] Table 1; [LPF] s_mx rule).
    q_i = x_i * 2^-e (exact), code_i = E2M1(q_i).
    Returns (packed codes [R, ceil(C/2)], scale bytes [R, ceil(C/32)])."""
    x = np.asarray(x, dtype=F32)
    R, C = x.shape
    xb = _blocks(x, MX_BLOCK)
    A_b = np.max(np.abs(xb), axis=-1).astype(F32)
    sbyte = e8m0_exponent(A_b)
    inv = np.ldexp(F32(1.0), 127 - sbyte.astype(np.int32)).astype(F32)   # 2^-(code-127), exact
    q = (xb * inv[..., None]).astype(F32)
    codes = e2m1_encode_rne(q).reshape(R, -1)[:, :C]
    return pack_nibbles(codes), sbyte


def mxfp4_dequantize(packed, sbytes, cols: int) -> np.ndarray:
    codes = unpack_nibbles(packed, cols)
    v = e2m1_decode(codes)
    s = np.repeat(e8m0_value(sbytes), MX_BLOCK, axis=1)[:, :cols]
    return (v * s).astype(F32)                                  # exact in range


# -------------------------------------------------------------- Hadamard ----
HADAMARD_GROUP = 128
HADAMARD_NORM = F32(1.0 / math.sqrt(128.0))   # fl32(1/sqrt(128))


def fwht_orthonormal(x: np.ndarray, group: int = HADAMARD_GROUP) -> np.ndarray:
    """Rotate every `group` contiguous channels by the orthonormal Hadamard
    matrix ([MS] section 4.1: x @ H with H @ H.T = I, done as a fast
    Walsh-Hadamard transform).  Sylvester (natural) order; butterfly stages
    h = 1, 2, 4, ..., group/2, each (a, b) -> (a+b, a-b) in float32; then one
    float32 multiply by fl32(1/sqrt(group))."""
    x = np.asarray(x, dtype=F32)
    R, C = x.shape
    assert C % group == 0
    y = x.reshape(R, C // group, group).copy()
    h = 1
    while h < group:
        v = y.reshape(R, C // group, group // (2 * h), 2, h)
        a = v[:, :, :, 0, :]
        b = v[:, :, :, 1, :]
        y = np.stack([(a + b).astype(F32), (a - b).astype(F32)], axis=3).reshape(R, C // group, group)
        h *= 2
    norm = F32(1.0 / math.sqrt(float(group)))
    return (y.reshape(R, C) * norm).astype(F32)


# ------------------------------------------------------ stochastic rounding --
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC'11): 10 rounds; each round multiplies words 0 and 2 by the
# two Philox constants, takes the 64-bit products' halves and xors them with
# words 1, 3 and the round key; the key is bumped by the Weyl constants between
# rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 on uint64 arrays holding 32-bit words."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    k0 = np.uint64(k0 & MASK32)
    k1 = np.uint64(k1 & MASK32)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        p0 = c0 * np.uint64(PHILOX_M0)
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def sr_bits_at(flat_index: np.ndarray, seed: int) -> np.ndarray:
    """16 random bits for each given flat element index i of a row-major tensor:
    Philox4x32-10 with counter (i//8 low word, i//8 high word, 0, 0) and key
    (seed low word, seed high word); output word (i%8)//2, its low 16 bits for
    even i%8 and high 16 bits for odd."""
    i = np.asarray(flat_index, dtype=np.uint64)
    g = i // np.uint64(8)
    w = philox4x32_10(g & np.uint64(MASK32), g >> np.uint64(32), 0, 0, seed & MASK32, (seed >> 32) & MASK32)
    words = np.stack(w, axis=-1)
    j = (i % np.uint64(8)).astype(np.int64)
    word = np.take_along_axis(words, (j // 2)[..., None], axis=-1)[..., 0]
    return np.where(j % 2 == 0, word & np.uint64(0xFFFF), word >> np.uint64(16)).astype(np.uint16)


def sr_bits(rows: int, cols: int, seed: int) -> np.ndarray:
    """sr_bits_at for every element of a [rows, cols] tensor."""
    return sr_bits_at(np.arange(rows * cols, dtype=np.uint64), seed).reshape(rows, cols)


def sr_round(q: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Stochastic E2M1 rounding ([WIKI] 技術實現與量化方法 names stochastic
    rounding as the NVFP4 element rounding option).  For lo <= |q| < hi adjacent
    E2M1 magnitudes and f = (|q|-lo)/(hi-lo), the position's top 22 bits
    D = floor(f * 2^22) plus 64 * u16 carry into the code: up to hi iff
    D + 64 * u16 >= 2^22 (probability floor(f * 2^16) / 2^16 for uniform u16).
    |q| >= 6 gives 6.  Sign from q."""
    q = np.asarray(q, dtype=F32)
    m = np.abs(q).astype(F64)
    mags = E2M1_MAGNITUDES
    lo_idx = np.clip(np.searchsorted(mags, m, side="right") - 1, 0, 7)
    hi_idx = np.minimum(lo_idx + 1, 7)
    lo = mags[lo_idx]
    hi = mags[hi_idx]
    span = np.where(hi_idx > lo_idx, hi - lo, 1.0)
    frac = np.where(hi_idx > lo_idx, (m - lo) / span, 0.0)   # exact in float64
    D = np.floor(frac * 2.0 ** 22)
    up = D + 64.0 * np.asarray(bits, dtype=F64) >= 2.0 ** 22
    code = np.where(up, hi_idx, lo_idx)
    sign = np.signbit(q).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def hadamard_quantize(x: np.ndarray, group: int = HADAMARD_GROUP, rounding: str = "rne",
                      seed: int = 0, amax=None):
    """FWHT rotation fused with NVFP4 quantization: the global amax (dynamic
    unless given) is that of the rotated tensor; stochastic rounding, when
    selected, applies to the element codes only.  Returns what nvfp4_quantize
    returns."""
    y = fwht_orthonormal(x, group)
    bits = sr_bits(*y.shape, seed) if rounding == "sr" else None
    return nvfp4_quantize(y, amax=amax, rounding=rounding, sr_bits=bits)


def hadamard_quantize_mx(x: np.ndarray, group: int = HADAMARD_GROUP, rounding: str = "rne",
                         seed: int = 0):
    """FWHT rotation fused with MXFP4 quantization ([MS] section 4.1 rotation,
    then mxfp4_quantize's E8M0 rule per 32 rotated values).  MXFP4 has no
    tensor scale, so nothing waits for a global amax.  Stochastic rounding, when
    selected, rounds q_i = y_i * 2^-e with the same 16-bit draws per flat
    element index as hadamard_quantize.
    Returns (packed codes [R, C/2], E8M0 bytes [R, C/32])."""
    y = fwht_orthonormal(x, group)
    if rounding == "rne":
        return mxfp4_quantize(y)
    if rounding != "sr":
        raise ValueError(rounding)
    R, C = y.shape
    yb = _blocks(y, MX_BLOCK)
    sbyte = e8m0_exponent(np.max(np.abs(yb), axis=-1).astype(F32))
    inv = np.ldexp(F32(1.0), 127 - sbyte.astype(np.int32)).astype(F32)
    q = (yb * inv[..., None]).astype(F32)
    codes = sr_round(q, _blocks(sr_bits(R, C, seed), MX_BLOCK)).reshape(R, -1)[:, :C]
    return pack_nibbles(codes), sbyte


def rotated_fp4_linear(x: np.ndarray, W: np.ndarray, group: int = HADAMARD_GROUP,
                       fmt: str = "nv"):
    """A linear layer y = x @ W^T run through the FP4 GEMM with both operands
    rotated along K ([MS] section 4.1: the rotation of the activations can be
    absorbed into the adjacent weights, so (x H)(W H)^T = x H H^T W^T = x W^T
    for orthonormal H): x H and W H are each quantized as hadamard_quantize
    (fmt "nv") or hadamard_quantize_mx (fmt "mx") does (W H once, offline),
    then multiplied exactly.  Returns (D_ref float64 [M, N], the tolerance
    magnitude, the two quantized operands)."""
    K = x.shape[1]
    if fmt == "nv":
        qx = hadamard_quantize(x, group)
        qw = hadamard_quantize(W, group)
        D, mag = scaled_gemm_ref(nv_operand_f64(qx[0], qx[1], qx[3], K),
                                 nv_operand_f64(qw[0], qw[1], qw[3], K), 1.0)
    else:
        qx = hadamard_quantize_mx(x, group)
        qw = hadamard_quantize_mx(W, group)
        D, mag = scaled_gemm_ref(mx_operand_f64(qx[0], qx[1], K), mx_operand_f64(qw[0], qw[1], K), 1.0)
    return D, mag, qx, qw


# -------------------------------------------------------------- GEMM/GEMV ---
def nv_operand_f64(packed, sbytes, g, cols: int) -> np.ndarray:
    """Exact float64 value of an NVFP4 operand: g * E4M3(s_b) * E2M1(v)."""
    v = e2m1_decode(unpack_nibbles(packed, cols))
    s = np.repeat(e4m3_decode(sbytes), NV_BLOCK, axis=1)[:, :cols]
    return float(g) * s * v


def mx_operand_f64(packed, sbytes, cols: int) -> np.ndarray:
    v = e2m1_decode(unpack_nibbles(packed, cols))
    s = np.repeat(e8m0_value(sbytes), MX_BLOCK, axis=1)[:, :cols]
    return s * v


def scaled_gemm_ref(A_hat: np.ndarray, W_hat: np.ndarray, g_d: float):
    """D_ref = g_d * A_hat @ W_hat^T in float64 ([MS] section 三: D = g_d *
    ((g_a s_a . A) @ (g_b s_b . W)); the concept API passes W.t(), so both
    operands are K-major).  Also returns the error scale
    |g_d| * sum_k |A_hat_ik * W_hat_jk| used by the acceptance rule."""
    A_hat = np.asarray(A_hat, dtype=F64)
    W_hat = np.asarray(W_hat, dtype=F64)
    D = float(g_d) * (A_hat @ W_hat.T)
    mag = abs(float(g_d)) * (np.abs(A_hat) @ np.abs(W_hat).T)
    return D, mag


def grouped_gemm_ref(A_hat: np.ndarray, W_hat: np.ndarray, offsets, g_d: float):
    """Grouped GEMM (one launch over E GEMMs, e.g. the experts of an MoE layer;
    [MS] section 6.1 names MoE expert weights as the NVFP4 candidates): rows
    offsets[e] .. offsets[e+1] of A_hat [M, K] times W_hat[e] [N, K] transposed,
    each exactly as scaled_gemm_ref.  Rows outside every group stay NaN (not
    written).  Returns (D [M, N], magnitude [M, N]) in float64."""
    A_hat = np.asarray(A_hat, dtype=F64)
    E, N, _ = W_hat.shape
    D = np.full((A_hat.shape[0], N), np.nan)
    mag = np.full((A_hat.shape[0], N), np.nan)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            D[lo:hi], mag[lo:hi] = scaled_gemm_ref(A_hat[lo:hi], W_hat[e], g_d)
    return D, mag


GEMM_REL_TOL = 1e-5            # |D - D_ref| <= 1e-5 * |g_d| * sum |a*b|
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def gemm_e4m3_output(D_f32: np.ndarray) -> np.ndarray:
    """The GEMM's E4M3 output from its float32 result D = fl(acc * alpha): one
    E4M3 byte per element (e4m3_encode_signed)."""
    return e4m3_encode_signed(np.asarray(D_f32, dtype=F32))


def gemm_nvfp4_output(D_f32: np.ndarray, amax):
    """The GEMM's NVFP4 output from its float32 result D = fl(acc * alpha): the
    next layer's input quantization done on the GEMM's result ([MS] section 三:
    the output is rescaled by g_d and stored at low precision; section 五: the
    tensor scales come from calibration).  The tensor amax is a given
    (calibrated) value: the global scale must be known before any output block
    is encoded, and the GEMM writes blocks as it finishes them.  Blocks of 16
    run along N, exactly as nvfp4_quantize with a static amax.
    Returns (codes [M, ceil(N/2)], scale bytes [M, ceil(N/16)], G, s_global)."""
    return nvfp4_quantize(np.asarray(D_f32, dtype=F32), amax=amax)


def f32_interval(D_ref, tol):
    """Every float32 value v with |v - D_ref| <= tol lies in [lo, hi], with lo, hi
    the float32 roundings of D_ref -+ tol (rounding to float32 is monotone, and
    v is its own rounding).  tol is widened by a relative 1e-6 so that neither
    the float64 rounding of D_ref -+ tol nor the float64 summation error of a
    reference dot product can move an end inside.  Returns float32 (lo, hi)."""
    D = np.asarray(D_ref, dtype=F64)
    t = np.asarray(tol, dtype=F64) * (1.0 + 1e-6)
    return (D - t).astype(F32), (D + t).astype(F32)


def e4m3_output_range(D_ref, tol):
    """Values the GEMM's E4M3 output can take when its float32 result lies within
    tol of the exact D_ref ([MS] section 五: the scaled-mm output written as
    float8_e4m3fn after g_d): [E4M3(lo), E4M3(hi)] decoded, (lo, hi) =
    f32_interval(D_ref, tol).  The encoder (sign, then the nearest magnitude,
    saturating) never decreases with its input, so every float32 in [lo, hi]
    encodes to a value inside the range; equal ends fix the output value (a
    zero's sign is fixed only when lo and hi have one sign).
    Returns float64 (v_lo, v_hi)."""
    lo, hi = f32_interval(D_ref, tol)
    return e4m3_decode(e4m3_encode_signed(lo)), e4m3_decode(e4m3_encode_signed(hi))


def _nv_scale_byte(block_amax, s_global):
    """E4M3 block-scale byte of nvfp4_quantize's step 2 for block amaxes A_b."""
    A_b = np.asarray(block_amax, dtype=F32)
    t = ((A_b / F32(6.0)).astype(F32) / F32(s_global)).astype(F32)
    return e4m3_encode_rne_sat(t)


def nvfp4_output_range(D_ref, tol, amax):
    """NVFP4 encodings ([LPF] two-level scaling, blocks of 16 along N, tensor
    amax given) of every float32 result that lies within tol of the exact
    D_ref [M, N].  With (lo, hi) = f32_interval(D_ref, tol):
      * s_global = fl(amax / 2688) (1 when amax is 0) is fixed;
      * a block's amax lies between the largest of its elements' smallest
        possible magnitudes (0 when lo <= 0 <= hi) and the largest of their
        largest; the scale byte never decreases with the block amax, so it
        lies in [byte_lo, byte_hi] (the bytes of those two amaxes);
      * at scale byte c, with r = fl(1 / fl(s_global * E4M3(c))) >= 0, an
        element's E2M1 value E2M1(fl(x * r)) never decreases with x, so it lies
        in [E2M1(fl(lo * r)), E2M1(fl(hi * r))].
    Returns (s_global, byte_lo [M, nb], byte_hi [M, nb], (v_lo, v_hi) at byte_lo,
    (v_lo, v_hi) at byte_hi), element values float64 [M, N]."""
    lo, hi = f32_interval(D_ref, tol)
    M, N = lo.shape
    s_global = nv_global_scale(F32(amax))
    straddle = (lo <= 0) & (hi >= 0)
    a_small = np.where(straddle, F32(0.0), np.minimum(np.abs(lo), np.abs(hi))).astype(F32)
    a_large = np.maximum(np.abs(lo), np.abs(hi)).astype(F32)
    byte_lo = _nv_scale_byte(np.max(_blocks(a_small, NV_BLOCK), axis=-1), s_global)
    byte_hi = _nv_scale_byte(np.max(_blocks(a_large, NV_BLOCK), axis=-1), s_global)

    def values_at(sbyte):
        s_b = (s_global * e4m3_decode(sbyte).astype(F32)).astype(F32)
        nz = s_b != 0
        r = np.where(nz, F32(1.0) / np.where(nz, s_b, F32(1.0)), F32(0.0)).astype(F32)
        r = np.repeat(r, NV_BLOCK, axis=1)[:, :N]
        return (e2m1_decode(e2m1_encode_rne((lo * r).astype(F32))),
                e2m1_decode(e2m1_encode_rne((hi * r).astype(F32))))

    return s_global, byte_lo, byte_hi, values_at(byte_lo), values_at(byte_hi)


def gemm_within_tolerance(D, D_ref, mag, out_bf16: bool = False):
    """Acceptance rule for GEMM/GEMV outputs: fp32 outputs within 1e-5 of the
    magnitude sum; bf16 outputs additionally allowed one bf16 rounding of D_ref."""
    D = np.asarray(D, dtype=F64)
    bound = GEMM_REL_TOL * mag
    if out_bf16:
        bound = bound + BF16_UNIT_ROUNDOFF * np.abs(D_ref)
    err = np.abs(D - D_ref)
    return bool(np.all(err <= bound)), err, bound


def gemv_ref(x: np.ndarray, Wq, Ws, g_w, g_d: float, K: int):
    """Batched GEMV: x [B, K] float32 is NVFP4-quantized on the fly with one
    dynamic tensor scale over all of [B, K] (bit-identical to nvfp4_quantize);
    y = g_d * x_hat @ W_hat^T in float64."""
    xq, xs, G, s_g = nvfp4_quantize(x)
    X_hat = nv_operand_f64(xq, xs, s_g, K)
    W_hat = nv_operand_f64(Wq, Ws, g_w, K)
    return scaled_gemm_ref(X_hat, W_hat, g_d)
