// Device-side codecs for micro-scaled FP4 on gfx950.
//
// Every function here performs the exact float32 operation sequence stated in
// include/fp4.h; sources of the formats:
//   E2M1 values and packing: "FP4" wiki (newton.com.tw), 技術原理 (ONNX rule);
//   E4M3 block scale, s_global / s_block: "low-precision floats" blog,
//     section "FP4 / MXFP4 / NVFP4";
//   E8M0 rounded-up power of two: same section (1.99 -> 2, 2.01 -> 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two float32 values -> two bf16 in one dword (a in the low half), round to
// nearest even: one v_cvt_pk_bf16_f32 on gfx950 (finite inputs give the bits
// of f32_to_bf16).
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
}

// ---------------------------------------------------------------- E2M1 --
// Code of the nearest E2M1 magnitude (ties to the even code), saturating at 6,
// with the sign bit of q.  The thresholds are the midpoints of
// {0, .5, 1, 1.5, 2, 3, 4, 6}; a midpoint goes to its even-coded neighbour.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  uint32_t u = __float_as_uint(q);
  float m = __uint_as_float(u & 0x7fffffffu);
  uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
               (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
               (uint32_t)(m > 5.0f);
  return c | ((u >> 28) & 8u);
}

// The gfx950 conversion v_cvt_scalef32_pk_fp4_f32 with scale 1.0 encodes two
// float32 values with exactly the rounding of e2m1_code (nearest, ties to the
// even code, saturating at 6, sign kept, denormals included); it writes the
// byte (first value in the low nibble) selected by SEL of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float q0, float q1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, 1.0f, SEL);
}

// Eight float32 values -> one dword of packed codes (value 2j in the low
// nibble of byte j).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* q) {
  uint32_t d = 0;
  d = e2m1_pack2<0>(d, q[0], q[1]);
  d = e2m1_pack2<1>(d, q[2], q[3]);
  d = e2m1_pack2<2>(d, q[4], q[5]);
  d = e2m1_pack2<3>(d, q[6], q[7]);
  return d;
}

// Value of a 4-bit code as float32.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// ---------------------------------------------------------------- E4M3 --
// Nearest E4M3 (bias 7) code of t >= 0, ties to even, subnormals kept,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  if (t < 0x1p-6f) {
    // subnormal range: multiples of 2^-9; t * 512 is exact, adding 2^23 rounds
    // it to the nearest integer with ties to even.
    float s = t * 512.0f;
    s = s + 8388608.0f;
    return __float_as_uint(s) - 0x4b000000u;
  }
  uint32_t u = __float_as_uint(t);
  u = u + 0x7ffffu + ((u >> 20) & 1u);      // round the mantissa to 3 bits
  uint32_t c = (u >> 20) - (120u << 3);     // exponent bias 127 -> 7
  return c > 0x7eu ? 0x7eu : c;
}

// Four float32 values -> four signed E4M3 bytes (value q in byte q): sign,
// then the nearest magnitude with ties to the even code, subnormals kept,
// saturating at 448.  gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into
// OCP E4M3 but turns magnitudes that round past 448 into NaN (0x7F), so the
// values are clamped to [-448, 448] first (v_med3_f32).
__device__ __forceinline__ uint32_t e4m3_pack4_signed(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// NVFP4 tensor scale: s_global = G / (6 * 448), 1 for an all-zero tensor.
__device__ __forceinline__ float nv_global_scale(float G) { return G != 0.0f ? G / 2688.0f : 1.0f; }

// NVFP4 block scale byte and element multiplier for block amax A_b:
//   t = (A_b / 6) / s_global -> E4M3;  s_b = s_global * E4M3(t);  r = 1 / s_b.
// r == 0 when s_b == 0: then x * r is a signed zero and every code is sign|0.
__device__ __forceinline__ void nv_block_scale(float Ab, float s_global, uint32_t& code, float& r) {
  float t = Ab / 6.0f;
  t = t / s_global;
  code = e4m3_code(t);
  float sb = s_global * e4m3_value(code);
  r = sb != 0.0f ? 1.0f / sb : 0.0f;
}

// f16 pair (h, h), h = E4M3 value * 2^-8 exactly: the byte's exponent and
// mantissa fields drop into the f16 fields (bias 7 against 15 gives the 2^-8;
// E4M3 subnormals land on f16 subnormals), its sign on the sign.  Bytes
// 0x7f / 0xff (NaN) read as +-480; quantizers never emit them.
__device__ __forceinline__ f16x2 e4m3_h2(uint32_t byte) {
  const uint32_t h = ((byte & 0x80u) << 8) | ((byte & 0x7fu) << 7);
  return __builtin_bit_cast(f16x2, h | (h << 16));
}

// f16 pair (h(b0), h(b1)) of the two E4M3 bytes of 16-bit word SEL of w, the
// same h as e4m3_h2 for every finite byte (v_cvt_scalef32_pk_f16_fp8 with the
// scale 2^-8, one instruction for two bytes; a NaN byte gives NaN).
template <bool SEL>
__device__ __forceinline__ f16x2 e4m3_pair_h(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 0x1p-8f, SEL);
}

// The 8 values E2M1(code) * E4M3 of one dword of codes (value 2j in the low
// nibble of byte j), given s = e4m3_h2 of the scale byte: the conversion
// scales the codes by 2^8 (exact) and the f16 product with E4M3 * 2^-8 is
// exact (at most 6 significant bits, magnitude in [2^-10, 2688]).
__device__ __forceinline__ f16x8 dq8(uint32_t codes, f16x2 s) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// ---------------------------------------------------------------- E8M0 --
// MXFP4 scale byte of block amax A (bit pattern of |A|): the smallest e with
// 6 * 2^e >= A, as clamp(e + 127, 0, 254).  For A = m * 2^E (1 <= m < 2):
// e = E - 2 when m <= 1.5, else E - 1.
__device__ __forceinline__ uint32_t e8m0_code(uint32_t abits) {
  int ef = (int)(abits >> 23);
  int c = ef - 2 + (int)((abits & 0x7fffffu) > 0x400000u);
  return c < 0 ? 0u : (uint32_t)c;
}

// 2^(127 - code): the exact element multiplier of an E8M0 byte.
__device__ __forceinline__ float e8m0_inv(uint32_t code) { return __uint_as_float((254u - code) << 23); }
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  return code ? __uint_as_float(code << 23) : 0x1p-127f;
}

// ------------------------------------------------------------ LDS staging --
// Loads the VPB 16-byte vectors of each of the nb (<= NT) blocks starting at
// block `base` (each block VPB consecutive vectors) with coalesced 128-bit
// loads (lane i of a wave reads bytes [16i, 16i+16) of a contiguous run), and
// hands thread t the vectors of block base + t.  Array k of the LDS buffer
// (VPB * (NT + 1) vectors) holds vector k of every block; the arrays are skewed
// by one vector so the writes of a 16-lane group hit distinct banks.  Every
// thread of the workgroup must call it.
template <int VPB, int NT>
__device__ __forceinline__ void stage_blocks(const u32x4* __restrict__ src, int64_t base, int nb,
                                             u32x4* lds, u32x4 (&out)[VPB]) {
#pragma unroll
  for (int k = 0; k < VPB; ++k) {
    const int i = threadIdx.x + NT * k;
    if (i < VPB * nb)
      lds[(i % VPB) * (NT + 1) + i / VPB] = __builtin_nontemporal_load(src + base * VPB + i);
  }
  __syncthreads();
  if ((int)threadIdx.x < nb) {
#pragma unroll
    for (int k = 0; k < VPB; ++k) out[k] = lds[k * (NT + 1) + threadIdx.x];
  }
  __syncthreads();
}

// The same staging split in two, so a kernel can issue a chunk's loads one
// chunk ahead: chunk_load reads vectors threadIdx.x + NT k (k < VPB) of the
// chunk (past the chunk's end the address is clamped onto its last vector, so
// the loaded registers are never selected on, which would make the load wait);
// chunk_deal writes them to LDS and hands thread t its block's VPB vectors.
template <int VPB, int NT>
__device__ __forceinline__ void chunk_load(const u32x4* __restrict__ src, int64_t base, int nb,
                                           u32x4 (&raw)[VPB]) {
#pragma unroll
  for (int k = 0; k < VPB; ++k) {
    const int i = threadIdx.x + NT * k;
    const int ic = i < VPB * nb ? i : VPB * nb - 1;
    raw[k] = __builtin_nontemporal_load(src + base * VPB + ic);
  }
}

template <int VPB, int NT>
__device__ __forceinline__ void chunk_deal(const u32x4 (&raw)[VPB], int nb, u32x4* lds,
                                           u32x4 (&out)[VPB]) {
#pragma unroll
  for (int k = 0; k < VPB; ++k) {
    const int i = threadIdx.x + NT * k;
    if (i < VPB * nb) lds[(i % VPB) * (NT + 1) + i / VPB] = raw[k];
  }
  __syncthreads();
  if ((int)threadIdx.x < nb) {
#pragma unroll
    for (int k = 0; k < VPB; ++k) out[k] = lds[k * (NT + 1) + threadIdx.x];
  }
  __syncthreads();
}

// ------------------------------------------------------- wave reductions --
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace fp4dev
