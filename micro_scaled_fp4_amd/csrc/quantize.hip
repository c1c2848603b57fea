// NVFP4 / MXFP4 quantization and dequantization kernels for gfx950.
//
// Encode: one lane owns one whole scale block (16 values for NVFP4, 32 for
// MXFP4), so the block amax, the scale and the codes need no cross-lane
// traffic.  A workgroup stages 256 consecutive blocks through LDS: every global
// load instruction is fully coalesced (lane i reads bytes [16i, 16i+16) of a
// contiguous run), then each lane reads its own block back from LDS.  Codes are
// written with 64/128-bit stores at consecutive lane addresses.
//
// Decode: one lane owns 8 output values (bf16: one 16-byte store) or 4 (float32:
// one 16-byte store), so stores are fully coalesced too.
//
// The "fast" kernels treat the tensor as one flat run of blocks; they need
// cols to be a multiple of the block and 16-byte aligned pointers.  The
// "generic" kernels take any shape and alignment (partial last blocks, odd
// rows) with scalar accesses.
#include <atomic>

#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 2048;      // 256 CUs x 8 workgroups, grid-stride beyond
constexpr int kAmaxThreads = 512;   // amax pass: 1024 workgroups x 8 waves fill every CU

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Workgroup max of a u32 (every thread gets the result).
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[NT / 64];
  v = wave_max_u32(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = umax(r, red[i]);
  __syncthreads();
  return r;
}

// Global amax from the partials of the first pass, or the given static amax.
__device__ __forceinline__ float resolve_amax(const float* amax_in, const uint32_t* partials,
                                              int npart) {
  if (partials == nullptr) return *amax_in;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = umax(m, partials[i]);
  return __uint_as_float(block_max_u32<>(m));
}

__device__ __forceinline__ u16x2 pkmax_abs(u16x2 m, uint32_t w) {
  const uint32_t a = w & 0x7fff7fffu;
  u16x2 av;
  __builtin_memcpy(&av, &a, 4);
  return __builtin_elementwise_max(m, av);
}

template <int N>
__device__ __forceinline__ void unpack_bf16(const u32x4* w, float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N / 8; ++k) {
    const uint32_t a[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * k + 2 * j] = bf16_lo(a[j]);
      v[8 * k + 2 * j + 1] = bf16_hi(a[j]);
    }
  }
}

template <int N>
__device__ __forceinline__ void unpack_f32(const u32x4* w, float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    v[4 * k] = __uint_as_float(w[k].x);
    v[4 * k + 1] = __uint_as_float(w[k].y);
    v[4 * k + 2] = __uint_as_float(w[k].z);
    v[4 * k + 3] = __uint_as_float(w[k].w);
  }
}

template <int N>
__device__ __forceinline__ float amax_of(const float (&v)[N]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) m = umax(m, __float_as_uint(v[j]) & 0x7fffffffu);
  return __uint_as_float(m);
}

// ------------------------------------------------------------------ amax --
// Per-workgroup max|x| over a contiguous range of 16-byte vectors, four
// vectors in flight per thread; bf16 pairs are reduced with packed u16 max on
// their magnitude bits (same order as the values).
template <bool BF16>
__global__ void __launch_bounds__(kAmaxThreads) k_amax(const void* __restrict__ x, int64_t n,
                                                       uint32_t* __restrict__ partials) {
  constexpr int kPer = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int64_t nvec = n / kPer;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int64_t chunk = ((nvec + gridDim.x - 1) / gridDim.x + 4 * kAmaxThreads - 1) /
                        (4 * kAmaxThreads) * (4 * kAmaxThreads);
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < nvec ? lo + chunk : nvec;
  u16x2 mh = {0, 0};
  uint32_t mf = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 4 * kAmaxThreads) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = (i + u * kAmaxThreads < hi) ? __builtin_nontemporal_load(xv + i + u * kAmaxThreads)
                                         : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (BF16) {
        mh = pkmax_abs(mh, v[u].x);
        mh = pkmax_abs(mh, v[u].y);
        mh = pkmax_abs(mh, v[u].z);
        mh = pkmax_abs(mh, v[u].w);
      } else {
        mf = umax(mf, umax(umax(v[u].x & 0x7fffffffu, v[u].y & 0x7fffffffu),
                           umax(v[u].z & 0x7fffffffu, v[u].w & 0x7fffffffu)));
      }
    }
  }
  uint32_t m0 = BF16 ? (uint32_t)(mh.x > mh.y ? mh.x : mh.y) : 0u;
  // tail elements (n not a multiple of the vector)
  if (blockIdx.x == 0) {
    for (int64_t t = nvec * kPer + threadIdx.x; t < n; t += kAmaxThreads) {
      if (BF16)
        m0 = umax(m0, (uint32_t)(reinterpret_cast<const uint16_t*>(x)[t] & 0x7fffu));
      else
        mf = umax(mf, reinterpret_cast<const uint32_t*>(x)[t] & 0x7fffffffu);
    }
  }
  uint32_t m = BF16 ? (m0 << 16) : mf;
  m = block_max_u32<kAmaxThreads>(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Scalar amax for unaligned inputs.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_amax_scalar(const void* __restrict__ x, int64_t n,
                                                          uint32_t* __restrict__ partials) {
  uint32_t m = 0;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * kThreads) {
    if (BF16)
      m = umax(m, (uint32_t)(reinterpret_cast<const uint16_t*>(x)[t] & 0x7fffu) << 16);
    else
      m = umax(m, reinterpret_cast<const uint32_t*>(x)[t] & 0x7fffffffu);
  }
  m = block_max_u32<>(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// ------------------------------------------------------------ NV quantize --
// Float32 squared error of encoding block v with scale s_b (multiplier r =
// 1/s_b, or 0 when s_b is 0): E = sum_i fl(fl(v_i - fl(s_b * E2M1(v_i * r)))^2),
// added in index order.  The scale search compares candidates by it.
template <int N>
__device__ __forceinline__ float block_sq_error(const float (&v)[N], float s_b, float r) {
  float E = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const uint32_t c = e2m1_pack2<0>(0u, v[i] * r, v[i + 1] * r);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);   // exact E2M1 values
    const float e0 = v[i] - s_b * d.x, e1 = v[i + 1] - s_b * d.y;
    E = E + e0 * e0;
    E = E + e1 * e1;
  }
  return E;
}

// E4M3 scale search ([NV] "高精度缩放": the block scale can be the one that
// makes the block's summed error smallest).  On entry code / r hold the amax
// rule's choice code0; the candidates code0 + d, d = -1, +1, ..., -W, +W, inside
// 0..126, replace the current choice only when their error is strictly smaller.
template <int N>
__device__ __forceinline__ void nv_search_scale(const float (&v)[N], float s_global, int window,
                                                uint32_t& code, float& r) {
  const int c0 = (int)code;
  float best = block_sq_error(v, s_global * e4m3_value(code), r);
  for (int d = 1; d <= window; ++d) {
#pragma unroll
    for (int sgn = -1; sgn <= 1; sgn += 2) {
      const int c = c0 + sgn * d;
      if (c < 0 || c > 126) continue;
      const float sb = s_global * e4m3_value((uint32_t)c);
      const float rc = sb != 0.0f ? 1.0f / sb : 0.0f;
      const float E = block_sq_error(v, sb, rc);
      if (E < best) {
        best = E;
        code = (uint32_t)c;
        r = rc;
      }
    }
  }
}

// max|x| of a block held as VPB raw 16-byte vectors (bf16 or float32).
template <bool BF16, int VPB>
__device__ __forceinline__ float raw_amax(const u32x4 (&w)[VPB]) {
  if (BF16) {
    u16x2 m = {0, 0};
#pragma unroll
    for (int k = 0; k < VPB; ++k) {
      m = pkmax_abs(m, w[k].x);
      m = pkmax_abs(m, w[k].y);
      m = pkmax_abs(m, w[k].z);
      m = pkmax_abs(m, w[k].w);
    }
    return __uint_as_float((uint32_t)(m.x > m.y ? m.x : m.y) << 16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < VPB; ++k) {
    m = umax(m, w[k].x & 0x7fffffffu);
    m = umax(m, w[k].y & 0x7fffffffu);
    m = umax(m, w[k].z & 0x7fffffffu);
    m = umax(m, w[k].w & 0x7fffffffu);
  }
  return __uint_as_float(m);
}

// Packed codes of one block of BS values (value 2j in the low nibble of byte j).
template <int BS>
struct CodeVec;
template <> struct CodeVec<8> { typedef uint32_t T; };
template <> struct CodeVec<16> { typedef u32x2 T; };
template <> struct CodeVec<32> { typedef u32x4 T; };

template <int BS>
__device__ __forceinline__ typename CodeVec<BS>::T pack_block(const float (&v)[BS]) {
  if constexpr (BS == 8) {
    return e2m1_pack8(v);
  } else if constexpr (BS == 16) {
    return u32x2{e2m1_pack8(v), e2m1_pack8(v + 8)};
  } else {
    return u32x4{e2m1_pack8(v), e2m1_pack8(v + 8), e2m1_pack8(v + 16), e2m1_pack8(v + 24)};
  }
}

// One lane per block of BS values (8, 16 or 32) of a flat run of blocks.
// SEARCH: the block scale comes from nv_search_scale over +-window codes.
template <bool BF16, int BS, bool SEARCH>
__global__ void __launch_bounds__(kThreads)
    k_nv_quant_fast(const void* __restrict__ x, int64_t nblk, uint8_t* __restrict__ q,
                    uint8_t* __restrict__ scales, const float* __restrict__ amax_in,
                    const uint32_t* __restrict__ partials, int npart, float* __restrict__ amax_out,
                    float* __restrict__ scale_out, bool reverse, int window) {
  constexpr int VPB = BS * (BF16 ? 2 : 4) / 16;   // 16-byte vectors per block
  __shared__ u32x4 lds[VPB * (kThreads + 1)];
  const float G = resolve_amax(amax_in, partials, npart);
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) *amax_out = G;
    *scale_out = s_global;
  }
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int64_t nchunk = (nblk + kThreads - 1) / kThreads;
  for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
    const int64_t base = (reverse ? nchunk - 1 - c : c) * kThreads;
    const int nb = (int)(nblk - base < kThreads ? nblk - base : kThreads);
    u32x4 w[VPB];
    stage_blocks<VPB, kThreads>(xv, base, nb, lds, w);
    if ((int)threadIdx.x >= nb) continue;
    uint32_t sc;
    float r;
    typename CodeVec<BS>::T codes;
    if (SEARCH) {
      float v[BS];
      if (BF16) unpack_bf16<BS>(w, v); else unpack_f32<BS>(w, v);
      nv_block_scale(amax_of(v), s_global, sc, r);
      nv_search_scale(v, s_global, window, sc, r);
#pragma unroll
      for (int j = 0; j < BS; ++j) v[j] = v[j] * r;
      codes = pack_block<BS>(v);
    } else {
      // block amax from the raw words (bf16: packed 16-bit max of the
      // magnitudes, same order as the values), then 8 values at a time, so
      // the block is never held in registers as float32 all at once
      nv_block_scale(raw_amax<BF16, VPB>(w), s_global, sc, r);
      uint32_t d[BS / 8];
#pragma unroll
      for (int k = 0; k < BS / 8; ++k) {
        float v[8];
        if (BF16) unpack_bf16<8>(w + k, v); else unpack_f32<8>(w + 2 * k, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * r;
        d[k] = e2m1_pack8(v);
      }
      if constexpr (BS == 8) codes = d[0];
      else if constexpr (BS == 16) codes = u32x2{d[0], d[1]};
      else codes = u32x4{d[0], d[1], d[2], d[3]};
    }
    const int64_t b = base + threadIdx.x;
    // (non-temporal: written once, read by another kernel; ~6% faster than
    // stores that allocate in L2)
    __builtin_nontemporal_store(codes, reinterpret_cast<typename CodeVec<BS>::T*>(q) + b);
    __builtin_nontemporal_store((uint8_t)sc, scales + b);
  }
}

// Any shape / alignment: one thread per (row, block).
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* x, int64_t idx) {
  if (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[idx] << 16);
  return reinterpret_cast<const float*>(x)[idx];
}

template <bool BF16, int BS, bool SEARCH>
__global__ void __launch_bounds__(kThreads)
    k_nv_quant_generic(const void* __restrict__ x, int64_t rows, int64_t cols,
                       uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                       const float* __restrict__ amax_in, const uint32_t* __restrict__ partials,
                       int npart, float* __restrict__ amax_out, float* __restrict__ scale_out,
                       int window) {
  const float G = resolve_amax(amax_in, partials, npart);
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) *amax_out = G;
    *scale_out = s_global;
  }
  const int64_t bpr = (cols + BS - 1) / BS, qstride = (cols + 1) / 2;
  const int64_t total = rows * bpr;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t r = t / bpr, j = t - r * bpr;
    const int64_t c0 = j * BS;
    const int len = (int)((cols - c0) < BS ? (cols - c0) : BS);
    float v[BS];
#pragma unroll
    for (int i = 0; i < BS; ++i) v[i] = i < len ? load_elem<BF16>(x, r * cols + c0 + i) : 0.0f;
    uint32_t sc;
    float rr;
    nv_block_scale(amax_of(v), s_global, sc, rr);
    if (SEARCH) nv_search_scale(v, s_global, window, sc, rr);
    uint8_t* qrow = q + r * qstride + c0 / 2;
    for (int i = 0; i < len; i += 2) {
      const uint32_t lo = e2m1_code(v[i] * rr);
      const uint32_t hi = (i + 1 < len) ? e2m1_code(v[i + 1] * rr) : 0u;
      qrow[i / 2] = (uint8_t)(lo | (hi << 4));
    }
    scales[r * bpr + j] = (uint8_t)sc;
  }
}

// ------------------------------------------------------------ MX quantize --
// bf16 input: v_cvt_scalef32_pk_fp4_bf16 divides a bf16 pair by the power of
// two 2^(byte-127) and encodes it with the E2M1 rounding (identical to
// E2M1(x * 2^-e) for every finite bf16 and every exponent), so the encode is
// one instruction per two values.
template <int SEL>
__device__ __forceinline__ uint32_t mx_pack2_bf16(uint32_t old, uint32_t w, float scale) {
  bf16x2 v;
  __builtin_memcpy(&v, &w, 4);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, v, scale, SEL);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_mx_quant_fast(const void* __restrict__ x, int64_t nblk, uint8_t* __restrict__ q,
                    uint8_t* __restrict__ scales) {
  constexpr int VPB = BF16 ? 4 : 8;
  __shared__ u32x4 lds[VPB * (kThreads + 1)];
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  for (int64_t base = (int64_t)blockIdx.x * kThreads; base < nblk;
       base += (int64_t)gridDim.x * kThreads) {
    const int nb = (int)(nblk - base < kThreads ? nblk - base : kThreads);
    u32x4 w[VPB];
    stage_blocks<VPB, kThreads>(xv, base, nb, lds, w);
    if ((int)threadIdx.x >= nb) continue;
    uint32_t w4[4];
    uint32_t sc;
    if (BF16) {
      u16x2 m = {0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = pkmax_abs(m, w[k].x);
        m = pkmax_abs(m, w[k].y);
        m = pkmax_abs(m, w[k].z);
        m = pkmax_abs(m, w[k].w);
      }
      sc = e8m0_code((uint32_t)(m.x > m.y ? m.x : m.y) << 16);
      const float scale = e8m0_value(sc);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t d = 0;
        d = mx_pack2_bf16<0>(d, w[k].x, scale);
        d = mx_pack2_bf16<1>(d, w[k].y, scale);
        d = mx_pack2_bf16<2>(d, w[k].z, scale);
        d = mx_pack2_bf16<3>(d, w[k].w, scale);
        w4[k] = d;
      }
    } else {
      float v[32];
      unpack_f32<32>(w, v);
      sc = e8m0_code(__float_as_uint(amax_of(v)));
      const float inv = e8m0_inv(sc);
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = v[j] * inv;     // exact power-of-two multiply
#pragma unroll
      for (int k = 0; k < 4; ++k) w4[k] = e2m1_pack8(v + 8 * k);
    }
    const int64_t b = base + threadIdx.x;
    __builtin_nontemporal_store(u32x4{w4[0], w4[1], w4[2], w4[3]}, reinterpret_cast<u32x4*>(q) + b);
    __builtin_nontemporal_store((uint8_t)sc, scales + b);
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_mx_quant_generic(const void* __restrict__ x, int64_t rows, int64_t cols,
                       uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  const int64_t bpr = (cols + 31) / 32, qstride = (cols + 1) / 2;
  const int64_t total = rows * bpr;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t r = t / bpr, j = t - r * bpr;
    const int64_t c0 = j * 32;
    const int len = (int)((cols - c0) < 32 ? (cols - c0) : 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = i < len ? load_elem<BF16>(x, r * cols + c0 + i) : 0.0f;
    const uint32_t sc = e8m0_code(__float_as_uint(amax_of(v)));
    const float inv = e8m0_inv(sc);
    uint8_t* qrow = q + r * qstride + c0 / 2;
    for (int i = 0; i < len; i += 2) {
      const uint32_t lo = e2m1_code(v[i] * inv);
      const uint32_t hi = (i + 1 < len) ? e2m1_code(v[i + 1] * inv) : 0u;
      qrow[i / 2] = (uint8_t)(lo | (hi << 4));
    }
    scales[r * bpr + j] = (uint8_t)sc;
  }
}

// ------------------------------------------------------------- dequantize --
// Codes -> float32 values v * scale for a power-of-two scale (the gfx950
// conversion applies only the exponent of its scale operand; with a power of
// two the products are exact).  Byte SEL of d holds two codes.
template <int SEL>
__device__ __forceinline__ f32x2 decode2(uint32_t d, float pow2) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, pow2, SEL);
}

template <int SEL>
__device__ __forceinline__ uint32_t decode2_bf16(uint32_t d, float pow2) {
  const bf16x2 h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, pow2, SEL);
  uint32_t r;
  __builtin_memcpy(&r, &h, 4);
  return r;
}

// float32 pair -> packed bf16, nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  uint32_t r;
  __builtin_memcpy(&r, &h, 4);
  return r;
}

// One lane per 8 values (bf16 out, 16-byte store) or 4 values (float32 out,
// 16-byte store).  `unit` indexes those groups over the flat tensor.
template <bool MX, bool BF16OUT, int BS>
__global__ void __launch_bounds__(kThreads)
    k_dequant_fast(const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
                   const float* __restrict__ global_scale, int64_t nunits, void* __restrict__ y) {
  constexpr int kVals = BF16OUT ? 8 : 4;
  constexpr int kBlock = BS;
  const float s_global = MX ? 1.0f : *global_scale;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kThreads) {
    const uint32_t d =
        BF16OUT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q) + u)
                : (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(q) + u);
    const uint32_t sb = scales[u * kVals / kBlock];
    u32x4 out;
    if (MX) {
      const float s = e8m0_value(sb);
      if (BF16OUT) {
        // v * 2^e is exact in bf16 (2 significant bits)
        out = u32x4{decode2_bf16<0>(d, s), decode2_bf16<1>(d, s), decode2_bf16<2>(d, s),
                    decode2_bf16<3>(d, s)};
      } else {
        const f32x2 a = decode2<0>(d, s), b = decode2<1>(d, s);
        out = u32x4{__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(b.x),
                    __float_as_uint(b.y)};
      }
    } else {
      const float s = s_global * e4m3_value(sb);        // s_b, as the quantizer computes it
      const f32x2 a = decode2<0>(d, 1.0f), b = decode2<1>(d, 1.0f);
      if (BF16OUT) {
        const f32x2 c = decode2<2>(d, 1.0f), e = decode2<3>(d, 1.0f);
        out = u32x4{pack_bf16(s * a.x, s * a.y), pack_bf16(s * b.x, s * b.y),
                    pack_bf16(s * c.x, s * c.y), pack_bf16(s * e.x, s * e.y)};
      } else {
        out = u32x4{__float_as_uint(s * a.x), __float_as_uint(s * a.y), __float_as_uint(s * b.x),
                    __float_as_uint(s * b.y)};
      }
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(y) + u);
  }
}

template <bool BF16OUT>
__global__ void __launch_bounds__(kThreads)
    k_dequant_generic(bool mx, int bs, const uint8_t* __restrict__ q,
                      const uint8_t* __restrict__ scales, const float* __restrict__ global_scale,
                      int64_t rows, int64_t cols, void* __restrict__ y) {
  const float s_global = mx ? 1.0f : *global_scale;
  const int64_t bpr = (cols + bs - 1) / bs, qstride = (cols + 1) / 2;
  const int64_t total = rows * cols;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t r = t / cols, c = t - r * cols;
    const uint32_t byte = q[r * qstride + c / 2];
    const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
    const uint32_t sb = scales[r * bpr + c / bs];
    const float v = mx ? e2m1_value(code) * e8m0_value(sb)
                       : (s_global * e4m3_value(sb)) * e2m1_value(code);
    if (BF16OUT)
      reinterpret_cast<uint16_t*>(y)[t] = (uint16_t)f32_to_bf16(v);
    else
      reinterpret_cast<float*>(y)[t] = v;
  }
}

__global__ void k_empty_scales(float* amax_out, float* scale_out) {
  if (threadIdx.x == 0) {
    if (amax_out) *amax_out = 0.0f;
    *scale_out = 1.0f;
  }
}

// After an amax pass the encode pass walks the tensor backwards, starting on the data
// the amax pass read last (the likeliest to still be cached).
constexpr bool kReverseAfterAmax = true;

inline int grid_for(int64_t work_items) {
  int64_t g = (work_items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (int)(g < kMaxGrid ? g : kMaxGrid);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool BF16, int BS, bool SEARCH>
void nv_quant_launch(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scales,
                     const float* amax_in, const uint32_t* partials, int npart, float* amax_out,
                     float* scale_out, int window, hipStream_t stream) {
  const bool fast = (cols % BS == 0) && aligned16(x) && aligned16(q);
  if (fast) {
    const int64_t nblk = rows * (cols / BS);
    const bool reverse = kReverseAfterAmax && amax_in == nullptr;
    hipLaunchKernelGGL((k_nv_quant_fast<BF16, BS, SEARCH>), dim3(grid_for(nblk)), dim3(kThreads), 0,
                       stream, x, nblk, q, scales, amax_in, partials, npart, amax_out, scale_out,
                       reverse, window);
  } else {
    hipLaunchKernelGGL((k_nv_quant_generic<BF16, BS, SEARCH>),
                       dim3(grid_for(rows * ((cols + BS - 1) / BS))), dim3(kThreads), 0, stream, x,
                       rows, cols, q, scales, amax_in, partials, npart, amax_out, scale_out, window);
  }
}

template <bool BF16>
hipError_t nv_quant_dispatch(const void* x, int64_t rows, int64_t cols, int block, int window,
                             uint8_t* q, uint8_t* scales, const float* amax_in,
                             const uint32_t* partials, int npart, float* amax_out,
                             float* scale_out, hipStream_t stream) {
#define FP4_NVQ(BS, S)                                                                       \
  nv_quant_launch<BF16, BS, S>(x, rows, cols, q, scales, amax_in, partials, npart, amax_out, \
                               scale_out, window, stream)
  const bool search = window > 0;
  switch (block) {
    case 8: if (search) FP4_NVQ(8, true); else FP4_NVQ(8, false); break;
    case 16: if (search) FP4_NVQ(16, true); else FP4_NVQ(16, false); break;
    case 32: if (search) FP4_NVQ(32, true); else FP4_NVQ(32, false); break;
    default: return hipErrorInvalidValue;
  }
#undef FP4_NVQ
  return hipGetLastError();
}

// Partial maxima of the amax pass for nvfp4_quantize_no_workspace: one copy per
// device, kept until the process ends.  Host code never names it directly (on
// the host the name is only a stand-in); it uses the device address from
// hipGetSymbolAddress, kept per device below.
static __device__ __align__(256) uint32_t scratch[fp4impl::kAmaxPartials];

constexpr int kScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kScratchDevices];

}  // namespace

namespace fp4impl {

hipError_t amax_scratch(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    // once per device, with that device current (two racing first calls both
    // look the address up; they get the same one)
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    p = reinterpret_cast<uintptr_t>(a);
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = reinterpret_cast<uint32_t*>(p);
  return hipSuccess;
}

hipError_t launch_amax(const void* x, bool bf16, int64_t n, uint32_t* partials, int* npart,
                       hipStream_t stream) {
  const int per = bf16 ? 8 : 4;
  const int64_t nvec = n / per;
  if (aligned16(x)) {
    // 4 vectors in flight per thread
    const int64_t g64 = (nvec + 4 * kAmaxThreads - 1) / (4 * kAmaxThreads);
    const int g = (int)(g64 < 1 ? 1 : (g64 > kAmaxPartials ? kAmaxPartials : g64));
    *npart = g;
    if (bf16)
      hipLaunchKernelGGL(k_amax<true>, dim3(g), dim3(kAmaxThreads), 0, stream, x, n, partials);
    else
      hipLaunchKernelGGL(k_amax<false>, dim3(g), dim3(kAmaxThreads), 0, stream, x, n, partials);
  } else {
    int g = grid_for((n + 3) / 4);
    if (g > kAmaxPartials) g = kAmaxPartials;
    *npart = g;
    if (bf16)
      hipLaunchKernelGGL(k_amax_scalar<true>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
    else
      hipLaunchKernelGGL(k_amax_scalar<false>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
  }
  return hipGetLastError();
}

hipError_t launch_nv_quant(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* q,
                           uint8_t* scales, const float* amax_in, const uint32_t* partials,
                           int npart, float* amax_out, float* scale_out, hipStream_t stream,
                           int block, int window) {
  return bf16 ? nv_quant_dispatch<true>(x, rows, cols, block, window, q, scales, amax_in, partials,
                                        npart, amax_out, scale_out, stream)
              : nv_quant_dispatch<false>(x, rows, cols, block, window, q, scales, amax_in,
                                         partials, npart, amax_out, scale_out, stream);
}

hipError_t launch_mx_quant(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* q,
                           uint8_t* scales, hipStream_t stream) {
  const bool fast = (cols % 32 == 0) && aligned16(x) && aligned16(q);
  if (fast) {
    const int64_t nblk = rows * (cols / 32);
    const int g = grid_for(nblk);
    if (bf16)
      hipLaunchKernelGGL(k_mx_quant_fast<true>, dim3(g), dim3(kThreads), 0, stream, x, nblk, q,
                         scales);
    else
      hipLaunchKernelGGL(k_mx_quant_fast<false>, dim3(g), dim3(kThreads), 0, stream, x, nblk, q,
                         scales);
  } else {
    const int g = grid_for(rows * ((cols + 31) / 32));
    if (bf16)
      hipLaunchKernelGGL(k_mx_quant_generic<true>, dim3(g), dim3(kThreads), 0, stream, x, rows,
                         cols, q, scales);
    else
      hipLaunchKernelGGL(k_mx_quant_generic<false>, dim3(g), dim3(kThreads), 0, stream, x, rows,
                         cols, q, scales);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(bool mx, const uint8_t* q, const uint8_t* scales,
                          const float* global_scale, int64_t rows, int64_t cols, void* y,
                          bool bf16_out, hipStream_t stream, int block) {
  const int bs = mx ? 32 : block;
  if (bs != 8 && bs != 16 && bs != 32) return hipErrorInvalidValue;
  const bool fast = (cols % bs == 0) && aligned16(q) && aligned16(y);
  if (fast) {
    const int64_t nunits = rows * cols / (bf16_out ? 8 : 4);
    const int g = grid_for(nunits);
#define FP4_DEQ_LAUNCH(M, B, S)                                                                 \
  hipLaunchKernelGGL((k_dequant_fast<M, B, S>), dim3(g), dim3(kThreads), 0, stream, q, scales,  \
                     global_scale, nunits, y)
    if (mx) {
      if (bf16_out) FP4_DEQ_LAUNCH(true, true, 32); else FP4_DEQ_LAUNCH(true, false, 32);
    } else if (bs == 16) {
      if (bf16_out) FP4_DEQ_LAUNCH(false, true, 16); else FP4_DEQ_LAUNCH(false, false, 16);
    } else if (bs == 8) {
      if (bf16_out) FP4_DEQ_LAUNCH(false, true, 8); else FP4_DEQ_LAUNCH(false, false, 8);
    } else {
      if (bf16_out) FP4_DEQ_LAUNCH(false, true, 32); else FP4_DEQ_LAUNCH(false, false, 32);
    }
#undef FP4_DEQ_LAUNCH
  } else {
    const int g = grid_for(rows * cols);
    if (bf16_out)
      hipLaunchKernelGGL(k_dequant_generic<true>, dim3(g), dim3(kThreads), 0, stream, mx, bs, q,
                         scales, global_scale, rows, cols, y);
    else
      hipLaunchKernelGGL(k_dequant_generic<false>, dim3(g), dim3(kThreads), 0, stream, mx, bs, q,
                         scales, global_scale, rows, cols, y);
  }
  return hipGetLastError();
}

hipError_t launch_empty_scales(float* amax_out, float* scale_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_empty_scales, dim3(1), dim3(64), 0, stream, amax_out, scale_out);
  return hipGetLastError();
}

}  // namespace fp4impl
