// Decode-time batched GEMV  y = g_d * x_hat @ W_hat^T  with NVFP4 weights and
// activations quantized on the fly (one tensor scale over the whole [B, K]).
//
// Written from the scaled-GEMM equation of the "NVIDIA NVFP4 与 Micro-Scaling"
// article (section 三); the 10100.com data-type article announces an "FP4 batch
// GEMV" whose text is not on the pages.
//
// y[b, n] = g_d * s_gx * g_w * sum_k x'[b, k] * w'[n, k] with x' = E4M3(s_xb) *
// E2M1(v_x) and w' = E4M3(s_wb) * E2M1(v_w): both are exact in fp16 (at most 6
// significant bits, magnitudes in [2^-10, 2688]), so their products are exact
// and only the float32 accumulation rounds.
//
// Launch 1 (k_gemv_xprep): x -> NVFP4 exactly as nvfp4_quantize does (every
//   workgroup reduces the small x for the global amax itself), stored in the
//   workspace as x' in fp16, [B][Kp] with K padded to a multiple of 128.
// Launch 2 (k_gemv_mfma): W streaming on v_mfma_f32_16x16x32_f16.  The batch
//   rows are the MFMA's M side (rows >= B are zero), 16 W rows its N side, so
//   one MFMA applies a W fragment to every batch row at once.  A workgroup is
//   persistent over 16-row strips of W; its waves split K (a wave keeps the
//   x' fragments of its K range in registers for the whole kernel), each lane
//   loads 16 contiguous bytes (32 codes) of one W row per 128-value step and
//   dequantizes them in registers (v_cvt_scalef32_pk_f16_fp4 applies the
//   scale's power of two, v_pk_mul_f16 its 3-bit mantissa); the K order inside
//   a step is permuted identically for x' and W.  The waves' partial 16x16
//   tiles are summed through LDS in a fixed order.
#include <atomic>

#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kPrepThreads = 256;
constexpr size_t kHeader = 256;        // workspace header: [0] s_global of x
constexpr int kMaxWaves = 16;
constexpr int kMaxSteps = 3;           // 128-value steps per wave kept in registers

inline int64_t kpad(int64_t K) { return (K + 127) / 128 * 128; }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// -------------------------------------------------------------- x prologue --
template <bool BF16>
__global__ void __launch_bounds__(kPrepThreads)
    k_gemv_xprep(const void* __restrict__ x, int64_t B, int64_t K, int64_t Kp,
                 uint8_t* __restrict__ ws) {
  __shared__ uint32_t red[kPrepThreads / 64];
  const int64_t n = B * K;
  // global amax of x (small: every workgroup reduces all of it)
  uint32_t m = 0;
  if (BF16) {
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t i = threadIdx.x; i < n / 8; i += kPrepThreads) {
      const u32x4 v = xv[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = w[j] & 0x7fff7fffu;
        m = umax(m, umax(a << 16, a & 0xffff0000u));
      }
    }
  } else {
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t i = threadIdx.x; i < n / 4; i += kPrepThreads) {
      const u32x4 v = xv[i];
      m = umax(umax(m, v.x & 0x7fffffffu), umax(v.y & 0x7fffffffu, umax(v.z & 0x7fffffffu, v.w & 0x7fffffffu)));
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
  const float s_global = nv_global_scale(__uint_as_float(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) reinterpret_cast<float*>(ws)[0] = s_global;

  // one thread per 16-value block of the padded [B, Kp] x'
  const int64_t bpr = Kp / 16;
  const int64_t blk = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x;
  if (blk >= B * bpr) return;
  const int64_t row = blk / bpr, c0 = (blk - row * bpr) * 16;
  _Float16* out = reinterpret_cast<_Float16*>(ws + kHeader) + row * Kp + c0;
  if (c0 >= K) {
#pragma unroll
    for (int j = 0; j < 16; ++j) out[j] = (_Float16)0.0f;
    return;
  }
  float v[16];
  const int64_t base = row * K + c0;
  if (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + base);
    const u32x4 a = p[0], c = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_lo(w[j]);
      v[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + base);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 a = p[j];
      v[4 * j] = a.x;
      v[4 * j + 1] = a.y;
      v[4 * j + 2] = a.z;
      v[4 * j + 3] = a.w;
    }
  }
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) am = umax(am, __float_as_uint(v[j]) & 0x7fffffffu);
  uint32_t sc;
  float r;
  nv_block_scale(__uint_as_float(am), s_global, sc, r);
  const float sv = e4m3_value(sc);
  _Float16 h[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) h[j] = (_Float16)(e2m1_value(e2m1_code(v[j] * r)) * sv);   // exact
  u32x4* o4 = reinterpret_cast<u32x4*>(out);
  uint32_t wd[8];
  __builtin_memcpy(wd, h, 32);
  o4[0] = u32x4{wd[0], wd[1], wd[2], wd[3]};
  o4[1] = u32x4{wd[4], wd[5], wd[6], wd[7]};
}

// --------------------------------------------------------- W streaming --
// E4M3 byte -> (power of two as the cvt scale operand, 3-bit mantissa as an
// f16 pair): normal 2^(E-7) * (1 + m/8), subnormal 2^-9 * m.
__device__ __forceinline__ void e4m3_split(uint32_t b, float& pow2, v2h& mant) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  pow2 = __uint_as_float(e ? ((e + 120u) << 23) : (118u << 23));
  const _Float16 mh = (_Float16)(e ? 1.0f + (float)m * 0.125f : (float)m);
  mant = v2h{mh, mh};
}

__device__ __forceinline__ v8h dequant8(uint32_t codes, float pow2, v2h mant) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 0) * mant;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 1) * mant;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 2) * mant;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 3) * mant;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// One 128-value step of a 16-row strip: this lane's 16 code bytes (32 values)
// and 2 scale bytes; zeros past K.
__device__ __forceinline__ void load_step(const uint8_t* __restrict__ wr,
                                          const uint8_t* __restrict__ sr, int kc, int K,
                                          u32x4& codes, uint32_t& sbytes) {
  if (kc < K) {
    codes = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + kc / 2));
    sbytes = *reinterpret_cast<const uint16_t*>(sr + kc / 16);
  } else {
    codes = u32x4{0, 0, 0, 0};
    sbytes = 0;
  }
}

__device__ __forceinline__ v4f mfma_step(v4f acc, const v8h (&xv)[4], const u32x4& codes,
                                         uint32_t sbytes) {
  float p0, p1;
  v2h m0, m1;
  e4m3_split(sbytes & 0xffu, p0, m0);
  e4m3_split(sbytes >> 8, p1, m1);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[0], dequant8(codes.x, p0, m0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[1], dequant8(codes.y, p0, m0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[2], dequant8(codes.z, p1, m1), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[3], dequant8(codes.w, p1, m1), acc, 0, 0, 0);
  return acc;
}

// Sums the waves' partial 16x16 tiles (fixed order) and writes y for strip n0.
template <bool YBF16>
__device__ __forceinline__ void reduce_store(v4f* red, v4f acc, int nwaves, int n0, int N, int B,
                                             float gscale, float g_d, void* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  red[wave * 64 + lane] = acc;
  __syncthreads();
  // output (b, n0 + c) sits in lane (b/4)*16 + c, element b%4, of every wave
  for (int o = threadIdx.x; o < 256; o += blockDim.x) {
    const int ob = o >> 4, oc = o & 15;
    const int src = (ob >> 2) * 16 + oc, el = ob & 3;
    float sum = red[src][el];
    for (int w = 1; w < nwaves; ++w) sum = sum + red[w * 64 + src][el];
    if (ob < B && n0 + oc < N) {
      const float v = (sum * gscale) * g_d;
      if (YBF16)
        reinterpret_cast<uint16_t*>(y)[(int64_t)ob * N + n0 + oc] = (uint16_t)f32_to_bf16(v);
      else
        reinterpret_cast<float*>(y)[(int64_t)ob * N + n0 + oc] = v;
    }
  }
  __syncthreads();
}

// RESIDENT: the wave's x' fragments (spw <= kMaxSteps steps) stay in registers
// and the next strip's W bytes are loaded while the current strip computes.
// Otherwise x' is re-read from the workspace (L2) for every step.
template <bool YBF16, bool RESIDENT>
__global__ void __launch_bounds__(kMaxWaves * 64)
    k_gemv_mfma(const uint8_t* __restrict__ W, const uint8_t* __restrict__ w_scales,
                const float* __restrict__ g_w, int N, int K, float g_d,
                const uint8_t* __restrict__ ws, int B, int Kp, int spw, void* __restrict__ y) {
  __shared__ v4f red[kMaxWaves * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int b = lane & 15, g = lane >> 4;
  const int T = Kp / 128;
  const int t0 = wave * spw;
  const _Float16* xp = reinterpret_cast<const _Float16*>(ws + kHeader);
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 16;
  const float gscale = reinterpret_cast<const float*>(ws)[0] * (*g_w);
  const int nstrips = (N + 15) / 16;
  const v8h zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  if (RESIDENT) {
    // x' fragments of this wave's K range: step i, MFMA sub-step s -> 8 fp16
    v8h xf[kMaxSteps][4];
#pragma unroll
    for (int i = 0; i < kMaxSteps; ++i) {
      const int t = t0 + i;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xf[i][s] = (i < spw && t < T && b < B)
                       ? *reinterpret_cast<const v8h*>(xp + (int64_t)b * Kp + 128 * t + 32 * g + 8 * s)
                       : zero8;
    }
    u32x4 nc[kMaxSteps];
    uint32_t ns[kMaxSteps];
    auto load_strip = [&](int strip) {
      const int row = min(strip * 16 + b, N - 1);
      const uint8_t* wr = W + (int64_t)row * wrow_bytes;
      const uint8_t* sr = w_scales + (int64_t)row * srow_bytes;
#pragma unroll
      for (int i = 0; i < kMaxSteps; ++i) {
        const int t = t0 + i;
        if (i < spw && t < T) {
          load_step(wr, sr, 128 * t + 32 * g, K, nc[i], ns[i]);
        } else {
          nc[i] = u32x4{0, 0, 0, 0};
          ns[i] = 0;
        }
      }
    };
    int strip = blockIdx.x;
    if (strip < nstrips) load_strip(strip);
    for (; strip < nstrips; strip += gridDim.x) {
      u32x4 cc[kMaxSteps];
      uint32_t cs[kMaxSteps];
#pragma unroll
      for (int i = 0; i < kMaxSteps; ++i) {
        cc[i] = nc[i];
        cs[i] = ns[i];
      }
      if (strip + (int)gridDim.x < nstrips) load_strip(strip + gridDim.x);
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < kMaxSteps; ++i)
        if (i < spw) acc = mfma_step(acc, xf[i], cc[i], cs[i]);
      reduce_store<YBF16>(red, acc, nwaves, strip * 16, N, B, gscale, g_d, y);
    }
  } else {
    for (int strip = blockIdx.x; strip < nstrips; strip += gridDim.x) {
      const int row = min(strip * 16 + b, N - 1);
      const uint8_t* wr = W + (int64_t)row * wrow_bytes;
      const uint8_t* sr = w_scales + (int64_t)row * srow_bytes;
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int i = 0; i < spw; ++i) {
        const int t = t0 + i;
        if (t >= T) break;
        u32x4 codes;
        uint32_t sbytes;
        load_step(wr, sr, 128 * t + 32 * g, K, codes, sbytes);
        v8h xv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv[s] = b < B ? *reinterpret_cast<const v8h*>(xp + (int64_t)b * Kp + 128 * t + 32 * g + 8 * s)
                        : zero8;
        acc = mfma_step(acc, xv, codes, sbytes);
      }
      reduce_store<YBF16>(red, acc, nwaves, strip * 16, N, B, gscale, g_d, y);
    }
  }
}

// ------------------------------------------------------ fused streaming GEMV --
// One workgroup of 16 waves per CU, persistent over rounds of strips.
// Prologue: every workgroup quantizes all of x itself (global amax, then
// per-block NVFP4 exactly as nvfp4_quantize) into LDS -- as exact fp16 x' when
// it fits (XF16), else as codes + scale bytes dequantized per use.  Its first x
// loads are issued before the first W loads so they do not queue behind them.
// Streaming: a round gives each of the kSlots wave pairs one 16-row strip; the
// two waves of a pair stream the two halves of K, kPairs pairs of 128-value
// steps in flight per wave.  At the round's end the upper half's partial tile
// goes through LDS (double-buffered by round parity, one barrier per round) to
// the lower half's wave, which adds it (fixed order) and writes y.
constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / 64;
constexpr int kSplit = 2;                       // waves per strip (K parts)
constexpr int kSlots = kStreamWaves / kSplit;   // strips per workgroup and round
constexpr int kPairs = 4;                       // pairs of steps in flight per wave
constexpr int kXRegVecs = 4;                    // 16-byte x vectors per thread held in registers
constexpr int kRedBytes = 2 * kSlots * 64 * 16; // double-buffered partial tiles

__host__ __device__ inline int xf16_row_bytes(int Kq) {
  const int base = Kq * 2 + Kq / 4;
  return base + ((64 - base % 256) & 255);
}

__device__ __forceinline__ uint32_t block_max_1024(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < kStreamWaves; ++i) r = umax(r, red[i]);
  __syncthreads();
  return r;
}

// f16 pair (h, h) for one E4M3 byte, h = E4M3 value * 2^-8 exactly: the byte's
// exponent and mantissa fields drop into the f16 fields (bias 7 against 15
// gives the 2^-8, E4M3 subnormals land on f16 subnormals) and its sign bit on
// the sign.  Bytes 0x7f / 0xff (NaN) read as +-480; quantizers never emit them.
__device__ __forceinline__ v2h e4m3_h2(uint32_t byte) {
  const uint32_t h = ((byte & 0x80u) << 8) | ((byte & 0x7fu) << 7);
  return __builtin_bit_cast(v2h, h | (h << 16));
}

// f16 pair (h(b0), h(b1)) of the two E4M3 bytes of 16-bit word SEL of w, the
// same h as e4m3_h2 for every finite byte (v_cvt_scalef32_pk_f16_fp8 with the
// scale 2^-8, one instruction for two bytes; a NaN byte gives NaN).
template <bool SEL>
__device__ __forceinline__ v2h e4m3_pair_h(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 0x1p-8f, SEL);
}

// The 8 values E2M1(code) * E4M3 of one dword of codes: the conversion scales
// by 2^8 (exact), and the f16 product with E4M3 * 2^-8 is exact (at most 6
// significant bits, magnitude in [2^-10, 2688]).
__device__ __forceinline__ v8h dq8(uint32_t codes, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// K order inside a pair (256 values of a 16-row strip): lane (b = l % 16,
// g = l / 16) feeds W row b and batch row b with values [64g + 32st, +32) in
// step st, 8 per MFMA; x' and W use the same order, so each MFMA sums the same
// products.  A lane's W scales for a pair are then 4 contiguous bytes.
//
// W scale bytes (SCM):
//   kScaleGroup  K % 256 == 0 and 16-aligned scales: the group's scales, 16 rows x
//                kPairs * 16 bytes, arrive with one 16-byte load per lane issued
//                with the group before (ring slot 0), pass through a 1 KB LDS
//                area per wave, and each pair reads its dword there.
//   kScaleDword  K % 64 == 0, 4-aligned: one dword load per pair.
//   kScaleHalf   otherwise: two 16-bit loads per pair.
constexpr int kScaleHalf = 0, kScaleDword = 1, kScaleGroup = 2;
constexpr int kBufferWord3 = 0x00020000;         // raw buffer descriptor word 3 (gfx9 family)
constexpr int kLoadNT = 2;                      // buffer load cache policy: nontemporal

template <bool XBF16, bool XF16, int SCM>
__global__ void __launch_bounds__(kStreamThreads, 1)
    k_gemv_stream(const void* __restrict__ x, int B, const uint8_t* __restrict__ W,
                  const uint8_t* __restrict__ w_scales, const float* __restrict__ g_w, int N,
                  int K, int Kq, int lds_x_bytes, float g_d, void* __restrict__ y, bool YBF16) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ uint32_t red_max[kStreamWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = lane & 15, g = lane >> 4;
  const int r8 = lane >> 3, c8 = lane & 7;
  const int nstrips = (N + 15) / 16;
  const int wrow = K / 2, srow = K / 16;
  // LDS: x' (zero past K up to Kq, a multiple of 256) | transpose tiles | partial tiles
  // XF16 x' row: value v at byte 2v + 16 (v / 64), rows 64 bytes apart modulo
  // 256, so the four lane groups' 32-value reads (and up to 4 batch rows) fall
  // on distinct LDS banks
  const int xf_row = xf16_row_bytes(Kq);
  const int xc_row = Kq / 2 + 16;                // codes row stride
  const int bpr = Kq / 16;                       // x blocks per padded row
  uint8_t* xs_base = lds + B * xc_row;           // scale bytes [B][bpr]
  uint8_t* tb = lds + lds_x_bytes + wave * 2048;
  v4f* red = reinterpret_cast<v4f*>(lds + lds_x_bytes + kStreamWaves * 2048);

  // ---- x: first blocks into registers (thread t owns blocks t + i * 1024)
  constexpr int VPB = XBF16 ? 2 : 4;             // 16-byte vectors per 16-value block
  constexpr int kXB = kXRegVecs / VPB;
  const int nblk = B * bpr;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  auto block_src = [&](int blk, bool& ok) {
    const int row = blk / bpr, c0 = (blk - row * bpr) * 16;
    ok = blk < nblk && c0 < K;
    return xv + (ok ? ((int64_t)row * K + c0) / (16 / VPB) : 0);
  };
  u32x4 xr[kXB][VPB];
#pragma unroll
  for (int i = 0; i < kXB; ++i) {
    bool ok;
    const u32x4* src = block_src(threadIdx.x + i * kStreamThreads, ok);
#pragma unroll
    for (int v = 0; v < VPB; ++v) xr[i][v] = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- W ring: a wave's elements are (round r, pair pbeg + e), e < Ep
  const int part = wave / kSlots, slot = wave - part * kSlots;
  const int Pq = Kq / 256;
  const int Ph = (Pq + kSplit - 1) / kSplit;
  const int pbeg = min(part * Ph, Pq), pend = min(pbeg + Ph, Pq);
  const int E = pend - pbeg;
  // a round is padded to whole groups of kPairs elements, so every loop
  // iteration below runs all kPairs ring slots; padding elements read nothing
  // (empty range) and are not computed
  const int Ep = (E + kPairs - 1) / kPairs * kPairs;
  const int G = gridDim.x * kSlots;              // strips per round
  const int s_first = slot * gridDim.x + blockIdx.x;
  const int R = (nstrips + G - 1) / G;
  const int nmine = s_first < nstrips ? (nstrips - s_first + G - 1) / G : 0;
  const int J = nmine * Ep;
  // All W and W-scale reads are buffer loads through a per-strip descriptor
  // whose range is the strip's rows that exist (N may end inside a strip).  A
  // read outside the range returns zeros without touching memory, so every
  // loop iteration issues the same loads with no branch around them (which
  // keeps kPairs elements in flight): look-ahead past the wave's last element
  // and padding elements get an empty range, and reads past K run into the
  // next row's codes (finite, against x' = 0) or off the range.  The lane's
  // offset inside the strip is fixed; the pair's offset is a scalar.
  u32x4 ra[kPairs], rb[kPairs];
  uint32_t rs[kPairs];
  u32x4 sg;                                      // scale group in flight
  const int w_lane = r8 * wrow + 16 * c8;
  const int s_lane = b * srow + 4 * g;
  const int g_lane = b * srow + 16 * g;          // group load: row b, pair g of the group
  uint8_t* sa = lds + lds_x_bytes + kStreamWaves * 2048 + kRedBytes + wave * 1024;
  int lr = 0, le = 0;                            // next element to load
  auto load_elem = [&](u32x4& a, u32x4& bb, uint32_t& sc, bool group) {
    const bool live = lr < nmine && le < E;
    const int r0 = lr < nmine ? (s_first + lr * G) * 16 : 0;
    const int rows = live ? min(16, N - r0) : 0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W) + (int64_t)r0 * wrow, 0, rows * wrow, kBufferWord3);
    const int pp = pbeg + le;
    a = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane, 128 * pp, kLoadNT);
    bb = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + 8 * wrow, 128 * pp, kLoadNT);
    if (SCM == kScaleGroup) {
      if (group) {   // the group's first element (le % kPairs == 0): its kPairs pairs
        const int grows = lr < nmine ? min(16, N - r0) : 0;
        const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(w_scales) + (int64_t)r0 * srow, 0, grows * srow, kBufferWord3);
        sg = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane, 16 * pp, 0);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(w_scales) + (int64_t)r0 * srow, 0, rows * srow, kBufferWord3);
      if (SCM == kScaleDword) {
        sc = __builtin_amdgcn_raw_buffer_load_b32(rsc, s_lane, 16 * pp, 0);
      } else {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rsc, s_lane, 16 * pp, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rsc, s_lane + 2, 16 * pp, 0);
        sc = lo | (hi << 16);
      }
    }
    if (++le >= Ep) { le = 0; ++lr; }
  };
#pragma unroll
  for (int i = 0; i < kPairs; ++i) load_elem(ra[i], rb[i], rs[i], i == 0);

  // ---- x -> NVFP4 (global amax over all of [B, K], then per 16-value block)
  auto vec_absmax = [&](const u32x4& v) {
    if (XBF16) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = w4[j] & 0x7fff7fffu;
        m = umax(m, umax(t << 16, t & 0xffff0000u));
      }
      return m;
    }
    return umax(umax(v.x & 0x7fffffffu, v.y & 0x7fffffffu),
                umax(v.z & 0x7fffffffu, v.w & 0x7fffffffu));
  };
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kXB; ++i)
#pragma unroll
    for (int v = 0; v < VPB; ++v) m = umax(m, vec_absmax(xr[i][v]));
  for (int blk0 = threadIdx.x + kXB * kStreamThreads; blk0 < nblk; blk0 += 2 * kStreamThreads) {
    u32x4 t[2][VPB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bool ok;
      const u32x4* src = block_src(blk0 + h * kStreamThreads, ok);
#pragma unroll
      for (int v = 0; v < VPB; ++v) t[h][v] = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < VPB; ++v) m = umax(m, vec_absmax(t[h][v]));
  }
  const float s_gx = nv_global_scale(__uint_as_float(block_max_1024(m, red_max)));
  auto quant_block = [&](int blk, const u32x4 (&vv)[VPB]) {
    const int row = blk / bpr, c0 = (blk - row * bpr) * 16;
    float v[16];
    if (XBF16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w4[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[8 * j + 2 * q] = bf16_lo(w4[q]);
          v[8 * j + 2 * q + 1] = bf16_hi(w4[q]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[4 * j] = __uint_as_float(vv[j].x);
        v[4 * j + 1] = __uint_as_float(vv[j].y);
        v[4 * j + 2] = __uint_as_float(vv[j].z);
        v[4 * j + 3] = __uint_as_float(vv[j].w);
      }
    }
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) am = umax(am, __float_as_uint(v[j]) & 0x7fffffffu);
    uint32_t sc;
    float r;
    nv_block_scale(__uint_as_float(am), s_gx, sc, r);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] * r;
    uint32_t c[2] = {e2m1_pack8(v), e2m1_pack8(v + 8)};
    if (c0 >= K) c[0] = c[1] = sc = 0u;        // padding past K: x' = 0
    if (XF16) {
      const v2h h = e4m3_h2(sc);
      v8h* dst = reinterpret_cast<v8h*>(lds + row * xf_row + c0 * 2 + 16 * (c0 / 64));
      dst[0] = dq8(c[0], h);
      dst[1] = dq8(c[1], h);
    } else {
      *reinterpret_cast<u32x2*>(lds + row * xc_row + c0 / 2) = u32x2{c[0], c[1]};
      xs_base[row * bpr + c0 / 16] = (uint8_t)sc;
    }
  };
#pragma unroll
  for (int i = 0; i < kXB; ++i) {
    const int blk = threadIdx.x + i * kStreamThreads;
    if (blk < nblk) quant_block(blk, xr[i]);
  }
  for (int blk = threadIdx.x + kXB * kStreamThreads; blk < nblk; blk += kStreamThreads) {
    bool ok;
    const u32x4* src = block_src(blk, ok);
    u32x4 t[VPB];
#pragma unroll
    for (int v = 0; v < VPB; ++v) t[v] = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
    quant_block(blk, t);
  }
  __syncthreads();
  const float gscale = s_gx * (*g_w);

  // ---- stream W
  // Transpose tile (wave-private, 16 rows x 128 bytes): 16-byte chunk c of row
  // r sits at chunk position c ^ (r & 7) ^ 4 (r >> 3), so the row-wise writes
  // and the MFMA-layout reads (rows b and b + 8 apart by 4 chunks) spread over
  // the banks.
  const int xrow = min(b, B - 1);               // batch rows >= B: any finite x, never stored
  auto finish = [&](int r, v4f a, bool valid) {
    if (kSplit > 1) {
      v4f* rp = red + ((r & 1) * kSlots + slot) * 64;
      if (part != 0) rp[lane] = a;
      __syncthreads();
      if (part != 0) return;
      a += rp[lane];
    }
    if (!valid) return;
    const int nn = (s_first + r * G) * 16 + b;   // D[4g + q][b] of this strip
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ob = 4 * g + q;
      if (ob < B && nn < N) {
        const float v = (a[q] * gscale) * g_d;
        if (YBF16)
          reinterpret_cast<uint16_t*>(y)[(int64_t)ob * N + nn] = (uint16_t)f32_to_bf16(v);
        else
          reinterpret_cast<float*>(y)[(int64_t)ob * N + nn] = v;
      }
    }
  };
  v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  int cr = 0, ce = 0;                            // element being computed
  const int wsw = (r8 ^ c8) << 4;
  // One element from ring slot i: stage its W codes (and in slot 0 the scale
  // group) in LDS, refill the slot with the element kPairs ahead, then
  // dequantize and accumulate.
  auto elem = [&](u32x4& ra_i, u32x4& rb_i, uint32_t& rs_i, int i) {
    uint32_t sw = rs_i;
    if (SCM == kScaleGroup && i == 0)
      *reinterpret_cast<u32x4*>(sa + lane * 16) = sg;   // [pair q][row b] x 16 bytes
    *reinterpret_cast<u32x4*>(tb + r8 * 128 + wsw) = ra_i;
    *reinterpret_cast<u32x4*>(tb + (8 + r8) * 128 + (wsw ^ 64)) = rb_i;
    load_elem(ra_i, rb_i, rs_i, i == 0);
    if (ce < E) {
      if (SCM == kScaleGroup)
        sw = *reinterpret_cast<const uint32_t*>(sa + (16 * i + b) * 16 + 4 * g);
      const int cpp = pbeg + ce;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int c = 2 * g + st;
        const u32x4 codes = *reinterpret_cast<const u32x4*>(
            tb + b * 128 + ((c ^ (b & 7) ^ ((b >> 3) << 2)) << 4));
        const int v0 = 256 * cpp + 64 * g + 32 * st;   // first of this lane's 32 values
        v8h xq[4];
        if (XF16) {
          const v8h* src = reinterpret_cast<const v8h*>(lds + xrow * xf_row + v0 * 2 + 16 * (v0 / 64));
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) xq[s4] = src[s4];
        } else {
          const u32x4 xc = *reinterpret_cast<const u32x4*>(lds + xrow * xc_row + v0 / 2);
          const uint32_t xsb = *reinterpret_cast<const uint16_t*>(xs_base + xrow * bpr + v0 / 16);
          const v2h hp = e4m3_pair_h<false>(xsb);
          const v2h h0 = v2h{hp.x, hp.x}, h1 = v2h{hp.y, hp.y};
          xq[0] = dq8(xc.x, h0);
          xq[1] = dq8(xc.y, h0);
          xq[2] = dq8(xc.z, h1);
          xq[3] = dq8(xc.w, h1);
        }
        const v2h wp = st ? e4m3_pair_h<true>(sw) : e4m3_pair_h<false>(sw);
        const v2h w0 = v2h{wp.x, wp.x}, w1 = v2h{wp.y, wp.y};
        v4f& acc = st ? acc1 : acc0;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xq[0], dq8(codes.x, w0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xq[1], dq8(codes.y, w0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xq[2], dq8(codes.z, w1), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xq[3], dq8(codes.w, w1), acc, 0, 0, 0);
      }
    }
    if (ce == Ep - 1) {
      finish(cr, acc0 + acc1, true);
      acc0 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      acc1 = acc0;
    }
    if (++ce == Ep) { ce = 0; ++cr; }
  };
  // element j lives in slot j % kPairs and is refilled with element j + kPairs;
  // J is a multiple of kPairs, so slot 0 always starts a group
  for (int j0 = 0; j0 < J; j0 += kPairs) {
#pragma unroll
    for (int i = 0; i < kPairs; ++i) elem(ra[i], rb[i], rs[i], i);
  }
  // Every wave takes part in all R rounds' exchanges: a wave whose part of K is
  // empty (Ep == 0) contributes zeros for its valid rounds, and rounds without
  // a strip for this slot exchange nothing that is stored.
  for (int r = Ep > 0 ? nmine : 0; r < R; ++r) finish(r, acc0, r < nmine);
}

// K = 0: every output is an empty sum.
template <typename T>
__global__ void __launch_bounds__(256) k_zero_fill(int64_t n, T* __restrict__ y) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) y[i] = 0;
}

// Compute units per device (0: not queried yet), cached per device so that
// calls from several host threads, or on devices of different sizes (compute
// partitions), each see their own device's count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_num_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    n = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0
            ? cus : 256;
    g_num_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

struct StreamArgs {
  const void* x;
  int B;
  const uint8_t* W;
  const uint8_t* w_scales;
  const float* g_w;
  int N, K, Kq, lds_x;
  float g_d;
  void* y;
  bool y_bf16;
};

template <bool XB, bool XF, int SCM>
hipError_t launch_stream(const StreamArgs& a, int grid, int lds, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&k_gemv_stream<XB, XF, SCM>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemv_stream<XB, XF, SCM>), dim3(grid), dim3(kStreamThreads), lds, stream,
                     a.x, a.B, a.W, a.w_scales, a.g_w, a.N, a.K, a.Kq, a.lds_x, a.g_d, a.y, a.y_bf16);
  return hipGetLastError();
}

}  // namespace

namespace fp4impl {

hipError_t launch_zero_fill(void* y, int64_t n, int elem_bytes, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t nb = (n + 255) / 256;
  const dim3 g0((unsigned)(nb < 4096 ? nb : 4096));
  if (elem_bytes == 4)
    hipLaunchKernelGGL(k_zero_fill<uint32_t>, g0, dim3(256), 0, stream, n, static_cast<uint32_t*>(y));
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(k_zero_fill<uint16_t>, g0, dim3(256), 0, stream, n, static_cast<uint16_t*>(y));
  else if (elem_bytes == 1)
    hipLaunchKernelGGL(k_zero_fill<uint8_t>, g0, dim3(256), 0, stream, n, static_cast<uint8_t*>(y));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

size_t gemv_workspace_bytes(int64_t B, int64_t K) {
  return kHeader + (size_t)(B * kpad(K) * 2);
}

hipError_t launch_gemv(const void* x, bool x_bf16, int64_t B, const uint8_t* W,
                       const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K, float g_d,
                       void* y, bool y_bf16, void* workspace, hipStream_t stream) {
  if (N > (1 << 30) || K > (1 << 30)) return hipErrorInvalidValue;
  const int ncu = num_cus();
  if (K == 0) return launch_zero_fill(y, B * N, y_bf16 ? 2 : 4, stream);
  const int nstrips = (int)((N + 15) / 16);
  // fused streaming kernel when the quantized x fits in LDS
  const int64_t Kq = (K + 255) / 256 * 256;
  const int64_t lds_f16 = B * xf16_row_bytes((int)Kq);
  const int64_t lds_fp4 = B * (Kq / 2 + 16) + B * (Kq / 16);
  int scm = kScaleHalf;
  if (K % 64 == 0 && reinterpret_cast<uintptr_t>(w_scales) % 4 == 0) scm = kScaleDword;
  if (K % 256 == 0 && reinterpret_cast<uintptr_t>(w_scales) % 16 == 0) scm = kScaleGroup;
  const int64_t lds_fixed = kStreamWaves * 2048 + kRedBytes + kStreamWaves * 1024;
  const int64_t lds_max = 160 * 1024 - 256;
  const bool xf16 = lds_f16 + lds_fixed <= lds_max;
  // (the strip-relative buffer offsets need 16 rows of W to span < 2^31 bytes;
  // the x' sizes above already keep K far below that)
  if ((xf16 || lds_fp4 + lds_fixed <= lds_max) && K < (1 << 27)) {
    const int lds_x = (int)(((xf16 ? lds_f16 : lds_fp4) + 15) / 16 * 16);
    const int lds = lds_x + (int)lds_fixed;
    const int grid = nstrips < ncu ? nstrips : ncu;
    const StreamArgs sa{x, (int)B, W, w_scales, g_w, (int)N, (int)K, (int)Kq, lds_x, g_d, y, y_bf16};
    const int sel = (x_bf16 ? 4 : 0) | (xf16 ? 2 : 0);
    switch (sel * 3 + scm) {
      case 0: return launch_stream<false, false, kScaleHalf>(sa, grid, lds, stream);
      case 1: return launch_stream<false, false, kScaleDword>(sa, grid, lds, stream);
      case 2: return launch_stream<false, false, kScaleGroup>(sa, grid, lds, stream);
      case 6: return launch_stream<false, true, kScaleHalf>(sa, grid, lds, stream);
      case 7: return launch_stream<false, true, kScaleDword>(sa, grid, lds, stream);
      case 8: return launch_stream<false, true, kScaleGroup>(sa, grid, lds, stream);
      case 12: return launch_stream<true, false, kScaleHalf>(sa, grid, lds, stream);
      case 13: return launch_stream<true, false, kScaleDword>(sa, grid, lds, stream);
      case 14: return launch_stream<true, false, kScaleGroup>(sa, grid, lds, stream);
      case 18: return launch_stream<true, true, kScaleHalf>(sa, grid, lds, stream);
      case 19: return launch_stream<true, true, kScaleDword>(sa, grid, lds, stream);
      default: return launch_stream<true, true, kScaleGroup>(sa, grid, lds, stream);
    }
  }

  // very long K: x' through the workspace, waves split K
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t Kp = kpad(K);
  const int64_t nblk = B * (Kp / 16);
  const dim3 g1((unsigned)((nblk + kPrepThreads - 1) / kPrepThreads));
  if (x_bf16)
    hipLaunchKernelGGL(k_gemv_xprep<true>, g1, dim3(kPrepThreads), 0, stream, x, B, K, Kp, ws);
  else
    hipLaunchKernelGGL(k_gemv_xprep<false>, g1, dim3(kPrepThreads), 0, stream, x, B, K, Kp, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int T = (int)(Kp / 128);
  int spw = (T + kMaxWaves - 1) / kMaxWaves;
  if (spw < 1) spw = 1;
  const int nwaves = (T + spw - 1) / spw;
  const bool resident = spw <= kMaxSteps;
  const int grid = nstrips < ncu ? nstrips : ncu;
  const dim3 blk(64 * nwaves);
#define FP4_GEMV_LAUNCH(YB, RES)                                                               \
  hipLaunchKernelGGL((k_gemv_mfma<YB, RES>), dim3(grid), blk, 0, stream, W, w_scales, g_w,     \
                     (int)N, (int)K, g_d, ws, (int)B, (int)Kp, spw, y)
  if (y_bf16) {
    if (resident) FP4_GEMV_LAUNCH(true, true); else FP4_GEMV_LAUNCH(true, false);
  } else {
    if (resident) FP4_GEMV_LAUNCH(false, true); else FP4_GEMV_LAUNCH(false, false);
  }
#undef FP4_GEMV_LAUNCH
  return hipGetLastError();
}

}  // namespace fp4impl
