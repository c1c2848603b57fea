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
// Kernels by shape (launch_gemv):
//   B <= 4: k_gemv_fp4, one launch (every workgroup quantizes the small x).
//   fp16 x' fits LDS: k_gemv_stream, x quantized in every workgroup.
//   else up to 16 rows with K a multiple of 256 up to 5120 (the decode shape
//     from 8 rows): k_gemv_xquant, then k_gemv_xreg (x' in registers).
//   else while x fits LDS as codes: k_gemv_xquant, then k_gemv_stream.
//   longer K: k_gemv_xquant, then k_gemv_mfma.
// k_gemv_xquant: x -> NVFP4 once, exactly as nvfp4_quantize does, into the
//   workspace: as exact fp16 x' rows (for the long-K kernel) or as codes +
//   scale bytes, zero past K.  Small x: every prep workgroup reduces all of x
//   for the global amax itself; larger x: a first launch writes per-workgroup
//   partial maxima (the quantizer's amax pass) and the prep reduces those.
// The streaming kernels (k_gemv_stream, k_gemv_fp4, k_gemv_xreg; below) run
//   one workgroup per CU, persistent over 16-row strips of W.
// Long K (x not fitting LDS): k_gemv_mfma, W streaming on
//   v_mfma_f32_16x16x32_f16.  The batch
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kPrepThreads = 512;
// Workspace: [0, 4 KiB) partial maxima of x (larger x) | [4 KiB, +256) header,
// s_global of x | from kWsData: x quantized by the prep launch.
constexpr size_t kWsPartials = 0;
constexpr size_t kWsHeader = 4096;
constexpr size_t kWsData = 4096 + 256;
// x of at most this many values: each prep workgroup reduces all of it for the
// amax (at most 16 workgroups, each reading at most 512 KB)
constexpr int64_t kSmallX = (int64_t)1 << 17;
constexpr int kMaxWaves = 16;
constexpr int kMaxSteps = 3;           // 128-value steps per wave kept in registers

inline int64_t kpad(int64_t K) { return (K + 127) / 128 * 128; }

// -------------------------------------------------------------- x prep --
// x [B, K] -> NVFP4 with one tensor scale over all of x, each step as
// nvfp4_quantize takes it: G = max|x| (from `partials` when given, else reduced
// here over all of x), s_global, then per 16-value block the E4M3 scale and
// the E2M1 codes.  F16OUT: x' = E4M3 * E2M1 (exact in fp16) as rows [B][Kpad];
// else codes [B][Kpad/2] followed by scale bytes [B][Kpad/16].  Blocks past K
// (up to Kpad) are zeros.  One thread per 16-value block of [B, Kpad].
template <bool BF16, bool F16OUT>
__global__ void __launch_bounds__(kPrepThreads)
    k_gemv_xquant(const void* __restrict__ x, int64_t B, int64_t K, int64_t Kpad,
                  const uint32_t* __restrict__ partials, int npart, uint8_t* __restrict__ ws) {
  __shared__ uint32_t red[kPrepThreads / 64];
  constexpr int kUnroll = 20;   // 16-byte vectors in flight per thread in the amax loop
  const int64_t bpr = Kpad / 16;
  const int64_t blk = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x;
  const int64_t row = blk / bpr, c0 = (blk - row * bpr) * 16;
  const bool live = blk < B * bpr && c0 < K;
  // this thread's block first, so its loads overlap the amax loads
  float v[16];
  {
    const int64_t base = live ? row * K + c0 : 0;
    if (BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + base);
      const u32x4 a = p[0], b = p[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
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
  }
  uint32_t m = 0;
  if (partials != nullptr) {
    for (int i = threadIdx.x; i < npart; i += kPrepThreads) m = umax(m, partials[i]);
  } else {
    const int64_t nvec = B * K / (BF16 ? 8 : 4);   // K % 32 == 0: whole 16-byte vectors
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t i0 = threadIdx.x; i0 < nvec; i0 += kUnroll * kPrepThreads) {
      u32x4 t[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + u * kPrepThreads;
        t[u] = i < nvec ? xv[i] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t w[4] = {t[u].x, t[u].y, t[u].z, t[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) {
            const uint32_t a = w[j] & 0x7fff7fffu;
            m = umax(m, umax(a << 16, a & 0xffff0000u));
          } else {
            m = umax(m, w[j] & 0x7fffffffu);
          }
        }
      }
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPrepThreads / 64; ++i) m = umax(m, red[i]);
  const float s_global = nv_global_scale(__uint_as_float(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<float*>(ws + kWsHeader) = s_global;

  if (blk >= B * bpr) return;
  uint8_t* data = ws + kWsData;
  uint32_t c[2] = {0u, 0u}, sc = 0u;
  if (live) {   // blocks past K (up to Kpad) stay zero
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) am = umax(am, __float_as_uint(v[j]) & 0x7fffffffu);
    float r;
    nv_block_scale(__uint_as_float(am), s_global, sc, r);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] * r;
    c[0] = e2m1_pack8(v);
    c[1] = e2m1_pack8(v + 8);
  }
  if (F16OUT) {
    const f16x2 h = e4m3_h2(sc);
    f16x8* out = reinterpret_cast<f16x8*>(data + 2 * (row * Kpad + c0));
    out[0] = dq8(c[0], h);     // exact: E2M1 * E4M3
    out[1] = dq8(c[1], h);
  } else {
    *reinterpret_cast<u32x2*>(data + row * (Kpad / 2) + c0 / 2) = u32x2{c[0], c[1]};
    data[B * (Kpad / 2) + blk] = (uint8_t)sc;
  }
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
  const _Float16* xp = reinterpret_cast<const _Float16*>(ws + kWsData);
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 16;
  const float gscale = *reinterpret_cast<const float*>(ws + kWsHeader) * (*g_w);
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

// ------------------------------------------------------ streaming GEMV --
// One workgroup of 16 waves per CU, persistent over rounds of strips.
// Prologue: narrow batches (fp16 x' fits LDS, XF16): every workgroup quantizes
// all of the small x itself (global amax, then per-block NVFP4 exactly as
// nvfp4_quantize) into LDS as exact fp16 x'.  Wider batches: x, quantized once
// by the prep launch, is copied from the workspace into LDS as codes + scale
// bytes, dequantized per use.  The first x loads are issued before the first W
// loads.
// Streaming: a round gives each of the kSlots wave pairs one 16-row strip; the
// two waves of a pair stream the two halves of K, kPairs pairs of 128-value
// steps in flight per wave.  At the round's end the upper half's partial tile
// goes through LDS (double-buffered by round parity, one barrier per round) to
// the lower half's wave, which adds it (fixed order) and writes y.
constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / 64;
constexpr int kSplit = 2;                       // waves per strip (K parts)
constexpr int kSlots = kStreamWaves / kSplit;   // strips per workgroup and round
constexpr int kPairs = 2;                       // pairs of steps in flight per wave (4: ~2 us slower at B = 16)
constexpr int kXRegVecs = 4;                    // 16-byte x vectors per thread held in registers
constexpr int kRedBytes = 2 * kSlots * 64 * 16; // double-buffered partial tiles
constexpr int kStreamLdsMax = 160 * 1024 - 256;  // dynamic LDS (the kernel has no static LDS)

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

// K order inside a pair (256 values of a 16-row strip): lane (b = l % 16,
// g = l / 16) feeds W row b and batch row b with values [64g + 32st, +32) in
// step st, 8 per MFMA; x' and W use the same order, so each MFMA sums the same
// products.  A lane's W scales for a pair are then 4 contiguous bytes.
//
// W scale bytes (SCM):
//   kScaleGroup  K % 256 == 0 and 16-aligned scales: the scales of kGroupPairs
//                pairs, 16 rows x 128 bytes, arrive with two loads of 8 rows x
//                128 bytes issued with the group's first pair, pass through a
//                2 KB LDS area per wave, and each pair reads its dword there
//                (loads of 16 rows x 64 bytes cost ~2 us more per call at the
//                decode shape).
//   kScaleDword  K % 64 == 0, 4-aligned: one dword load per pair.
//   kScaleHalf   otherwise: two 16-bit loads per pair.
constexpr int kScaleHalf = 0, kScaleDword = 1, kScaleGroup = 2;
constexpr int kGroupPairs = 8;                   // pairs per W scale group
constexpr int kGroupLds = 16 * kGroupPairs * 16; // a scale group in LDS: [pair][16 rows] x 16 bytes
constexpr int kBufferWord3 = 0x00020000;         // raw buffer descriptor word 3 (gfx9 family)
constexpr int kLoadNT = 2;                      // buffer load cache policy: nontemporal
constexpr int kBufferFar = 0x7ffffff0;          // a buffer offset past every range: reads 0

// XSRC: where x comes from -- kXFromWs: the prep launch's quantized x in the
// workspace; kXBf16 / kXF32: x itself, quantized here by every workgroup.
constexpr int kXFromWs = 0, kXBf16 = 1, kXF32 = 2;

template <int XSRC, bool XF16, int SCM>
__global__ void __launch_bounds__(kStreamThreads, 1)
    k_gemv_stream(const void* __restrict__ x, const uint8_t* __restrict__ ws, int B,
                  const uint8_t* __restrict__ W, const uint8_t* __restrict__ w_scales,
                  const float* __restrict__ g_w, int N, int K, int Kq, int lds_x_bytes, float g_d,
                  void* __restrict__ y, bool YBF16) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ uint32_t red_max[kStreamWaves];
  constexpr bool XBF16 = XSRC == kXBf16;
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

  // ---- x.  kXFromWs: the prep launch's x from the workspace (fp16 x' rows
  // [B][Kq] when XF16, else codes [B][Kq/2] followed by scale bytes
  // [B][Kq/16]), copied to LDS in 16-byte chunks.  Otherwise x itself, which
  // this workgroup quantizes (below).  Either way the first x loads are issued
  // before the first W loads, so they do not queue behind them in the
  // in-order load queue.
  const int row_chunks = XF16 ? Kq / 8 : Kq / 32;          // 16-byte chunks per x row
  const int nchunk = B * row_chunks + (XF16 ? 0 : B * bpr / 16);
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(ws + kWsData);
  auto x_dst = [&](int c) {
    if (XF16 || c < B * row_chunks) {
      const int row = c / row_chunks, k = c - row * row_chunks;
      // XF16: chunk k holds values 8k .. 8k + 7, at byte 2 (8k) + 16 (8k / 64)
      return reinterpret_cast<u32x4*>(XF16 ? lds + row * xf_row + 16 * k + 16 * (k / 8)
                                           : lds + row * xc_row + 16 * k);
    }
    return reinterpret_cast<u32x4*>(xs_base + 16 * (c - B * row_chunks));
  };
  u32x4 xr[kXRegVecs];  // workspace chunks (XSRC == kXFromWs)
  if constexpr (XSRC == kXFromWs) {
#pragma unroll
    for (int i = 0; i < kXRegVecs; ++i) {
      const int c = threadIdx.x + i * kStreamThreads;
      xr[i] = xsrc[c < nchunk ? c : 0];
    }
  }

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
  u32x4 xrb[kXB][VPB];  // x blocks (XSRC != kXFromWs)
  if constexpr (XSRC != kXFromWs) {
#pragma unroll
    for (int i = 0; i < kXB; ++i) {
      bool ok;
      const u32x4* src = block_src(threadIdx.x + i * kStreamThreads, ok);
#pragma unroll
      for (int v = 0; v < VPB; ++v) xrb[i][v] = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
    }
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
  u32x4 sga, sgb;                                 // scale group in flight
  const int w_lane = r8 * wrow + 16 * c8;
  const int s_lane = b * srow + 4 * g;
  const int g_lane = r8 * srow + 16 * c8;        // group loads: rows r8, 8 + r8, pair c8 of the group
  uint8_t* sa = lds + lds_x_bytes + kStreamWaves * 2048 + kRedBytes + wave * kGroupLds;
  int lr = 0, le = 0;                            // next element to load
  auto load_elem = [&](u32x4& a, u32x4& bb, uint32_t& sc) {
    const bool live = lr < nmine && le < E;
    const int r0 = lr < nmine ? (s_first + lr * G) * 16 : 0;
    const int rows = live ? min(16, N - r0) : 0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W) + (int64_t)r0 * wrow, 0, rows * wrow, kBufferWord3);
    const int pp = pbeg + le;
    a = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane, 128 * pp, kLoadNT);
    bb = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + 8 * wrow, 128 * pp, kLoadNT);
    if (SCM == kScaleGroup) {
      if (le % kGroupPairs == 0) {   // a scale group's first pair: the group's scale bytes
        const int grows = lr < nmine ? min(16, N - r0) : 0;
        const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(w_scales) + (int64_t)r0 * srow, 0, grows * srow, kBufferWord3);
        // (a group can reach past the scale row, and past the last row's end:
        // such reads fail the range check and return zeros)
        sga = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane, 16 * pp, 0);
        sgb = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane + 8 * srow, 16 * pp, 0);
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
  for (int i = 0; i < kPairs; ++i) load_elem(ra[i], rb[i], rs[i]);

  float s_gx;
  if constexpr (XSRC == kXFromWs) {
    // ---- x into LDS
  #pragma unroll
    for (int i = 0; i < kXRegVecs; ++i) {
      const int c = threadIdx.x + i * kStreamThreads;
      if (c < nchunk) *x_dst(c) = xr[i];
    }
    for (int c = threadIdx.x + kXRegVecs * kStreamThreads; c < nchunk; c += kStreamThreads)
      *x_dst(c) = xsrc[c];
    __syncthreads();
    s_gx = *reinterpret_cast<const float*>(ws + kWsHeader);
  } else {
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
      for (int v = 0; v < VPB; ++v) m = umax(m, vec_absmax(xrb[i][v]));
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
    const float s_gx_here = nv_global_scale(__uint_as_float(block_max_1024(m, red_max)));
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
      nv_block_scale(__uint_as_float(am), s_gx_here, sc, r);
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
      if (blk < nblk) quant_block(blk, xrb[i]);
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
    s_gx = s_gx_here;
  }
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
    const int q = ce % kGroupPairs;              // pair within its scale group
    if (SCM == kScaleGroup && q == 0) {          // [pair q][row b] x 16 bytes
      *reinterpret_cast<u32x4*>(sa + (16 * c8 + r8) * 16) = sga;
      *reinterpret_cast<u32x4*>(sa + (16 * c8 + 8 + r8) * 16) = sgb;
    }
    *reinterpret_cast<u32x4*>(tb + r8 * 128 + wsw) = ra_i;
    *reinterpret_cast<u32x4*>(tb + (8 + r8) * 128 + (wsw ^ 64)) = rb_i;
    load_elem(ra_i, rb_i, rs_i);
    if (ce < E) {
      if (SCM == kScaleGroup)
        sw = *reinterpret_cast<const uint32_t*>(sa + (16 * q + b) * 16 + 4 * g);
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

// ------------------------------------------------- FP4-MFMA GEMV (B <= 4) --
// Narrow batches: W's codes go into the FP4 MFMA as they are
// (v_mfma_scale_f32_16x16x128_f8f6f4, both operands E2M1, unit scales), with no
// dequantization.  W is loaded 8 rows x 128 contiguous bytes per instruction
// (16 rows x 64 bytes, the MFMA's operand shape, reads HBM ~35% slower) and
// reaches the MFMA layout through a wave-private XOR-swizzled LDS tile.  x is the other operand, laid out
// block-diagonally: for MFMA t of a 128-value step, row m of the x operand is
// batch row 2t + m / 8 restricted to the step's 16-value block m % 8 (zero
// elsewhere), so D[m][n] = sum over that block of E2M1(x) E2M1(w), one exact
// block dot product per output.  Lane (g, n) of the MFMA output holds
// D[4g + j][n], j = 0..3: W row n against x blocks 4 (g % 2) + j of batch row
// 2t + g / 2; it applies the two E4M3 block scales, acc += (s_x s_w) D, the
// product exact (at most 8 + 12 significant bits), one rounding per block (so
// a fused multiply-add gives the same sum in one instruction); W's
// four scale bytes for those blocks are contiguous.  Rounds, strips, the split
// of K between two waves and the exchange of partial sums are those of
// k_gemv_stream; every workgroup quantizes the small x itself.
// Pairs of 128-value steps in flight per wave (deeper rings measured slower).
// W's scale bytes come in groups of kGroupPairs pairs: 16 rows x 128 bytes, two
// loads of 8 rows x 128 bytes issued with the group's first pair and passed on
// through a 2 KB LDS area per wave (16-byte loads from 16 rows x 64 bytes cost
// ~2 us more per call at the decode shape; per-pair loads of a few bytes from
// 16 rows each would double the memory requests).
constexpr int kFp4Pairs = 2;
constexpr int kFp4WaveLds = 2048 + kGroupLds;   // transpose tile + scale group

template <bool XBF16, int NMF>
__global__ void __launch_bounds__(kStreamThreads, 1)
    k_gemv_fp4(const void* __restrict__ x, int B, const uint8_t* __restrict__ W,
               const uint8_t* __restrict__ w_scales, const float* __restrict__ g_w, int N, int K,
               int Kq, float g_d, void* __restrict__ y, bool YBF16) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ uint32_t red_max[kStreamWaves];
  typedef int v8i __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int nstrips = (N + 15) / 16;
  const int wrow = K / 2, srow = K / 16;
  const int S = Kq / 128;                        // 128-value steps
  const int bpr = Kq / 16;                       // x blocks per padded row
  // LDS: W transpose tiles [16 waves] x 2 KB | W scale groups [16 waves] x
  // [kGroupPairs pairs][16 rows] x 16 bytes | x operand tiles [NMF][S][64 lanes]
  // x 16 bytes | x block scales (E4M3 values) [2 NMF][bpr] floats | partial
  // sums [2][kSlots][64][NMF] floats
  uint8_t* tb = lds + wave * 2048;
  uint8_t* sgw = lds + kStreamWaves * 2048 + wave * kGroupLds;
  u32x4* xt = reinterpret_cast<u32x4*>(lds + kStreamWaves * kFp4WaveLds);
  float* sxs = reinterpret_cast<float*>(lds + kStreamWaves * kFp4WaveLds + NMF * S * 1024);
  float* red = sxs + 2 * NMF * bpr;

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

  // ---- W ring: a wave's elements are (round r, pair pbeg + e), e < Ep (as in
  // k_gemv_stream).  A pair is 16 strip rows x 128 bytes: lane l loads the
  // 16-byte chunk l % 8 of rows l / 8 and 8 + l / 8.  Chunk c holds values
  // 256 p + 32 c .. +32, which the MFMA of step c / 4 takes as K group c % 4 (x's
  // operand tiles follow the same order).  With a scale group's first pair p,
  // lane l loads the 16 scale bytes of pair p + l % 8 of rows l / 8 and
  // 8 + l / 8.
  const int part = wave / kSlots, slot = wave - part * kSlots;
  const int Pq = Kq / 256;
  const int Ph = (Pq + kSplit - 1) / kSplit;
  const int pbeg = min(part * Ph, Pq), pend = min(pbeg + Ph, Pq);
  const int E = pend - pbeg;
  const int Ep = (E + kFp4Pairs - 1) / kFp4Pairs * kFp4Pairs;
  const int G = gridDim.x * kSlots;
  const int s_first = slot * gridDim.x + blockIdx.x;
  const int R = (nstrips + G - 1) / G;
  const int nmine = s_first < nstrips ? (nstrips - s_first + G - 1) / G : 0;
  const int J = nmine * Ep;
  u32x4 ra[kFp4Pairs], rb[kFp4Pairs];
  u32x4 sga, sgb;                                // scale group in flight
  const int r8 = lane >> 3, c8 = lane & 7;
  const int w_lane = r8 * wrow + 16 * c8;
  const int g_lane = r8 * srow + 16 * c8;
  int lr = 0, le = 0;                            // next element to load
  auto load_elem = [&](int i) {
    const bool live = lr < nmine && le < E;
    const int r0 = lr < nmine ? (s_first + lr * G) * 16 : 0;
    const int rows = live ? min(16, N - r0) : 0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W) + (int64_t)r0 * wrow, 0, rows * wrow, kBufferWord3);
    const int pp = pbeg + le;
    ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane, 128 * pp, kLoadNT);
    rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + 8 * wrow, 128 * pp, kLoadNT);
    if (le % kGroupPairs == 0) {   // a scale group's first pair: the group's scale bytes
      const int grows = lr < nmine ? min(16, N - r0) : 0;
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(w_scales) + (int64_t)r0 * srow, 0, grows * srow, kBufferWord3);
      // (a group can reach past the scale row, and past the last row's end:
      // such reads fail the range check and return zeros)
      sga = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane, 16 * pp, 0);
      sgb = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane + 8 * srow, 16 * pp, 0);
    }
    if (++le >= Ep) { le = 0; ++lr; }
  };
#pragma unroll
  for (int i = 0; i < kFp4Pairs; ++i) load_elem(i);

  // ---- x operand tiles and block scales start at zero (padding blocks, the
  // other batch row of a tile, batch rows past B); the barriers of the amax
  // reduction order these stores before the quantized blocks' stores
  for (int i = threadIdx.x; i < NMF * S * 64; i += kStreamThreads) xt[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < 2 * NMF * bpr; i += kStreamThreads) sxs[i] = 0.0f;

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
  for (int blk0 = threadIdx.x + kXB * kStreamThreads; blk0 < nblk; blk0 += kStreamThreads) {
    bool ok;
    const u32x4* src = block_src(blk0, ok);
#pragma unroll
    for (int v = 0; v < VPB; ++v) m = umax(m, vec_absmax(ok ? src[v] : u32x4{0u, 0u, 0u, 0u}));
  }
  const float s_gx = nv_global_scale(__uint_as_float(block_max_1024(m, red_max)));
  auto quant_block = [&](int blk, const u32x4 (&vv)[VPB]) {
    const int row = blk / bpr, kb = blk - row * bpr;
    if (kb * 16 >= K) return;                    // padding past K stays zero
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
    sxs[row * bpr + kb] = e4m3_value(sc);
    // tile t = row / 2, x row m = 8 (row % 2) + i of step kb / 8, block i = kb % 8
    // in K group i / 2 (lane m + 16 (i / 2)), half i % 2 of that lane's 16 bytes
    const int i = kb & 7, mrow = ((row & 1) << 3) | i;
    uint8_t* dst = reinterpret_cast<uint8_t*>(xt) +
                   (((row >> 1) * S + (kb >> 3)) * 64 + mrow + 16 * (i >> 1)) * 16 + 8 * (i & 1);
    *reinterpret_cast<u32x2*>(dst) = u32x2{e2m1_pack8(v), e2m1_pack8(v + 8)};
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
  float acc[NMF];
#pragma unroll
  for (int t = 0; t < NMF; ++t) acc[t] = 0.0f;
  // Sum over the lane pair holding one (batch row, W row) -- g and g ^ 1 -- then
  // over the two K parts (the upper part's sums go through LDS, double-buffered
  // by round parity, one barrier per round), in a fixed order; write y.
  auto finish = [&](int r, bool valid) {
    float a[NMF];
#pragma unroll
    for (int t = 0; t < NMF; ++t) a[t] = acc[t] + __shfl_xor(acc[t], 16, 64);
    float* rp = red + (((r & 1) * kSlots + slot) * 64 + lane) * NMF;
    if (part != 0) {
#pragma unroll
      for (int t = 0; t < NMF; ++t) rp[t] = a[t];
    }
    __syncthreads();
    if (part != 0 || !valid) return;
#pragma unroll
    for (int t = 0; t < NMF; ++t) a[t] = a[t] + rp[t];
    const int nn = (s_first + r * G) * 16 + n16;
    if ((g & 1) == 0 && nn < N) {
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        const int ob = 2 * t + (g >> 1);
        if (ob < B) {
          const float v = (a[t] * gscale) * g_d;
          if (YBF16)
            reinterpret_cast<uint16_t*>(y)[(int64_t)ob * N + nn] = (uint16_t)f32_to_bf16(v);
          else
            reinterpret_cast<float*>(y)[(int64_t)ob * N + nn] = v;
        }
      }
    }
  };
  int cr = 0, ce = 0;                            // element being computed
  const float* sx_lane = sxs + (g >> 1) * bpr + 4 * (g & 1);
  // transpose tile: 16-byte chunk c of row r at chunk position c ^ (r % 8) ^ 4 (r / 8)
  const int wsw = (r8 ^ c8) << 4;
  auto elem = [&](int i) {
    const int q = ce % kGroupPairs;                // pair within its scale group
    if (q == 0) {                                // [pair q][row n] x 16 bytes
      *reinterpret_cast<u32x4*>(sgw + (16 * c8 + r8) * 16) = sga;
      *reinterpret_cast<u32x4*>(sgw + (16 * c8 + 8 + r8) * 16) = sgb;
    }
    *reinterpret_cast<u32x4*>(tb + r8 * 128 + wsw) = ra[i];
    *reinterpret_cast<u32x4*>(tb + (8 + r8) * 128 + (wsw ^ 64)) = rb[i];
    load_elem(i);
    if (ce < E) {
      const int step = 2 * (pbeg + ce);
      // row n's scale bytes of this pair, blocks 8 st + 4 (g % 2) .. +3
      const u32x2 sw2 = u32x2{*reinterpret_cast<const uint32_t*>(sgw + (16 * q + n16) * 16 + 4 * (g & 1)),
                              *reinterpret_cast<const uint32_t*>(sgw + (16 * q + n16) * 16 + 8 + 4 * (g & 1))};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int c = 4 * st + g;                  // the chunk that is this lane's K group
        const u32x4 wv = *reinterpret_cast<const u32x4*>(
            tb + n16 * 128 + ((c ^ (n16 & 7) ^ ((n16 >> 3) << 2)) << 4));
        const uint32_t sw = st ? sw2.y : sw2.x;
        const v8i wo = {(int)wv.x, (int)wv.y, (int)wv.z, (int)wv.w, 0, 0, 0, 0};
        // the four E4M3 scale bytes of W row n, blocks 4 (g % 2) .. +3 of the step
        const f32x2 w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, false);
        const f32x2 w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, true);
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
          const u32x4 xo4 = xt[(t * S + step + st) * 64 + lane];
          const v8i xo = {(int)xo4.x, (int)xo4.y, (int)xo4.z, (int)xo4.w, 0, 0, 0, 0};
          const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              xo, wo, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, 127, 0, 127);
          const f32x4 sx = *reinterpret_cast<const f32x4*>(sx_lane + 2 * t * bpr + 8 * (step + st));
          acc[t] = __builtin_fmaf(sx.x * w01.x, d.x, acc[t]);
          acc[t] = __builtin_fmaf(sx.y * w01.y, d.y, acc[t]);
          acc[t] = __builtin_fmaf(sx.z * w23.x, d.z, acc[t]);
          acc[t] = __builtin_fmaf(sx.w * w23.y, d.w, acc[t]);
        }
      }
    }
    if (ce == Ep - 1) {
      finish(cr, true);
#pragma unroll
      for (int t = 0; t < NMF; ++t) acc[t] = 0.0f;
    }
    if (++ce == Ep) { ce = 0; ++cr; }
  };
  for (int j0 = 0; j0 < J; j0 += kFp4Pairs) {
#pragma unroll
    for (int i = 0; i < kFp4Pairs; ++i) elem(i);
  }
  // every wave takes part in all R rounds' exchanges (see k_gemv_stream)
  for (int r = Ep > 0 ? nmine : 0; r < R; ++r) finish(r, r < nmine);
}

// ------------------------------------------ GEMV with x' in registers --
// Batches whose fp16 x' does not fit LDS, up to 16 rows, K a multiple of 256
// up to 5120: x, quantized once by the prep launch (codes + scale bytes), is copied into LDS
// and each wave dequantizes its share of it once, into registers, instead of
// once per strip (fp16 x' of 16 rows x 5120 values would need all of LDS).
// A workgroup of 8 waves (two per SIMD, 256 registers each) serves two strips
// at a time; the four waves of a strip take a quarter of K each and hold its
// exact fp16 x' (at most 5 pairs of 128-value steps: 160 registers) for the
// whole kernel.  W streams as in k_gemv_stream (8 rows x 128 bytes per load,
// through a wave-private transpose tile; W scale bytes of the wave's pairs of
// a strip with two loads of 8 rows x 16 bytes per pair), with a ring of one
// round (the wave's pairs of its next strip) in flight.  Per round, the three
// upper quarters' partial tiles go through LDS (double-buffered by round
// parity, one barrier per round) to the lowest quarter's wave, which adds them
// in a fixed order and writes y.  K order inside a pair and the MFMA use are
// those of k_gemv_stream.
constexpr int kXrThreads = 512;
constexpr int kXrWaves = kXrThreads / 64;
constexpr int kXrSplit = 4;                      // waves per strip (K parts)
constexpr int kXrSlots = kXrWaves / kXrSplit;    // strips per workgroup and round
constexpr int kXrMaxPairs = 5;                   // pairs of x' per wave (K <= 5120)
constexpr int kXrChunks = 6;                     // 16-byte x chunks per thread (16 rows, K <= 5120)

// LDS for x of B rows of Kq values: codes [B][Kq / 2 + 16] then scale bytes
// [B][Kq / 16] (a multiple of 16 bytes); 16 spare bytes follow
__host__ __device__ inline int xreg_lds_bytes(int B, int Kq) { return B * (Kq / 2 + 16) + B * (Kq / 16); }

// y is written through a buffer descriptor with 32-bit offsets (the host
// keeps B * N * sizeof(y) below 2^31).
template <bool YBF16>
__global__ void __launch_bounds__(kXrThreads, 1)
    k_gemv_xreg(const uint8_t* __restrict__ ws, int B, const uint8_t* __restrict__ W,
                const uint8_t* __restrict__ w_scales, const float* __restrict__ g_w, int N, int K,
                int Kq, float g_d, void* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kXrWaves][2048];
  __shared__ __attribute__((aligned(16))) uint8_t sgroup[kXrWaves][kGroupLds];
  __shared__ v4f red[2][kXrSlots][kXrSplit - 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = lane & 15, g = lane >> 4;
  const int r8 = lane >> 3, c8 = lane & 7;
  const int nstrips = (N + 15) / 16;
  const int wrow = K / 2, srow = K / 16;
  const int part = wave / kXrSlots, slot = wave - part * kXrSlots;
  const int Pq = Kq / 256;
  const int Ph = (Pq + kXrSplit - 1) / kXrSplit;  // <= kXrMaxPairs (host check)
  const int pbeg = min(part * Ph, Pq), pend = min(pbeg + Ph, Pq);
  const int E = pend - pbeg;                       // this wave's pairs
  const int G = gridDim.x * kXrSlots;              // strips per round
  const int s_first = slot * gridDim.x + blockIdx.x;
  const int R = (nstrips + G - 1) / G;             // rounds (the same in every workgroup)
  const int nmine = s_first < nstrips ? (nstrips - s_first + G - 1) / G : 0;
  uint8_t* tb = tiles[wave];
  uint8_t* sa = sgroup[wave];

  // ---- x from the workspace (codes [B][Kq/2], then scale bytes [B][Kq/16]) in
  // 16-byte chunks, into registers first: these loads are issued before W's
  // so that waiting for them does not wait for W (loads complete in order)
  const int xc_row = Kq / 2 + 16, bpr = Kq / 16;
  const int row_chunks = Kq / 32;
  const int nchunk = B * row_chunks + B * bpr / 16;
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(ws + kWsData);
  u32x4 xch[kXrChunks];
#pragma unroll
  for (int i = 0; i < kXrChunks; ++i) {
    const int c = threadIdx.x + i * kXrThreads;
    xch[i] = xsrc[c < nchunk ? c : 0];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- W ring: slot e holds pair pbeg + e of the strip of round r.  Reads of
  // rounds without a strip and of pairs past E go through an empty range
  // (zeros, no memory touched).
  u32x4 ra[kXrMaxPairs], rb[kXrMaxPairs];
  u32x4 sga, sgb;                                  // scale bytes of a round's pairs in flight
  const int w_lane = r8 * wrow + 16 * c8;
  // scale loads: lane (r8, c8) takes the 16 bytes of pair pbeg + c8 of rows r8
  // and 8 + r8 (pairs past E: offset out of every range)
  const int g_lane = c8 < E ? r8 * srow + 16 * c8 : kBufferFar;
  const int g_lane8 = c8 < E ? (8 + r8) * srow + 16 * c8 : kBufferFar;
  auto strip_rows = [&](int r) {
    const int r0 = r < nmine ? (s_first + r * G) * 16 : 0;
    return r < nmine ? min(16, N - r0) : 0;
  };
  auto strip_row0 = [&](int r) { return r < nmine ? (s_first + r * G) * 16 : 0; };
  auto load_pair = [&](int r, int e) {
    const int r0 = strip_row0(r);
    const int rows = e < E ? strip_rows(r) : 0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W) + (int64_t)r0 * wrow, 0, rows * wrow, kBufferWord3);
    ra[e] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane, 128 * (pbeg + e), kLoadNT);
    rb[e] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + 8 * wrow, 128 * (pbeg + e), kLoadNT);
  };
  auto load_scales = [&](int r) {
    const int r0 = strip_row0(r);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w_scales) + (int64_t)r0 * srow, 0, strip_rows(r) * srow, kBufferWord3);
    sga = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane, 16 * pbeg, 0);
    sgb = __builtin_amdgcn_raw_buffer_load_b128(rsc, g_lane8, 16 * pbeg, 0);
  };
  // issue order: the scale bytes, then the pairs in order, as inside the loop,
  // so that the loop's waits count only the loads it needs (loads complete in
  // order)
  __builtin_amdgcn_sched_barrier(0);
  load_scales(0);
#pragma unroll
  for (int e = 0; e < kXrMaxPairs; ++e) {
    __builtin_amdgcn_sched_barrier(0);
    load_pair(0, e);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- x into LDS, then this wave's x' into registers: lane (b, g) holds
  // x'[b][256 p + 64 g + 32 st + 8 s4, +8) (batch rows >= B: row B - 1, any
  // finite x, never stored)
  // (every thread stores every chunk, those past nchunk into a spare 16 bytes
  // after x: a store under a branch would let the compiler move its load
  // there, behind W's)
#pragma unroll
  for (int i = 0; i < kXrChunks; ++i) {
    const int c = threadIdx.x + i * kXrThreads;
    const int row = c / row_chunks;
    const int off = c >= nchunk ? xreg_lds_bytes(B, Kq)
                    : c < B * row_chunks ? row * xc_row + 16 * (c - row * row_chunks)
                                         : B * xc_row + 16 * (c - B * row_chunks);
    *reinterpret_cast<u32x4*>(xlds + off) = xch[i];
  }
  __syncthreads();
  const int xrow = min(b, B - 1);
  v8h xr[kXrMaxPairs][2][4];
#pragma unroll
  for (int e = 0; e < kXrMaxPairs; ++e) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // (registers past E are never used: any pair inside x)
      const int v0 = 256 * min(pbeg + min(e, max(E - 1, 0)), Pq - 1) + 64 * g + 32 * st;
      const u32x4 xc = *reinterpret_cast<const u32x4*>(xlds + xrow * xc_row + v0 / 2);
      const uint32_t xsb = *reinterpret_cast<const uint16_t*>(xlds + B * xc_row + xrow * bpr + v0 / 16);
      const v2h hp = e4m3_pair_h<false>(xsb);
      const v2h h0 = v2h{hp.x, hp.x}, h1 = v2h{hp.y, hp.y};
      xr[e][st][0] = dq8(xc.x, h0);
      xr[e][st][1] = dq8(xc.y, h0);
      xr[e][st][2] = dq8(xc.z, h1);
      xr[e][st][3] = dq8(xc.w, h1);
    }
  }

  const float gscale = *reinterpret_cast<const float*>(ws + kWsHeader) * (*g_w);
  const __amdgpu_buffer_rsrc_t ry =
      __builtin_amdgcn_make_buffer_rsrc(y, 0, B * N * (YBF16 ? 2 : 4), kBufferWord3);
  const int wsw = (r8 ^ c8) << 4;
  for (int r = 0; r < R; ++r) {
    const bool mine = r < nmine;
    v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
    for (int e = 0; e < kXrMaxPairs; ++e) {
      if (e == 0) {   // [pair q][row] x 16 bytes
        *reinterpret_cast<u32x4*>(sa + (16 * c8 + r8) * 16) = sga;
        *reinterpret_cast<u32x4*>(sa + (16 * c8 + 8 + r8) * 16) = sgb;
        load_scales(r + 1);
      }
      *reinterpret_cast<u32x4*>(tb + r8 * 128 + wsw) = ra[e];
      *reinterpret_cast<u32x4*>(tb + (8 + r8) * 128 + (wsw ^ 64)) = rb[e];
      load_pair(r + 1, e);
      if (mine && e < E) {
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(sa + (16 * e + b) * 16 + 4 * g);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int c = 2 * g + st;
          const u32x4 codes = *reinterpret_cast<const u32x4*>(
              tb + b * 128 + ((c ^ (b & 7) ^ ((b >> 3) << 2)) << 4));
          const v2h wp = st ? e4m3_pair_h<true>(sw) : e4m3_pair_h<false>(sw);
          const v2h w0 = v2h{wp.x, wp.x}, w1 = v2h{wp.y, wp.y};
          v4f& acc = st ? acc1 : acc0;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xr[e][st][0], dq8(codes.x, w0), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xr[e][st][1], dq8(codes.y, w0), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xr[e][st][2], dq8(codes.z, w1), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xr[e][st][3], dq8(codes.w, w1), acc, 0, 0, 0);
        }
      }
    }
    // the upper quarters' partial tiles to the lowest quarter's wave (every
    // wave takes part in every round's barrier)
    v4f a = acc0 + acc1;
    if (part != 0) red[r & 1][slot][part - 1][lane] = a;
    __syncthreads();
    if (part == 0 && mine) {
#pragma unroll
      for (int p = 0; p < kXrSplit - 1; ++p) a += red[r & 1][slot][p][lane];
      const int n0 = (s_first + r * G) * 16;     // D[4g + q][b] of this strip
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ob = 4 * g + q;
        if (ob < B && n0 + b < N) {
          const float v = (a[q] * gscale) * g_d;
          if (YBF16)
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16(v), ry,
                                                  2 * (ob * N + b), 2 * n0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, 4 * (ob * N + b), 4 * n0, 0);
        }
      }
    }
  }
}

// K = 0: every output is an empty sum.
template <typename T>
__global__ void __launch_bounds__(256) k_zero_fill(int64_t n, T* __restrict__ y) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) y[i] = 0;
}

struct StreamArgs {
  const void* x;
  const uint8_t* ws;
  int B;
  const uint8_t* W;
  const uint8_t* w_scales;
  const float* g_w;
  int N, K, Kq, lds_x;
  float g_d;
  void* y;
  bool y_bf16;
};

template <bool XB, int NMF>
hipError_t launch_fp4(const StreamArgs& a, int grid, int lds, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = fp4impl::set_lds_limit_once(
      lds_set, reinterpret_cast<const void*>(&k_gemv_fp4<XB, NMF>), kStreamLdsMax);
  if (e != hipSuccess) return e;
  if (lds > kStreamLdsMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemv_fp4<XB, NMF>), dim3(grid), dim3(kStreamThreads), lds, stream, a.x, a.B,
                     a.W, a.w_scales, a.g_w, a.N, a.K, a.Kq, a.g_d, a.y, a.y_bf16);
  return hipGetLastError();
}

template <int XS, bool XF, int SCM>
hipError_t launch_stream(const StreamArgs& a, int grid, int lds, hipStream_t stream) {
  // the limit is set once per device to the most any call of this kernel uses
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = fp4impl::set_lds_limit_once(
      lds_set, reinterpret_cast<const void*>(&k_gemv_stream<XS, XF, SCM>), kStreamLdsMax);
  if (e != hipSuccess) return e;
  if (lds > kStreamLdsMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemv_stream<XS, XF, SCM>), dim3(grid), dim3(kStreamThreads), lds, stream,
                     a.x, a.ws, a.B, a.W, a.w_scales, a.g_w, a.N, a.K, a.Kq, a.lds_x, a.g_d, a.y,
                     a.y_bf16);
  return hipGetLastError();
}

template <bool YB>
hipError_t launch_xreg(const uint8_t* ws, int64_t B, const uint8_t* W, const uint8_t* w_scales,
                       const float* g_w, int64_t N, int64_t K, int64_t Kq, float g_d, void* y,
                       int grid, int lds_x, hipStream_t stream) {
  // the most dynamic LDS any call uses (16 rows, K = 5120), set once per device
  static std::atomic<uint64_t> lds_set{0};
  const int lds_max = xreg_lds_bytes(16, 256 * kXrSplit * kXrMaxPairs) + 16;
  const hipError_t e = fp4impl::set_lds_limit_once(
      lds_set, reinterpret_cast<const void*>(&k_gemv_xreg<YB>), lds_max);
  if (e != hipSuccess) return e;
  if (lds_x > lds_max) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemv_xreg<YB>, dim3(grid), dim3(kXrThreads), lds_x, stream, ws, (int)B, W,
                     w_scales, g_w, (int)N, (int)K, (int)Kq, g_d, y);
  return hipGetLastError();
}

// x [B, K] -> the workspace (k_gemv_xquant), with the amax of a larger x from
// per-workgroup partial maxima first.
hipError_t launch_xquant(const void* x, bool x_bf16, int64_t B, int64_t K, int64_t Kpad,
                         bool f16_out, uint8_t* ws, hipStream_t stream) {
  const uint32_t* partials = nullptr;
  int npart = 0;
  if (B * K > kSmallX) {
    uint32_t* p = reinterpret_cast<uint32_t*>(ws + kWsPartials);
    hipError_t e = fp4impl::launch_amax(x, x_bf16, B * K, p, &npart, stream);
    if (e != hipSuccess) return e;
    partials = p;
  }
  const int64_t nblk = B * (Kpad / 16);
  const dim3 grid((unsigned)((nblk + kPrepThreads - 1) / kPrepThreads));
#define FP4_XQ(XB, F16)                                                                    \
  hipLaunchKernelGGL((k_gemv_xquant<XB, F16>), grid, dim3(kPrepThreads), 0, stream, x, B, K, \
                     Kpad, partials, npart, ws)
  if (x_bf16) {
    if (f16_out) FP4_XQ(true, true); else FP4_XQ(true, false);
  } else {
    if (f16_out) FP4_XQ(false, true); else FP4_XQ(false, false);
  }
#undef FP4_XQ
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
  // the larger of the streaming kernel's x (fp16 rows of K rounded up to 256)
  // and the long-K kernel's (fp16 rows of K rounded up to 128)
  const int64_t Kq = (K + 255) / 256 * 256;
  return kWsData + (size_t)(B * Kq * 2);
}

hipError_t launch_gemv(const void* x, bool x_bf16, int64_t B, const uint8_t* W,
                       const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K, float g_d,
                       void* y, bool y_bf16, void* workspace, hipStream_t stream) {
  if (N > (1 << 30) || K > (1 << 30)) return hipErrorInvalidValue;
  const int ncu = fp4impl::num_cus();
  if (K == 0) return launch_zero_fill(y, B * N, y_bf16 ? 2 : 4, stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int nstrips = (int)((N + 15) / 16);
  // streaming kernel when the quantized x fits in LDS
  const int64_t Kq = (K + 255) / 256 * 256;
  const int64_t lds_f16 = B * xf16_row_bytes((int)Kq);
  const int64_t lds_fp4 = B * (Kq / 2 + 16) + B * (Kq / 16);
  int scm = kScaleHalf;
  if (K % 64 == 0 && reinterpret_cast<uintptr_t>(w_scales) % 4 == 0) scm = kScaleDword;
  if (K % 256 == 0 && reinterpret_cast<uintptr_t>(w_scales) % 16 == 0) scm = kScaleGroup;
  const int64_t lds_fixed = kStreamWaves * 2048 + kRedBytes + kStreamWaves * kGroupLds;
  const int64_t lds_max = kStreamLdsMax;
  const bool xf16 = lds_f16 + lds_fixed <= lds_max;
  // (the strip-relative buffer offsets need 16 rows of W to span < 2^31 bytes;
  // the x' sizes above already keep K far below that)
  // narrow batches (K a multiple of 64, 4-aligned scale rows): the FP4-MFMA kernel
  if (B <= 4 && K % 64 == 0 && reinterpret_cast<uintptr_t>(w_scales) % 4 == 0 && K < (1 << 27)) {
    const int nmf = (int)((B + 1) / 2);
    const int64_t lds_k = kStreamWaves * kFp4WaveLds + nmf * (Kq / 128) * 1024 + 2 * nmf * (Kq / 16) * 4 +
                          2 * kSlots * 64 * nmf * 4;
    if (lds_k <= lds_max) {
      const int grid = nstrips < ncu ? nstrips : ncu;
      const StreamArgs sa{x, ws, (int)B, W, w_scales, g_w, (int)N, (int)K, (int)Kq, 0, g_d, y, y_bf16};
      if (x_bf16)
        return nmf == 1 ? launch_fp4<true, 1>(sa, grid, (int)lds_k, stream)
                        : launch_fp4<true, 2>(sa, grid, (int)lds_k, stream);
      return nmf == 1 ? launch_fp4<false, 1>(sa, grid, (int)lds_k, stream)
                      : launch_fp4<false, 2>(sa, grid, (int)lds_k, stream);
    }
  }
  // fp16 x' too large for LDS, up to 16 batch rows, K a multiple of 256 up to
  // 5120, 16-aligned scale rows: x quantized once, then x' held in registers;
  // the grid is cut so that every workgroup serves the same number of rounds
  if (!xf16 && B <= 16 && K % 256 == 0 && Kq / 256 <= kXrSplit * kXrMaxPairs &&
      reinterpret_cast<uintptr_t>(w_scales) % 16 == 0 && B * N * 4 < ((int64_t)1 << 31)) {
    const int lds_x = xreg_lds_bytes((int)B, (int)Kq) + 16;
    hipError_t e = launch_xquant(x, x_bf16, B, K, Kq, false, ws, stream);
    if (e != hipSuccess) return e;
    const int per_round = ncu * kXrSlots;
    const int rounds = (nstrips + per_round - 1) / per_round;
    const int grid = (nstrips + kXrSlots * rounds - 1) / (kXrSlots * rounds);
    return y_bf16 ? launch_xreg<true>(ws, B, W, w_scales, g_w, N, K, Kq, g_d, y, grid, lds_x, stream)
                  : launch_xreg<false>(ws, B, W, w_scales, g_w, N, K, Kq, g_d, y, grid, lds_x, stream);
  }
  if ((xf16 || lds_fp4 + lds_fixed <= lds_max) && K < (1 << 27)) {
    // x' fits LDS as fp16 (narrow batches): every workgroup quantizes the
    // small x itself, one launch in all; wider batches: the prep launch
    // quantizes x once into the workspace (in every workgroup that work would
    // cost more than the extra launch)
    const int xs = xf16 ? (x_bf16 ? kXBf16 : kXF32) : kXFromWs;
    if (xs == kXFromWs) {
      hipError_t e = launch_xquant(x, x_bf16, B, K, Kq, false, ws, stream);
      if (e != hipSuccess) return e;
    }
    const int lds_x = (int)(((xf16 ? lds_f16 : lds_fp4) + 15) / 16 * 16);
    const int lds = lds_x + (int)lds_fixed;
    const int grid = nstrips < ncu ? nstrips : ncu;
    const StreamArgs sa{x, ws, (int)B, W, w_scales, g_w, (int)N, (int)K, (int)Kq, lds_x, g_d, y, y_bf16};
    switch (xs * 3 + scm) {
      case 0: return launch_stream<kXFromWs, false, kScaleHalf>(sa, grid, lds, stream);
      case 1: return launch_stream<kXFromWs, false, kScaleDword>(sa, grid, lds, stream);
      case 2: return launch_stream<kXFromWs, false, kScaleGroup>(sa, grid, lds, stream);
      case 3: return launch_stream<kXBf16, true, kScaleHalf>(sa, grid, lds, stream);
      case 4: return launch_stream<kXBf16, true, kScaleDword>(sa, grid, lds, stream);
      case 5: return launch_stream<kXBf16, true, kScaleGroup>(sa, grid, lds, stream);
      case 6: return launch_stream<kXF32, true, kScaleHalf>(sa, grid, lds, stream);
      case 7: return launch_stream<kXF32, true, kScaleDword>(sa, grid, lds, stream);
      default: return launch_stream<kXF32, true, kScaleGroup>(sa, grid, lds, stream);
    }
  }

  // very long K: x' through the workspace, waves split K
  const int64_t Kp = kpad(K);
  hipError_t e = launch_xquant(x, x_bf16, B, K, Kp, true, ws, stream);
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
