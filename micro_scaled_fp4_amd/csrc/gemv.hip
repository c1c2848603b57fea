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
#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kPrepThreads = 256;
constexpr size_t kHeader = 256;        // workspace header: [0] s_global of x
constexpr int kMaxWaves = 16;
constexpr int kMaxSteps = 4;           // 128-value steps per wave kept in registers

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

  // x' fragments of this wave's K range: step i, MFMA sub-step s -> 8 fp16
  v8h xf[kMaxSteps][4];
  if (RESIDENT) {
#pragma unroll
    for (int i = 0; i < kMaxSteps; ++i) {
      const int t = t0 + i;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (i < spw && t < T && b < B)
          xf[i][s] = *reinterpret_cast<const v8h*>(xp + (int64_t)b * Kp + 128 * t + 32 * g + 8 * s);
        else
          xf[i][s] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  const float gscale = reinterpret_cast<const float*>(ws)[0] * (*g_w);
  const int nstrips = (N + 15) / 16;
  for (int strip = blockIdx.x; strip < nstrips; strip += gridDim.x) {
    const int n0 = strip * 16;
    const int row = min(n0 + b, N - 1);
    const uint8_t* wr = W + (int64_t)row * wrow_bytes;
    const uint8_t* sr = w_scales + (int64_t)row * srow_bytes;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i0 = 0; i0 < spw; i0 += kMaxSteps) {
      u32x4 codes[kMaxSteps];
      uint32_t sbytes[kMaxSteps];
#pragma unroll
      for (int i = 0; i < kMaxSteps; ++i) {
        const int t = t0 + i0 + i;
        const int kc = 128 * t + 32 * g;
        if (i0 + i < spw && t < T && kc < K) {
          codes[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + kc / 2));
          sbytes[i] = *reinterpret_cast<const uint16_t*>(sr + kc / 16);
        } else {
          codes[i] = u32x4{0, 0, 0, 0};
          sbytes[i] = 0;
        }
      }
#pragma unroll
      for (int i = 0; i < kMaxSteps; ++i) {
        if (i0 + i >= spw) break;
        const int t = t0 + i0 + i;
        v8h xv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (RESIDENT) {
            xv[s] = xf[i][s];
          } else {
            xv[s] = (t < T && b < B) ? *reinterpret_cast<const v8h*>(xp + (int64_t)b * Kp + 128 * t + 32 * g + 8 * s)
                                     : v8h{0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
        float p0, p1;
        v2h m0, m1;
        e4m3_split(sbytes[i] & 0xffu, p0, m0);
        e4m3_split(sbytes[i] >> 8, p1, m1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[0], dequant8(codes[i].x, p0, m0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[1], dequant8(codes[i].y, p0, m0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[2], dequant8(codes[i].z, p1, m1), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[3], dequant8(codes[i].w, p1, m1), acc, 0, 0, 0);
      }
    }
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
}

int g_num_cus = 0;

}  // namespace

namespace fp4impl {

size_t gemv_workspace_bytes(int64_t B, int64_t K) {
  return kHeader + (size_t)(B * kpad(K) * 2);
}

hipError_t launch_gemv(const void* x, bool x_bf16, int64_t B, const uint8_t* W,
                       const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K, float g_d,
                       void* y, bool y_bf16, void* workspace, hipStream_t stream) {
  if (N > (1 << 30) || K > (1 << 30)) return hipErrorInvalidValue;
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

  if (g_num_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      g_num_cus = cus;
    else
      g_num_cus = 256;
  }
  const int T = (int)(Kp / 128);
  int spw = (T + kMaxWaves - 1) / kMaxWaves;
  if (spw < 1) spw = 1;
  const int nwaves = (T + spw - 1) / spw;
  const bool resident = spw <= kMaxSteps;
  const int nstrips = (int)((N + 15) / 16);
  const int grid = nstrips < g_num_cus ? nstrips : g_num_cus;
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
