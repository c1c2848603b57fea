// Decode-time batched GEMV  y = g_d * x_hat @ W_hat^T  with NVFP4 weights and
// activations quantized on the fly (one tensor scale over the whole [B, K]).
//
// Written from the scaled-GEMM equation of the "NVIDIA NVFP4 与 Micro-Scaling"
// article (section 三); the 10100.com data-type article announces an "FP4 batch
// GEMV" whose text is not on the pages.
//
// Two launches: (1) x -> NVFP4 into the workspace, bit-identical to
// nvfp4_quantize (every workgroup reduces the tiny x for the global amax
// itself, so no cross-workgroup pass is needed); (2) stream W.
// Accumulation: each 16-value block contributes s_x * s_w * sum(v_x * v_w),
// which is exact in float32 (E2M1 products are multiples of 1/4, a block dot
// needs <= 12 bits, the two E4M3 scales <= 8); block terms are summed in
// float32, first along a lane's chunks, then by a butterfly across lanes.
#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr size_t kHeader = 256;  // workspace header: [0] s_global of x

inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = umax(r, red[i]);
  __syncthreads();
  return r;
}

template <bool BF16>
__device__ __forceinline__ void load16(const void* __restrict__ x, int64_t b, float (&v)[16]) {
  if (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x) + 2 * b;
    const u32x4 a = p[0], c = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_lo(w[j]);
      v[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(x) + 4 * b;
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

__device__ __forceinline__ uint32_t pack8(const uint32_t (&c)[8]) {
  return c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) |
         (c[6] << 24) | (c[7] << 28);
}

// x [n elements, n % 16 == 0] -> codes, scale bytes, s_global in the workspace.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_gemv_xquant(const void* __restrict__ x, int64_t n, uint8_t* __restrict__ ws,
                  size_t codes_off, size_t scales_off) {
  // global amax of x (x is small; every workgroup reduces all of it)
  const int per = BF16 ? 8 : 4;
  const int64_t nvec = n / per;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < nvec; i += kThreads) {
    const u32x4 v = xv[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
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
  const float G = __uint_as_float(block_max_u32(m));
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) reinterpret_cast<float*>(ws)[0] = s_global;
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b < n / 16) {
    float v[16];
    load16<BF16>(x, b, v);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = umax(amax, __float_as_uint(v[j]) & 0x7fffffffu);
    uint32_t sc;
    float r;
    nv_block_scale(__uint_as_float(amax), s_global, sc, r);
    uint32_t c[8], d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c[j] = e2m1_code(v[j] * r);
      d[j] = e2m1_code(v[8 + j] * r);
    }
    reinterpret_cast<u32x2*>(ws + codes_off)[b] = u32x2{pack8(c), pack8(d)};
    ws[scales_off + b] = (uint8_t)sc;
  }
}

// W streaming: each wave handles two rows, 32 lanes per row; a lane walks
// 32-value chunks (16 code bytes + 2 scale bytes) of its row.
template <int B, bool YBF16>
__global__ void __launch_bounds__(kThreads)
    k_gemv(const uint8_t* __restrict__ W, const uint8_t* __restrict__ w_scales,
           const float* __restrict__ g_w, int64_t N, int64_t K, float g_d,
           const uint8_t* __restrict__ ws, size_t codes_off, size_t scales_off,
           void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t n = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const int sub = lane & 31;
  const int64_t nchunk = K / 32;
  const uint8_t* xq = ws + codes_off;
  const uint8_t* xs = ws + scales_off;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  if (n < N) {
    const uint8_t* wrow = W + n * (K / 2);
    const uint8_t* srow = w_scales + n * (K / 16);
    for (int64_t c = sub; c < nchunk; c += 32) {
      const u32x4 wc = *reinterpret_cast<const u32x4*>(wrow + 16 * c);
      const uint32_t wsc = *reinterpret_cast<const uint16_t*>(srow + 2 * c);
      const uint32_t ww[4] = {wc.x, wc.y, wc.z, wc.w};
      float wv[32];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[8 * k + j] = e2m1_value((ww[k] >> (4 * j)) & 15u);
      const float sw0 = e4m3_value(wsc & 0xffu), sw1 = e4m3_value(wsc >> 8);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const u32x4 xc = *reinterpret_cast<const u32x4*>(xq + (int64_t)b * (K / 2) + 16 * c);
        const uint32_t xsc = *reinterpret_cast<const uint16_t*>(xs + (int64_t)b * (K / 16) + 2 * c);
        const uint32_t xw[4] = {xc.x, xc.y, xc.z, xc.w};
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int j = 0; j < 8; ++j) d0 = __builtin_fmaf(e2m1_value((xw[k] >> (4 * j)) & 15u), wv[8 * k + j], d0);
#pragma unroll
        for (int k = 2; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 8; ++j) d1 = __builtin_fmaf(e2m1_value((xw[k] >> (4 * j)) & 15u), wv[8 * k + j], d1);
        const float t0 = d0 * (e4m3_value(xsc & 0xffu) * sw0);   // exact
        const float t1 = d1 * (e4m3_value(xsc >> 8) * sw1);      // exact
        acc[b] = acc[b] + t0;
        acc[b] = acc[b] + t1;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) acc[b] = acc[b] + __shfl_xor(acc[b], off, 64);
  }
  if (sub == 0 && n < N) {
    const float g = reinterpret_cast<const float*>(ws)[0] * (*g_w);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = (acc[b] * g) * g_d;
      if (YBF16)
        reinterpret_cast<uint16_t*>(y)[(int64_t)b * N + n] = (uint16_t)f32_to_bf16(v);
      else
        reinterpret_cast<float*>(y)[(int64_t)b * N + n] = v;
    }
  }
}

template <int B>
hipError_t launch_gemv_b(const uint8_t* W, const uint8_t* w_scales, const float* g_w, int64_t N,
                         int64_t K, float g_d, const uint8_t* ws, size_t codes_off,
                         size_t scales_off, void* y, bool y_bf16, hipStream_t stream) {
  const int rows_per_wg = 2 * (kThreads / 64);
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
  if (y_bf16)
    hipLaunchKernelGGL((k_gemv<B, true>), grid, dim3(kThreads), 0, stream, W, w_scales, g_w, N, K,
                       g_d, ws, codes_off, scales_off, y);
  else
    hipLaunchKernelGGL((k_gemv<B, false>), grid, dim3(kThreads), 0, stream, W, w_scales, g_w, N, K,
                       g_d, ws, codes_off, scales_off, y);
  return hipGetLastError();
}

}  // namespace

namespace fp4impl {

size_t gemv_workspace_bytes(int64_t B, int64_t K) {
  return kHeader + align16((size_t)(B * K / 2)) + align16((size_t)(B * K / 16));
}

hipError_t launch_gemv(const void* x, bool x_bf16, int64_t B, const uint8_t* W,
                       const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K, float g_d,
                       void* y, bool y_bf16, void* workspace, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t codes_off = kHeader;
  const size_t scales_off = kHeader + align16((size_t)(B * K / 2));
  const int64_t n = B * K;
  const int64_t nblk = n / 16;
  const dim3 g1((unsigned)((nblk + kThreads - 1) / kThreads));
  if (x_bf16)
    hipLaunchKernelGGL(k_gemv_xquant<true>, g1, dim3(kThreads), 0, stream, x, n, ws, codes_off,
                       scales_off);
  else
    hipLaunchKernelGGL(k_gemv_xquant<false>, g1, dim3(kThreads), 0, stream, x, n, ws, codes_off,
                       scales_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define FP4_GEMV_CASE(BB) \
  case BB: return launch_gemv_b<BB>(W, w_scales, g_w, N, K, g_d, ws, codes_off, scales_off, y, y_bf16, stream);
  switch (B) {
    FP4_GEMV_CASE(1) FP4_GEMV_CASE(2) FP4_GEMV_CASE(3) FP4_GEMV_CASE(4)
    FP4_GEMV_CASE(5) FP4_GEMV_CASE(6) FP4_GEMV_CASE(7) FP4_GEMV_CASE(8)
    FP4_GEMV_CASE(9) FP4_GEMV_CASE(10) FP4_GEMV_CASE(11) FP4_GEMV_CASE(12)
    FP4_GEMV_CASE(13) FP4_GEMV_CASE(14) FP4_GEMV_CASE(15) FP4_GEMV_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef FP4_GEMV_CASE
}

}  // namespace fp4impl
