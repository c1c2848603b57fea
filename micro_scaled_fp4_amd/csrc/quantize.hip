// NVFP4 / MXFP4 quantization and dequantization kernels for gfx950.
//
// Layout: one lane owns one whole scale block (16 values for NVFP4, 32 for
// MXFP4), so the block amax, the scale and the element codes need no cross-lane
// traffic; a wave covers 64 consecutive blocks, i.e. 2 KiB (NV, bf16) of
// contiguous input per pass, read with 128-bit loads, and writes 512 contiguous
// code bytes with 64-bit stores.
//
// The "fast" kernels treat the tensor as one flat run of blocks; they need
// cols to be a multiple of the block and 16-byte aligned pointers.  The
// "generic" kernels take any shape and alignment (partial last blocks, odd
// rows) with scalar accesses.
#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 2048;  // 256 CUs x 8 workgroups, grid-stride beyond

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Workgroup max of a u32 (every thread gets the result).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = umax(r, red[i]);
  __syncthreads();
  return r;
}

// Global amax from the partials of the first pass, or the given static amax.
__device__ __forceinline__ float resolve_amax(const float* amax_in, const uint32_t* partials,
                                              int npart) {
  if (partials == nullptr) return *amax_in;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = umax(m, partials[i]);
  return __uint_as_float(block_max_u32(m));
}

// ------------------------------------------------------------------ amax --
template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_amax(const void* __restrict__ x, int64_t n,
                                                   uint32_t* __restrict__ partials) {
  constexpr int kPer = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int64_t nvec = n / kPer;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m0 = 0, m1 = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = xv[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16) {
          const uint32_t a = w[j] & 0x7fff7fffu;
          m0 = umax(m0, a & 0xffffu);
          m1 = umax(m1, a >> 16);
        } else {
          m0 = umax(m0, w[j] & 0x7fffffffu);
        }
      }
    }
  }
  for (; i < nvec; i += stride) {
    const u32x4 v = xv[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (BF16) {
        const uint32_t a = w[j] & 0x7fff7fffu;
        m0 = umax(m0, a & 0xffffu);
        m1 = umax(m1, a >> 16);
      } else {
        m0 = umax(m0, w[j] & 0x7fffffffu);
      }
    }
  }
  // tail elements (n not a multiple of the vector)
  if (blockIdx.x == 0) {
    for (int64_t t = nvec * kPer + threadIdx.x; t < n; t += kThreads) {
      if (BF16) {
        m0 = umax(m0, (uint32_t)(reinterpret_cast<const uint16_t*>(x)[t] & 0x7fffu));
      } else {
        m0 = umax(m0, reinterpret_cast<const uint32_t*>(x)[t] & 0x7fffffffu);
      }
    }
  }
  uint32_t m = BF16 ? (umax(m0, m1) << 16) : m0;
  m = block_max_u32(m);
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
  m = block_max_u32(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// ------------------------------------------------------------ NV quantize --
// Loads the 16 values of block b as float32.
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

template <int N>
__device__ __forceinline__ float amax_of(const float (&v)[N]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) m = umax(m, __float_as_uint(v[j]) & 0x7fffffffu);
  return __uint_as_float(m);
}

// Packs 8 codes (element 2j low nibble of byte j).
__device__ __forceinline__ uint32_t pack8(const uint32_t (&c)[8]) {
  return c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12) | (c[4] << 16) | (c[5] << 20) |
         (c[6] << 24) | (c[7] << 28);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_nv_quant_fast(const void* __restrict__ x, int64_t nblk, uint8_t* __restrict__ q,
                    uint8_t* __restrict__ scales, const float* __restrict__ amax_in,
                    const uint32_t* __restrict__ partials, int npart, float* __restrict__ amax_out,
                    float* __restrict__ scale_out) {
  const float G = resolve_amax(amax_in, partials, npart);
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) *amax_out = G;
    *scale_out = s_global;
  }
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    float v[16];
    load16<BF16>(x, b, v);
    uint32_t sc;
    float r;
    nv_block_scale(amax_of(v), s_global, sc, r);
    uint32_t c[8], d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c[j] = e2m1_code(v[j] * r);
      d[j] = e2m1_code(v[8 + j] * r);
    }
    reinterpret_cast<u32x2*>(q)[b] = u32x2{pack8(c), pack8(d)};
    scales[b] = (uint8_t)sc;
  }
}

// Any shape / alignment: one thread per (row, block).
template <bool BF16, int BS>
__device__ __forceinline__ float load_elem(const void* x, int64_t idx) {
  if (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[idx] << 16);
  return reinterpret_cast<const float*>(x)[idx];
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_nv_quant_generic(const void* __restrict__ x, int64_t rows, int64_t cols,
                       uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                       const float* __restrict__ amax_in, const uint32_t* __restrict__ partials,
                       int npart, float* __restrict__ amax_out, float* __restrict__ scale_out) {
  const float G = resolve_amax(amax_in, partials, npart);
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) *amax_out = G;
    *scale_out = s_global;
  }
  const int64_t bpr = (cols + 15) / 16, qstride = (cols + 1) / 2;
  const int64_t total = rows * bpr;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t r = t / bpr, j = t - r * bpr;
    const int64_t c0 = j * 16;
    const int len = (int)((cols - c0) < 16 ? (cols - c0) : 16);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = i < len ? load_elem<BF16, 16>(x, r * cols + c0 + i) : 0.0f;
    uint32_t sc;
    float rr;
    nv_block_scale(amax_of(v), s_global, sc, rr);
    uint8_t* qrow = q + r * qstride + c0 / 2;
    for (int i = 0; i < len; i += 2) {
      uint32_t lo = e2m1_code(v[i] * rr);
      uint32_t hi = (i + 1 < len) ? e2m1_code(v[i + 1] * rr) : 0u;
      qrow[i / 2] = (uint8_t)(lo | (hi << 4));
    }
    scales[r * bpr + j] = (uint8_t)sc;
  }
}

// ------------------------------------------------------------ MX quantize --
template <bool BF16>
__device__ __forceinline__ void load32(const void* __restrict__ x, int64_t b, float (&v)[32]) {
  if (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x) + 4 * b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 a = p[k];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = bf16_lo(w[j]);
        v[8 * k + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(x) + 8 * b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 a = p[j];
      v[4 * j] = a.x;
      v[4 * j + 1] = a.y;
      v[4 * j + 2] = a.z;
      v[4 * j + 3] = a.w;
    }
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_mx_quant_fast(const void* __restrict__ x, int64_t nblk, uint8_t* __restrict__ q,
                    uint8_t* __restrict__ scales) {
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    float v[32];
    load32<BF16>(x, b, v);
    const uint32_t sc = e8m0_code(__float_as_uint(amax_of(v)));
    const float inv = e8m0_inv(sc);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = e2m1_code(v[8 * k + j] * inv);
      w[k] = pack8(c);
    }
    reinterpret_cast<u32x4*>(q)[b] = u32x4{w[0], w[1], w[2], w[3]};
    scales[b] = (uint8_t)sc;
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
    for (int i = 0; i < 32; ++i) v[i] = i < len ? load_elem<BF16, 32>(x, r * cols + c0 + i) : 0.0f;
    const uint32_t sc = e8m0_code(__float_as_uint(amax_of(v)));
    const float inv = e8m0_inv(sc);
    uint8_t* qrow = q + r * qstride + c0 / 2;
    for (int i = 0; i < len; i += 2) {
      uint32_t lo = e2m1_code(v[i] * inv);
      uint32_t hi = (i + 1 < len) ? e2m1_code(v[i + 1] * inv) : 0u;
      qrow[i / 2] = (uint8_t)(lo | (hi << 4));
    }
    scales[r * bpr + j] = (uint8_t)sc;
  }
}

// ------------------------------------------------------------- dequantize --
template <bool BF16OUT, int N>
__device__ __forceinline__ void store_vals(void* __restrict__ y, int64_t b, const float (&v)[N]) {
  if (BF16OUT) {
    u32x4* p = reinterpret_cast<u32x4*>(y) + (N / 8) * b;
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f32_to_bf16(v[8 * k + 2 * j]) | (f32_to_bf16(v[8 * k + 2 * j + 1]) << 16);
      p[k] = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(y) + (N / 4) * b;
#pragma unroll
    for (int k = 0; k < N / 4; ++k)
      p[k] = f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
  }
}

template <bool BF16OUT>
__global__ void __launch_bounds__(kThreads)
    k_nv_dequant_fast(const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
                      const float* __restrict__ global_scale, int64_t nblk, void* __restrict__ y) {
  const float s_global = *global_scale;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    const u32x2 c = reinterpret_cast<const u32x2*>(q)[b];
    const float sb = s_global * e4m3_value(scales[b]);
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = sb * e2m1_value((c.x >> (4 * j)) & 15u);
      v[8 + j] = sb * e2m1_value((c.y >> (4 * j)) & 15u);
    }
    store_vals<BF16OUT, 16>(y, b, v);
  }
}

template <bool BF16OUT>
__global__ void __launch_bounds__(kThreads)
    k_mx_dequant_fast(const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
                      int64_t nblk, void* __restrict__ y) {
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    const u32x4 c = reinterpret_cast<const u32x4*>(q)[b];
    const float s = e8m0_value(scales[b]);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * k + j] = e2m1_value((w[k] >> (4 * j)) & 15u) * s;
    store_vals<BF16OUT, 32>(y, b, v);
  }
}

template <bool BF16OUT>
__global__ void __launch_bounds__(kThreads)
    k_dequant_generic(bool mx, const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
                      const float* __restrict__ global_scale, int64_t rows, int64_t cols,
                      void* __restrict__ y) {
  const int bs = mx ? 32 : 16;
  const float s_global = mx ? 1.0f : *global_scale;
  const int64_t bpr = (cols + bs - 1) / bs, qstride = (cols + 1) / 2;
  const int64_t total = rows * cols;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t r = t / cols, c = t - r * cols;
    const uint32_t byte = q[r * qstride + c / 2];
    const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
    const uint32_t sb = scales[r * bpr + c / bs];
    const float v = mx ? e2m1_value(code) * e8m0_value(sb) : (s_global * e4m3_value(sb)) * e2m1_value(code);
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

inline int grid_for(int64_t work_items) {
  int64_t g = (work_items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (int)(g < kMaxGrid ? g : kMaxGrid);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

namespace fp4impl {

hipError_t launch_amax(const void* x, bool bf16, int64_t n, uint32_t* partials, int* npart,
                       hipStream_t stream) {
  const int per = bf16 ? 8 : 4;
  int64_t nvec = n / per;
  // 4 vectors in flight per thread on the unrolled path
  int g = grid_for((nvec + 3) / 4);
  if (g > kAmaxPartials) g = kAmaxPartials;
  *npart = g;
  if (aligned16(x)) {
    if (bf16)
      hipLaunchKernelGGL(k_amax<true>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
    else
      hipLaunchKernelGGL(k_amax<false>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
  } else {
    if (bf16)
      hipLaunchKernelGGL(k_amax_scalar<true>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
    else
      hipLaunchKernelGGL(k_amax_scalar<false>, dim3(g), dim3(kThreads), 0, stream, x, n, partials);
  }
  return hipGetLastError();
}

hipError_t launch_nv_quant(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* q,
                           uint8_t* scales, const float* amax_in, const uint32_t* partials,
                           int npart, float* amax_out, float* scale_out, hipStream_t stream) {
  const bool fast = (cols % 16 == 0) && aligned16(x) && aligned16(q);
  if (fast) {
    const int64_t nblk = rows * (cols / 16);
    const int g = grid_for(nblk);
    if (bf16)
      hipLaunchKernelGGL(k_nv_quant_fast<true>, dim3(g), dim3(kThreads), 0, stream, x, nblk, q,
                         scales, amax_in, partials, npart, amax_out, scale_out);
    else
      hipLaunchKernelGGL(k_nv_quant_fast<false>, dim3(g), dim3(kThreads), 0, stream, x, nblk, q,
                         scales, amax_in, partials, npart, amax_out, scale_out);
  } else {
    const int g = grid_for(rows * ((cols + 15) / 16));
    if (bf16)
      hipLaunchKernelGGL(k_nv_quant_generic<true>, dim3(g), dim3(kThreads), 0, stream, x, rows,
                         cols, q, scales, amax_in, partials, npart, amax_out, scale_out);
    else
      hipLaunchKernelGGL(k_nv_quant_generic<false>, dim3(g), dim3(kThreads), 0, stream, x, rows,
                         cols, q, scales, amax_in, partials, npart, amax_out, scale_out);
  }
  return hipGetLastError();
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
                          bool bf16_out, hipStream_t stream) {
  const int bs = mx ? 32 : 16;
  const bool fast = (cols % bs == 0) && aligned16(q) && aligned16(y);
  if (fast) {
    const int64_t nblk = rows * (cols / bs);
    const int g = grid_for(nblk);
    if (mx) {
      if (bf16_out)
        hipLaunchKernelGGL(k_mx_dequant_fast<true>, dim3(g), dim3(kThreads), 0, stream, q, scales,
                           nblk, y);
      else
        hipLaunchKernelGGL(k_mx_dequant_fast<false>, dim3(g), dim3(kThreads), 0, stream, q,
                           scales, nblk, y);
    } else {
      if (bf16_out)
        hipLaunchKernelGGL(k_nv_dequant_fast<true>, dim3(g), dim3(kThreads), 0, stream, q, scales,
                           global_scale, nblk, y);
      else
        hipLaunchKernelGGL(k_nv_dequant_fast<false>, dim3(g), dim3(kThreads), 0, stream, q,
                           scales, global_scale, nblk, y);
    }
  } else {
    const int g = grid_for(rows * cols);
    if (bf16_out)
      hipLaunchKernelGGL(k_dequant_generic<true>, dim3(g), dim3(kThreads), 0, stream, mx, q,
                         scales, global_scale, rows, cols, y);
    else
      hipLaunchKernelGGL(k_dequant_generic<false>, dim3(g), dim3(kThreads), 0, stream, mx, q,
                         scales, global_scale, rows, cols, y);
  }
  return hipGetLastError();
}

hipError_t launch_empty_scales(float* amax_out, float* scale_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_empty_scales, dim3(1), dim3(64), 0, stream, amax_out, scale_out);
  return hipGetLastError();
}

}  // namespace fp4impl
