// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
// Every launcher enqueues on `stream`, never synchronizes and returns the HIP
// status of its launches.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace fp4impl {

// Raises kernel fn's dynamic-LDS limit to `bytes` on the current device, once
// per device: `done` is the caller's set of devices (bit d for device d < 64)
// on which that kernel's limit is already set.  Thread-safe: two first calls
// racing may both set the attribute, which is idempotent, and a device bit is
// published only after its attribute call succeeded.  Devices >= 64 set it on
// every call.
inline hipError_t set_lds_limit_once(std::atomic<uint64_t>& done, const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Compute units of the current device, looked up once per device (devices
// >= 64: on every call), so calls on devices of different sizes (compute
// partitions) each see their own count.
inline int num_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int cus = 0;
  const int n = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                        cus > 0
                    ? cus
                    : 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

constexpr int kAmaxPartials = 1024;  // FP4_AMAX_WORKSPACE_BYTES / 4

// ---- quantize.hip ---------------------------------------------------------
// Per-workgroup partial max|x| (float bit patterns) of n elements; writes
// *npart <= kAmaxPartials entries of partials.
hipError_t launch_amax(const void* x, bool bf16, int64_t n, uint32_t* partials, int* npart,
                       hipStream_t stream);

// Device address, on the current device, of the library's own array of
// kAmaxPartials partial maxima (looked up once per device, then cached).
hipError_t amax_scratch(uint32_t** out);

// NVFP4 quantize.  Exactly one of (amax_in) or (partials, npart) gives G.
// block: 8, 16 or 32 values per E4M3 scale; window > 0: the scale byte is
// searched over +-window codes around the amax rule's (least squared error).
hipError_t launch_nv_quant(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* q,
                           uint8_t* scales, const float* amax_in, const uint32_t* partials,
                           int npart, float* amax_out, float* scale_out, hipStream_t stream,
                           int block = 16, int window = 0);

hipError_t launch_mx_quant(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* q,
                           uint8_t* scales, hipStream_t stream);

// block: NVFP4 values per scale (8, 16, 32); MXFP4 always 32.
hipError_t launch_dequant(bool mx, const uint8_t* q, const uint8_t* scales,
                          const float* global_scale, int64_t rows, int64_t cols, void* y,
                          bool bf16_out, hipStream_t stream, int block = 16);

// Writes G = 0 and s_global = 1 (empty tensors).
hipError_t launch_empty_scales(float* amax_out, float* scale_out, hipStream_t stream);

// ---- hadamard.hip ---------------------------------------------------------
hipError_t launch_hadamard_amax(const void* x, bool bf16, int64_t rows, int64_t cols,
                                uint32_t* partials, int* npart, hipStream_t stream);
hipError_t launch_hadamard_quant(const void* x, bool bf16, int64_t rows, int64_t cols, bool sr,
                                 uint64_t seed, uint8_t* q, uint8_t* scales, const float* amax_in,
                                 const uint32_t* partials, int npart, float* amax_out,
                                 float* scale_out, hipStream_t stream);

// y = x H per 128-channel group, float32 or bf16 (cols % 128 == 0, 16-byte aligned).
hipError_t launch_hadamard_rotate(const void* x, bool bf16, int64_t rows, int64_t cols, void* y,
                                  bool y_bf16, hipStream_t stream);
// x H per 128-channel group, then MXFP4 (one pass; RNE or stochastic codes).
hipError_t launch_hadamard_quant_mx(const void* x, bool bf16, int64_t rows, int64_t cols, bool sr,
                                    uint64_t seed, uint8_t* q, uint8_t* scales,
                                    hipStream_t stream);

// ---- gemv.hip -------------------------------------------------------------
// Writes n zeros of elem_bytes (4: float, 2: bf16, 1: E4M3) each to y: the result
// of a contraction over K = 0.
hipError_t launch_zero_fill(void* y, int64_t n, int elem_bytes, hipStream_t stream);
size_t gemv_workspace_bytes(int64_t B, int64_t K);
hipError_t launch_gemv(const void* x, bool x_bf16, int64_t B, const uint8_t* W,
                       const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K, float g_d,
                       void* y, bool y_bf16, void* workspace, hipStream_t stream);

// ---- gemm.hip -------------------------------------------------------------
hipError_t launch_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales, const float* g_a,
                       const uint8_t* W, const uint8_t* w_scales, const float* g_b, float g_d,
                       int64_t M, int64_t N, int64_t K, void* D, int d_bytes, hipStream_t stream);
// The same GEMM with d_bytes = 0: D receives NVFP4 codes [M, ceil(N/2)] and
// d_scales the E4M3 bytes [M, ceil(N/16)] of fl(acc * alpha), quantized at the
// given tensor amax *d_amax; *d_gscale receives its s_global.
hipError_t launch_gemm_nvfp4_out(bool mx, const uint8_t* A, const uint8_t* a_scales,
                                 const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                                 const float* g_b, float g_d, int64_t M, int64_t N, int64_t K,
                                 void* D, int d_bytes, uint8_t* d_scales, const float* d_amax,
                                 float* d_gscale, hipStream_t stream);
// One launch over ngroups GEMMs: group e multiplies rows offsets[e] ..
// offsets[e+1] of A (and writes those rows of D) by W + e N K/2 with tensor
// scale g_b[e] (NVFP4).  d_bytes 4 / 2 / 1 (float32, bf16, E4M3).
hipError_t launch_grouped_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales,
                               const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                               const float* g_b, float g_d, int64_t ngroups,
                               const int32_t* offsets, int64_t M, int64_t N, int64_t K, void* D,
                               int d_bytes, hipStream_t stream);
// *out = s_global of the tensor amax *amax (one thread).
hipError_t launch_nv_global_scale(const float* amax, float* out, hipStream_t stream);

}  // namespace fp4impl
