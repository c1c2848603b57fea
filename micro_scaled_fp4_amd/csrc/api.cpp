// C-ABI entry points of libfp4.so: host-side argument checks, the gfx950 check
// and dispatch to the kernel launchers.  Nothing here allocates device memory
// or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "fp4.h"
#include "fp4_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

fp4_status hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s", where, hipGetErrorString(e));
  return FP4_ERR_HIP;
}

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

fp4_status check_arch() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return FP4_ERR_ARCH;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? FP4_OK : FP4_ERR_ARCH;
}

bool valid_dtype(fp4_dtype t) { return t == FP4_F32 || t == FP4_BF16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

#define FP4_TRY_LAUNCH(expr, where)            \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// Shared front half of the NVFP4-producing calls.
fp4_status check_quant_args(const void* x, fp4_dtype xt, int64_t rows, int64_t cols,
                            const uint8_t* q, const uint8_t* scales, const float* global_amax,
                            int amax_given, const float* global_scale, const void* workspace,
                            size_t workspace_bytes) {
  if (!valid_dtype(xt)) return FP4_ERR_DTYPE;
  if (rows < 0 || cols < 0) return FP4_ERR_SHAPE;
  if (global_scale == nullptr) return FP4_ERR_NULL;
  if (amax_given && global_amax == nullptr) return FP4_ERR_NULL;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (x == nullptr || q == nullptr || scales == nullptr) return FP4_ERR_NULL;
  if (!amax_given) {
    if (workspace == nullptr || workspace_bytes < FP4_AMAX_WORKSPACE_BYTES) return FP4_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP4_ERR_ALIGN;
  }
  if (!aligned(x, xt == FP4_BF16 ? 2 : 4) || !aligned(global_scale, 4) ||
      (global_amax && !aligned(global_amax, 4)))
    return FP4_ERR_ALIGN;
  return FP4_OK;
}

fp4_status dequantize_blocks(fp4_format fmt, int block, const uint8_t* q,
                                    const uint8_t* scales, const float* global_scale, int64_t rows,
                                    int64_t cols, void* y, fp4_dtype yt, hipStream_t stream) {
  if (fmt != FP4_NVFP4 && fmt != FP4_MXFP4) return FP4_ERR_DTYPE;
  if (!valid_dtype(yt)) return FP4_ERR_DTYPE;
  if (rows < 0 || cols < 0) return FP4_ERR_SHAPE;
  if (fmt == FP4_MXFP4 && global_scale != nullptr) return FP4_ERR_DTYPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (q == nullptr || scales == nullptr || y == nullptr) return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && global_scale == nullptr) return FP4_ERR_NULL;
  if (!aligned(y, yt == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_dequant(fmt == FP4_MXFP4, q, scales, global_scale, rows, cols, y,
                                         yt == FP4_BF16, stream, block),
                 "fp4_dequantize");
  return FP4_OK;
}

}  // namespace

extern "C" {

const char* fp4_status_string(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_SHAPE: return "invalid shape";
    case FP4_ERR_DTYPE: return "invalid dtype, format or rounding mode";
    case FP4_ERR_ALIGN: return "pointer misaligned";
    case FP4_ERR_ARCH: return "current device is not gfx950 (MI355X)";
    case FP4_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4_ERR_HIP: return "HIP runtime error";
    case FP4_ERR_ALIAS: return "an output aliases an input it must not alias";
  }
  return "unknown status";
}

const char* fp4_last_hip_error(void) { return g_last_hip_error; }

fp4_status nvfp4_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* scales, float* global_amax, int amax_given, float* global_scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return nvfp4_quantize_ex(x, xt, rows, cols, 16, 0, q, scales, global_amax, amax_given,
                           global_scale, workspace, workspace_bytes, stream);
}

fp4_status nvfp4_quantize_ex(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int block,
                             int scale_search, uint8_t* q, uint8_t* scales, float* global_amax,
                             int amax_given, float* global_scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (block != 8 && block != 16 && block != 32) return FP4_ERR_SHAPE;
  if (scale_search < 0 || scale_search > FP4_MAX_SCALE_SEARCH) return FP4_ERR_SHAPE;
  fp4_status st = check_quant_args(x, xt, rows, cols, q, scales, global_amax, amax_given,
                                   global_scale, workspace, workspace_bytes);
  if (st != FP4_OK) return st;
  if ((st = check_arch()) != FP4_OK) return st;
  const bool bf16 = xt == FP4_BF16;
  if (rows == 0 || cols == 0) {
    FP4_TRY_LAUNCH(fp4impl::launch_empty_scales(amax_given ? nullptr : global_amax, global_scale,
                                                stream),
                   "nvfp4_quantize");
    return FP4_OK;
  }
  uint32_t* partials = nullptr;
  int npart = 0;
  if (!amax_given) {
    partials = static_cast<uint32_t*>(workspace);
    FP4_TRY_LAUNCH(fp4impl::launch_amax(x, bf16, rows * cols, partials, &npart, stream),
                   "nvfp4_quantize/amax");
  }
  FP4_TRY_LAUNCH(fp4impl::launch_nv_quant(x, bf16, rows, cols, q, scales,
                                          amax_given ? global_amax : nullptr, partials, npart,
                                          amax_given ? nullptr : global_amax, global_scale, stream,
                                          block, scale_search),
                 "nvfp4_quantize/encode");
  return FP4_OK;
}

fp4_status nvfp4_quantize_no_workspace(const void* x, fp4_dtype xt, int64_t rows, int64_t cols,
                                       uint8_t* q, uint8_t* scales, float* global_amax,
                                       int amax_given, float* global_scale, hipStream_t stream) {
  // the same checks as nvfp4_quantize, with a stand-in for the workspace it
  // does not take (never dereferenced: the library's scratch replaces it)
  fp4_status st = check_quant_args(x, xt, rows, cols, q, scales, global_amax, amax_given,
                                   global_scale, reinterpret_cast<const void*>(FP4_AMAX_WORKSPACE_BYTES),
                                   FP4_AMAX_WORKSPACE_BYTES);
  if (st != FP4_OK) return st;
  if ((st = check_arch()) != FP4_OK) return st;
  const bool bf16 = xt == FP4_BF16;
  if (rows == 0 || cols == 0) {
    FP4_TRY_LAUNCH(fp4impl::launch_empty_scales(amax_given ? nullptr : global_amax, global_scale,
                                                stream),
                   "nvfp4_quantize_no_workspace");
    return FP4_OK;
  }
  uint32_t* partials = nullptr;
  int npart = 0;
  if (!amax_given) {
    FP4_TRY_LAUNCH(fp4impl::amax_scratch(&partials), "nvfp4_quantize_no_workspace/scratch");
    // the amax pass never uses more than kAmaxPartials workgroups, so every
    // size fits the scratch; the first pass writes every partial the second reads
    FP4_TRY_LAUNCH(fp4impl::launch_amax(x, bf16, rows * cols, partials, &npart, stream),
                   "nvfp4_quantize_no_workspace/amax");
  }
  FP4_TRY_LAUNCH(fp4impl::launch_nv_quant(x, bf16, rows, cols, q, scales,
                                          amax_given ? global_amax : nullptr, partials, npart,
                                          amax_given ? nullptr : global_amax, global_scale, stream),
                 "nvfp4_quantize_no_workspace/encode");
  return FP4_OK;
}

fp4_status mxfp4_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* scales, hipStream_t stream) {
  if (!valid_dtype(xt)) return FP4_ERR_DTYPE;
  if (rows < 0 || cols < 0) return FP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (x == nullptr || q == nullptr || scales == nullptr) return FP4_ERR_NULL;
  if (!aligned(x, xt == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_mx_quant(x, xt == FP4_BF16, rows, cols, q, scales, stream),
                 "mxfp4_quantize");
  return FP4_OK;
}

fp4_status fp4_dequantize(fp4_format fmt, const uint8_t* q, const uint8_t* scales,
                          const float* global_scale, int64_t rows, int64_t cols, void* y,
                          fp4_dtype yt, hipStream_t stream) {
  return dequantize_blocks(fmt, 16, q, scales, global_scale, rows, cols, y, yt, stream);
}

fp4_status nvfp4_dequantize_ex(const uint8_t* q, const uint8_t* scales, const float* global_scale,
                               int64_t rows, int64_t cols, int block, void* y, fp4_dtype yt,
                               hipStream_t stream) {
  if (block != 8 && block != 16 && block != 32) return FP4_ERR_SHAPE;
  return dequantize_blocks(FP4_NVFP4, block, q, scales, global_scale, rows, cols, y, yt, stream);
}


fp4_status fp4_scaled_gemm(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                           const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                           const float* g_b, float g_d, int64_t M, int64_t N, int64_t K, void* D,
                           fp4_dtype dt, hipStream_t stream) {
  if (fmt != FP4_NVFP4 && fmt != FP4_MXFP4) return FP4_ERR_DTYPE;
  if (!valid_dtype(dt) && dt != FP4_E4M3) return FP4_ERR_DTYPE;
  const int d_bytes = dt == FP4_F32 ? 4 : dt == FP4_BF16 ? 2 : 1;
  if (M < 0 || N < 0 || K < 0) return FP4_ERR_SHAPE;
  if (K % 32 != 0) return FP4_ERR_SHAPE;
  if (M > FP4_GEMM_MAX_MN || N > FP4_GEMM_MAX_MN || K > FP4_GEMM_MAX_K) return FP4_ERR_SHAPE;
  if (fmt == FP4_MXFP4 && (g_a != nullptr || g_b != nullptr)) return FP4_ERR_DTYPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (K == 0) {   // empty contraction: D = 0, operands are not read
    if (D == nullptr) return FP4_ERR_NULL;
    if (!aligned(D, d_bytes)) return FP4_ERR_ALIGN;
    fp4_status st = check_arch();
    if (st != FP4_OK) return st;
    FP4_TRY_LAUNCH(fp4impl::launch_zero_fill(D, M * N, d_bytes, stream), "fp4_scaled_gemm");
    return FP4_OK;
  }
  if (A == nullptr || a_scales == nullptr || W == nullptr || w_scales == nullptr || D == nullptr)
    return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && (g_a == nullptr || g_b == nullptr)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(W, 16) || !aligned(D, d_bytes)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_gemm(fmt == FP4_MXFP4, A, a_scales, g_a, W, w_scales, g_b, g_d, M,
                                      N, K, D, d_bytes, stream),
                 "fp4_scaled_gemm");
  return FP4_OK;
}

fp4_status fp4_scaled_gemm_nvfp4_out(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                                     const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                                     const float* g_b, float g_d, int64_t M, int64_t N, int64_t K,
                                     uint8_t* Dq, uint8_t* d_scales, const float* d_amax,
                                     float* d_global_scale, hipStream_t stream) {
  if (fmt != FP4_NVFP4 && fmt != FP4_MXFP4) return FP4_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return FP4_ERR_SHAPE;
  if (K % 32 != 0) return FP4_ERR_SHAPE;
  if (M > FP4_GEMM_MAX_MN || N > FP4_GEMM_MAX_MN || K > FP4_GEMM_MAX_K) return FP4_ERR_SHAPE;
  if (fmt == FP4_MXFP4 && (g_a != nullptr || g_b != nullptr)) return FP4_ERR_DTYPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (Dq == nullptr || d_scales == nullptr || d_amax == nullptr || d_global_scale == nullptr)
    return FP4_ERR_NULL;
  if (!aligned(d_amax, 4) || !aligned(d_global_scale, 4)) return FP4_ERR_ALIGN;
  // workgroup 0 writes *d_global_scale while the others still read *d_amax
  if (static_cast<const void*>(d_amax) == static_cast<const void*>(d_global_scale))
    return FP4_ERR_ALIAS;
  if (K == 0) {   // empty contraction: D = 0 encodes as codes 0 and scale bytes 0
    fp4_status st = check_arch();
    if (st != FP4_OK) return st;
    FP4_TRY_LAUNCH(fp4impl::launch_zero_fill(Dq, M * ((N + 1) / 2), 1, stream), "fp4_scaled_gemm_nvfp4_out");
    FP4_TRY_LAUNCH(fp4impl::launch_zero_fill(d_scales, M * ((N + 15) / 16), 1, stream),
                   "fp4_scaled_gemm_nvfp4_out");
    FP4_TRY_LAUNCH(fp4impl::launch_nv_global_scale(d_amax, d_global_scale, stream),
                   "fp4_scaled_gemm_nvfp4_out");
    return FP4_OK;
  }
  if (A == nullptr || a_scales == nullptr || W == nullptr || w_scales == nullptr) return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && (g_a == nullptr || g_b == nullptr)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(W, 16)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_gemm_nvfp4_out(fmt == FP4_MXFP4, A, a_scales, g_a, W, w_scales, g_b,
                                                g_d, M, N, K, Dq, 0, d_scales, d_amax,
                                                d_global_scale, stream),
                 "fp4_scaled_gemm_nvfp4_out");
  return FP4_OK;
}

fp4_status fp4_grouped_gemm(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                            const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                            const float* g_b, float g_d, int64_t num_groups,
                            const int32_t* offsets, int64_t M_total, int64_t N, int64_t K,
                            void* D, fp4_dtype dt, hipStream_t stream) {
  if (fmt != FP4_NVFP4 && fmt != FP4_MXFP4) return FP4_ERR_DTYPE;
  if (!valid_dtype(dt) && dt != FP4_E4M3) return FP4_ERR_DTYPE;
  const int d_bytes = dt == FP4_F32 ? 4 : dt == FP4_BF16 ? 2 : 1;
  if (num_groups < 1 || M_total < 0 || N < 0 || K < 0 || K % 32 != 0) return FP4_ERR_SHAPE;
  if (M_total > FP4_GEMM_MAX_MN || N > FP4_GEMM_MAX_MN || K > FP4_GEMM_MAX_K ||
      num_groups > FP4_GROUPED_MAX_GROUPS)
    return FP4_ERR_SHAPE;
  if (((M_total + 255) / 256 + num_groups) * ((N + 255) / 256) >= (int64_t)1 << 31) return FP4_ERR_SHAPE;
  if (fmt == FP4_MXFP4 && (g_a != nullptr || g_b != nullptr)) return FP4_ERR_DTYPE;
  if (M_total == 0 || N == 0) return FP4_OK;
  if (D == nullptr) return FP4_ERR_NULL;
  if (!aligned(D, d_bytes)) return FP4_ERR_ALIGN;
  if (K == 0) {   // every group's contraction is empty: D = 0
    fp4_status st = check_arch();
    if (st != FP4_OK) return st;
    FP4_TRY_LAUNCH(fp4impl::launch_zero_fill(D, M_total * N, d_bytes, stream), "fp4_grouped_gemm");
    return FP4_OK;
  }
  if (A == nullptr || a_scales == nullptr || W == nullptr || w_scales == nullptr ||
      offsets == nullptr)
    return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && (g_a == nullptr || g_b == nullptr)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(W, 16) || !aligned(offsets, 4)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_grouped_gemm(fmt == FP4_MXFP4, A, a_scales, g_a, W, w_scales, g_b,
                                              g_d, num_groups, offsets, M_total, N, K, D, d_bytes,
                                              stream),
                 "fp4_grouped_gemm");
  return FP4_OK;
}

size_t fp4_gemv_workspace_bytes(int64_t B, int64_t K) {
  if (B < 0 || K < 0) return 0;
  return fp4impl::gemv_workspace_bytes(B, K);
}

fp4_status fp4_gemv_batched(const void* x, fp4_dtype xt, int64_t B, const uint8_t* W,
                            const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K,
                            float g_d, void* y, fp4_dtype yt, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(xt) || !valid_dtype(yt)) return FP4_ERR_DTYPE;
  if (B < 1 || B > 16 || N < 0 || K < 0 || K % 32 != 0) return FP4_ERR_SHAPE;
  if (N > FP4_GEMV_MAX_N || K > FP4_GEMV_MAX_K) return FP4_ERR_SHAPE;
  if (N == 0) return FP4_OK;
  if (K == 0) {   // empty contraction: y = 0, x, W and the workspace are not read
    if (y == nullptr) return FP4_ERR_NULL;
    if (!aligned(y, yt == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
    fp4_status st = check_arch();
    if (st != FP4_OK) return st;
    FP4_TRY_LAUNCH(fp4impl::launch_zero_fill(y, B * N, yt == FP4_BF16 ? 2 : 4, stream), "fp4_gemv_batched");
    return FP4_OK;
  }
  if (x == nullptr || W == nullptr || w_scales == nullptr || g_w == nullptr || y == nullptr)
    return FP4_ERR_NULL;
  if (workspace == nullptr || workspace_bytes < fp4impl::gemv_workspace_bytes(B, K))
    return FP4_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(w_scales, 2) ||
      !aligned(y, yt == FP4_BF16 ? 2 : 4))
    return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_gemv(x, xt == FP4_BF16, B, W, w_scales, g_w, N, K, g_d, y,
                                      yt == FP4_BF16, workspace, stream),
                 "fp4_gemv_batched");
  return FP4_OK;
}

fp4_status hadamard_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                             fp4_rounding mode, uint64_t seed, uint8_t* q, uint8_t* scales,
                             float* global_amax, int amax_given, float* global_scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (mode != FP4_RNE && mode != FP4_SR) return FP4_ERR_DTYPE;
  if (group != 128) return FP4_ERR_SHAPE;
  if (cols % group != 0) return FP4_ERR_SHAPE;
  fp4_status st = check_quant_args(x, xt, rows, cols, q, scales, global_amax, amax_given,
                                   global_scale, workspace, workspace_bytes);
  if (st != FP4_OK) return st;
  if (rows != 0 && cols != 0 && (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 2)))
    return FP4_ERR_ALIGN;
  if ((st = check_arch()) != FP4_OK) return st;
  const bool bf16 = xt == FP4_BF16;
  if (rows == 0 || cols == 0) {
    FP4_TRY_LAUNCH(fp4impl::launch_empty_scales(amax_given ? nullptr : global_amax, global_scale,
                                                stream),
                   "hadamard_quantize");
    return FP4_OK;
  }
  uint32_t* partials = nullptr;
  int npart = 0;
  if (!amax_given) {
    partials = static_cast<uint32_t*>(workspace);
    FP4_TRY_LAUNCH(fp4impl::launch_hadamard_amax(x, bf16, rows, cols, partials, &npart, stream),
                   "hadamard_quantize/amax");
  }
  FP4_TRY_LAUNCH(fp4impl::launch_hadamard_quant(x, bf16, rows, cols, mode == FP4_SR, seed, q,
                                                scales, amax_given ? global_amax : nullptr,
                                                partials, npart,
                                                amax_given ? nullptr : global_amax, global_scale,
                                                stream),
                 "hadamard_quantize/encode");
  return FP4_OK;
}

fp4_status hadamard_quantize_mx(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                                fp4_rounding mode, uint64_t seed, uint8_t* q, uint8_t* scales,
                                hipStream_t stream) {
  if (!valid_dtype(xt)) return FP4_ERR_DTYPE;
  if (mode != FP4_RNE && mode != FP4_SR) return FP4_ERR_DTYPE;
  if (group != 128 || rows < 0 || cols < 0 || cols % group != 0) return FP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (x == nullptr || q == nullptr || scales == nullptr) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_hadamard_quant_mx(x, xt == FP4_BF16, rows, cols, mode == FP4_SR,
                                                   seed, q, scales, stream),
                 "hadamard_quantize_mx");
  return FP4_OK;
}

fp4_status hadamard_rotate(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                           void* y, fp4_dtype yt, hipStream_t stream) {
  if (!valid_dtype(xt) || !valid_dtype(yt)) return FP4_ERR_DTYPE;
  if (group != 128 || rows < 0 || cols < 0 || cols % group != 0) return FP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (x == nullptr || y == nullptr) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return FP4_ERR_ALIGN;
  fp4_status st = check_arch();
  if (st != FP4_OK) return st;
  FP4_TRY_LAUNCH(fp4impl::launch_hadamard_rotate(x, xt == FP4_BF16, rows, cols, y, yt == FP4_BF16,
                                                 stream),
                 "hadamard_rotate");
  return FP4_OK;
}

}  // extern "C"
