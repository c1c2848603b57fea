// Block-scaled FP4 GEMM  D = g_d * ((g_a s_a . A) @ (g_b s_b . W)^T)  for gfx950.
//
// "NVIDIA NVFP4 与 Micro-Scaling" article, section 三 (scaled GEMM equation) and
// section 五 (A_fp4 [M, K/2] with a_scale [M, K/16]; W [N, K] used as W.t()):
// the block scales are broadcast per block, products of low-precision inputs
// are accumulated in float32, and g_d scales the output.
//
// MXFP4 (E8M0 per 32): the gfx950 block-scaled MFMA consumes exactly this
// format -- v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands and one E8M0
// scale per lane, covering (row, 32-value block).  Each MFMA result is exact
// (FP4 x FP4 x 2^k products are exact and the 64-term sums fit the float32
// accumulator at these exponents); only the float32 accumulation rounds.
//
// NVFP4 (E4M3 per 16): no gfx950 MFMA takes E4M3 block scales, and FP8 cannot
// hold E2M1 x E4M3 products exactly (up to 6 significant bits), so each lane
// dequantizes its operand fragment to fp16 in registers: v_cvt_scalef32_pk_f16_fp4
// applies the scale's power of two (exact), one v_pk_mul_f16 applies its 3-bit
// mantissa (exact: <= 6 significant bits), then v_mfma_f32_32x32x16_f16
// accumulates in float32.  Ceiling: the dense fp16 MFMA rate.
//
// Tiling: 256x256 output tile per workgroup, 4 waves in a 2x2 grid, 128x128 per
// wave (4x4 MFMA tiles of 32x32).  K advances 128 values (64 bytes per row)
// per stage; operand stages are double-buffered in LDS with a 16-byte row pad
// (80-byte row stride keeps the 16-byte fragment reads of 8 consecutive rows on
// distinct banks).  Global loads for stage k+1 are in flight while stage k
// computes.  Inside a 64-value half stage, lane group g = lane/32 owns values
// [32g, 32g+32) of its row, so one 16-byte LDS read feeds the whole half
// (MXFP4: one MFMA; NVFP4: four MFMAs whose K order is permuted identically for
// both operands, which leaves the sum unchanged).
// Workgroup -> tile map: workgroups are dealt round-robin to the 8 XCDs, so
// each XCD is given a contiguous range of tiles; tiles are visited in groups
// of 8 row-tiles so concurrently running workgroups of an XCD share operand
// rows in its L2.
#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 128;   // BK in FP4 values
constexpr int kRowBytes = BK / 2;             // 64
constexpr int kRowStride = kRowBytes + 16;    // 80 (padded)
constexpr int kTileBytes = BM * kRowStride;   // 20480
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

template <bool MX>
struct Cfg {
  static constexpr int kScalesPerRow = MX ? BK / 32 : BK / 16;    // per stage: 4 or 8
  static constexpr int kScaleBytes = BM * kScalesPerRow;
  static constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
};

// ----------------------------------------------------------- tile mapping --
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  int t = bid;
  if (T % kXcds == 0) t = (bid % kXcds) * (T / kXcds) + bid / kXcds;
  const int in_group = kGroupM * tiles_n;
  const int group = t / in_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int r = t - group * in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// ------------------------------------------------------------- stage loads --
template <bool MX>
struct StageRegs {
  u32x4 a[4], w[4];
  uint32_t as[MX ? 1 : 2], ws[MX ? 1 : 2];
};

// Thread t loads 16-byte chunks t + 256 j (j < 4) of each 256x64-byte tile and
// the scale bytes of row t.  Rows past the matrix edge are clamped (their
// results are never stored); chunks past K are zero (value 0).
template <bool MX>
__device__ __forceinline__ void load_stage(StageRegs<MX>& r, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ as,
                                           const uint8_t* __restrict__ W,
                                           const uint8_t* __restrict__ ws, int m0, int n0, int M,
                                           int N, int K, int k0) {
  const int t = threadIdx.x;
  const int64_t rowb = K / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + kThreads * j;
    const int row = c >> 2, ch = c & 3;
    const int kc = k0 + 32 * ch;                 // first value of the chunk
    const int ra = min(m0 + row, M - 1), rw = min(n0 + row, N - 1);
    if (kc < K) {
      r.a[j] = *reinterpret_cast<const u32x4*>(A + (int64_t)ra * rowb + kc / 2);
      r.w[j] = *reinterpret_cast<const u32x4*>(W + (int64_t)rw * rowb + kc / 2);
    } else {
      r.a[j] = u32x4{0, 0, 0, 0};
      r.w[j] = u32x4{0, 0, 0, 0};
    }
  }
  constexpr int bs = MX ? 32 : 16;
  const int nsc = K / bs;
  const int kb = k0 / bs;
  const int ra = min(m0 + t, M - 1), rw = min(n0 + t, N - 1);
  const uint8_t* pa = as + (int64_t)ra * nsc;
  const uint8_t* pw = ws + (int64_t)rw * nsc;
#pragma unroll
  for (int q = 0; q < (MX ? 1 : 2); ++q) {
    uint32_t va = 0, vw = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = kb + 4 * q + i;
      if (b < nsc) {
        va |= (uint32_t)pa[b] << (8 * i);
        vw |= (uint32_t)pw[b] << (8 * i);
      }
    }
    r.as[q] = va;
    r.ws[q] = vw;
  }
}

template <bool MX>
__device__ __forceinline__ void store_stage(const StageRegs<MX>& r, uint8_t* __restrict__ lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + kThreads * j;
    const int row = c >> 2, ch = c & 3;
    *reinterpret_cast<u32x4*>(lds + row * kRowStride + 16 * ch) = r.a[j];
    *reinterpret_cast<u32x4*>(lds + kTileBytes + row * kRowStride + 16 * ch) = r.w[j];
  }
  constexpr int spr = Cfg<MX>::kScalesPerRow;
  uint32_t* sa = reinterpret_cast<uint32_t*>(lds + 2 * kTileBytes);
  uint32_t* sw = reinterpret_cast<uint32_t*>(lds + 2 * kTileBytes + Cfg<MX>::kScaleBytes);
#pragma unroll
  for (int q = 0; q < (MX ? 1 : 2); ++q) {
    sa[t * (spr / 4) + q] = r.as[q];
    sw[t * (spr / 4) + q] = r.ws[q];
  }
}

// --------------------------------------------------------- NV fragment dequant --
// E4M3 byte -> (power of two as f32 for the cvt scale operand, 3-bit mantissa
// factor as an f16 pair).  Normal: 2^(E-7) * (1 + m/8); subnormal: 2^-9 * m.
__device__ __forceinline__ void e4m3_split(uint32_t b, float& pow2, v2h& mant) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  pow2 = __uint_as_float(e ? ((e + 120u) << 23) : (118u << 23));
  const float mf = e ? 1.0f + (float)m * 0.125f : (float)m;
  const _Float16 mh = (_Float16)mf;   // exact
  mant = v2h{mh, mh};
}

// 8 FP4 codes (one dword) -> 8 fp16 values v * scale.
__device__ __forceinline__ v8h dequant8(uint32_t codes, float pow2, v2h mant) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 0) * mant;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 1) * mant;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 2) * mant;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 3) * mant;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// ------------------------------------------------------------------ kernel --
template <bool MX, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads, 1)
    k_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ as,
           const uint8_t* __restrict__ W, const uint8_t* __restrict__ ws,
           const float* __restrict__ g_a, const float* __restrict__ g_b, float g_d, int M, int N,
           int K, void* __restrict__ D, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  StageRegs<MX> st;
  load_stage<MX>(st, A, as, W, ws, m0, n0, M, N, K, 0);
  store_stage<MX>(st, smem);
  __syncthreads();

  constexpr int kStage = Cfg<MX>::kStageBytes;
  constexpr int spr = Cfg<MX>::kScalesPerRow;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_stage<MX>(st, A, as, W, ws, m0, n0, M, N, K, (kt + 1) * BK);
    const uint8_t* buf = smem + (kt & 1) * kStage;
    const uint8_t* la = buf + (wm * 128 + l32) * kRowStride + 16 * g;
    const uint8_t* lw = buf + kTileBytes + (wn * 128 + l32) * kRowStride + 16 * g;
    const uint8_t* lsa = buf + 2 * kTileBytes + (wm * 128 + l32) * spr;
    const uint8_t* lsw = buf + 2 * kTileBytes + Cfg<MX>::kScaleBytes + (wn * 128 + l32) * spr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 fa[4], fw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = *reinterpret_cast<const u32x4*>(la + i * 32 * kRowStride + 32 * h);
        fw[i] = *reinterpret_cast<const u32x4*>(lw + i * 32 * kRowStride + 32 * h);
      }
      if constexpr (MX) {
        uint32_t sa[4], sw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sa[i] = lsa[i * 32 * spr + 2 * h + g];
          sw[i] = lsw[i * 32 * spr + 2 * h + g];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v8i av = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v8i bv = {(int)fw[j].x, (int)fw[j].y, (int)fw[j].z, (int)fw[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, bv, acc[i][j], 4, 4, 0, (int)sa[i], 0, (int)sw[j]);
          }
        }
      } else {
        // lane group g holds values [32g, 32g+32) of this 64-value half: NV
        // blocks 4h+2g (dwords 0,1) and 4h+2g+1 (dwords 2,3)
        float pa[4][2], pw[4][2];
        v2h ma[4][2], mw[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            e4m3_split(lsa[i * 32 * spr + 4 * h + 2 * g + b], pa[i][b], ma[i][b]);
            e4m3_split(lsw[i * 32 * spr + 4 * h + 2 * g + b], pw[i][b], mw[i][b]);
          }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8h da[4], dw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            da[i] = dequant8(fa[i][s], pa[i][s >> 1], ma[i][s >> 1]);
            dw[i] = dequant8(fw[i][s], pw[i][s >> 1], mw[i][s >> 1]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[i], dw[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_stage<MX>(st, smem + ((kt + 1) & 1) * kStage);
    __syncthreads();
  }

  // epilogue: D = acc * ((g_a * g_b) * g_d)
  float alpha = g_d;
  if (!MX) alpha = ((*g_a) * (*g_b)) * g_d;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < M) {
          const float v = acc[i][j][r] * alpha;
          if (OUT_BF16)
            reinterpret_cast<uint16_t*>(D)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16(v);
          else
            reinterpret_cast<float*>(D)[(int64_t)row * N + col] = v;
        }
      }
    }
}

template <bool MX, bool OUT_BF16>
hipError_t launch_t(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K, void* D,
                    hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  constexpr int lds = Cfg<MX>::kLdsBytes;
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<MX, OUT_BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm<MX, OUT_BF16>), dim3(tiles_m * tiles_n), dim3(kThreads), lds, stream,
                     A, as, W, ws, g_a, g_b, g_d, M, N, K, D, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

namespace fp4impl {

hipError_t launch_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales, const float* g_a,
                       const uint8_t* W, const uint8_t* w_scales, const float* g_b, float g_d,
                       int64_t M, int64_t N, int64_t K, void* D, bool d_bf16, hipStream_t stream) {
  if (M > (1 << 30) || N > (1 << 30) || K > (1 << 30)) return hipErrorInvalidValue;
  if (mx) {
    return d_bf16 ? launch_t<true, true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                         (int)K, D, stream)
                  : launch_t<true, false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                          (int)K, D, stream);
  }
  return d_bf16 ? launch_t<false, true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                        (int)K, D, stream)
                : launch_t<false, false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                         (int)K, D, stream);
}

}  // namespace fp4impl
