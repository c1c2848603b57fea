// Block-scaled FP4 GEMM  D = g_d * ((g_a s_a . A) @ (g_b s_b . W)^T)  for gfx950.
//
// "NVIDIA NVFP4 与 Micro-Scaling" article, section 三 (scaled GEMM equation) and
// section 五 (A_fp4 [M, K/2] with a_scale [M, K/16]; W [N, K] used as W.t()):
// the block scales are broadcast per block, products of low-precision inputs
// are accumulated in float32, and g_d scales the output.
//
// MXFP4 (E8M0 per 32): the gfx950 block-scaled MFMA consumes exactly this
// format -- v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands and one E8M0
// scale byte per lane, covering (row, 32-value block), chosen from a scale
// dword by the instruction's byte select.  Each MFMA result is exact (FP4 x
// FP4 x 2^k products are exact and the 128-term sums fit the float32
// accumulator at these exponents); only the float32 accumulation rounds.
//
// NVFP4 (E4M3 per 16): no gfx950 MFMA takes E4M3 block scales, and FP8 cannot
// hold E2M1 x E4M3 products exactly (up to 6 significant bits), so each lane
// dequantizes its operand fragment to fp16 in registers:
// v_cvt_scalef32_pk_f16_fp4 with the constant scale 2^8, times the E4M3 scale
// byte moved into fp16 fields (= E4M3 * 2^-8), both exact; then
// v_mfma_f32_16x16x32_f16 accumulates in float32.  Ceiling: the fp16 MFMA rate.
//
// Tiling: BM x BN (256 x 256) output tile per workgroup, 2 x 2 waves, each with
// its own 8 x 8 block of 16x16 MFMA tiles (accumulators in AGPRs).  K advances 256 values
// (128 bytes per row) per stage; stages are double-buffered in LDS through
// registers (the next stage's global loads are in flight while this stage
// computes; one barrier per stage).  A 16-byte chunk c of tile row r is stored
// at chunk position c ^ ((r >> 1) & 7): the 16 rows of a fragment read then
// cover all 64 banks.  Inside a stage, lane group g (lane / 16) takes values
// [64g + 32ks, +32) in k-step ks, identically for both operands (the MFMA sum
// does not depend on the K order), so a lane's scale bytes for the stage are
// contiguous: 2 bytes (MXFP4, byte ks selected by the MFMA) or 4 (NVFP4).
// The MFMA's first operand is the W fragment, so each lane ends with 4
// consecutive columns of one output row (one 8- or 16-byte store).
// Workgroup -> tile map: workgroups are dealt round-robin to the 8 XCDs, so
// each XCD is given a contiguous range of tiles; tiles are visited in groups
// of 8 row-tiles so concurrently running workgroups of an XCD share operand
// rows in its L2.
#include <type_traits>

#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWavesM = 2, kWavesN = 2;       // wave grid of the workgroup
constexpr int kThreads = 64 * kWavesM * kWavesN;
// 16-row MFMA tiles per wave: 8 of A by 8 of W (256 accumulator registers)
constexpr int kTM = 8;
constexpr int kTN = 8;
constexpr int BM = 16 * kTM * kWavesM;        // 256 rows of A per workgroup
constexpr int BN = 16 * kTN * kWavesN;        // 256 rows of W
constexpr int BK = 256;                       // FP4 values per stage
constexpr int kRowBytes = BK / 2;             // 128
constexpr int kTileA = BM * kRowBytes;        // 32 KB
constexpr int kTileW = BN * kRowBytes;        // 32 KB
// 16-byte chunks per thread for a tile of ROWS rows (ROWS * 8 is a multiple of kThreads)
template <int ROWS>
constexpr int chunks_of() { return ROWS * kRowBytes / 16 / kThreads; }
static_assert(BM * kRowBytes % (16 * kThreads) == 0 && BN * kRowBytes % (16 * kThreads) == 0,
              "tiles must split evenly over the threads");
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;      // raw buffer descriptor word 3 (gfx9 family)
constexpr int kOutOfRange = 0x7ffffff0;       // a buffer offset past every range: reads 0

template <bool MX>
struct Cfg {
  static constexpr int kScaleRow = MX ? BK / 32 : BK / 16;          // scale bytes per row per stage
  static constexpr int kScaleA = BM * kScaleRow;
  static constexpr int kScaleW = BN * kScaleRow;
  static constexpr int kStageBytes = kTileA + kTileW + kScaleA + kScaleW;
  static constexpr int kLdsBytes = 2 * kStageBytes;                 // 136 KB (MX) / 144 KB (NV)
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

__device__ __forceinline__ int swz(int row, int chunk) {   // byte offset in a tile
  return row * kRowBytes + 16 * (chunk ^ ((row >> 1) & 7));
}

// ------------------------------------------------------------- stage loads --
// Thread t loads 16-byte chunks t + kThreads j of each ROWS-row x 128-byte
// tile (row = chunk / 8) and the stage's scale bytes of row t.  Reads go
// through per-tile buffer descriptors whose range is the tile's rows that
// exist; chunks past K and rows past the matrix read zeros (value 0, and the
// scale bytes of such rows are never stored to an output).
// One operand's part of a stage: its chunks and its scale bytes.
template <bool MX, int ROWS>
struct StageRegs {
  u32x4 d[chunks_of<ROWS>()];
  uint32_t s[MX ? 2 : 4];
};

template <bool MX, bool SCALE_VEC, int ROWS>
__device__ __forceinline__ void load_part(StageRegs<MX, ROWS>& r, __amdgpu_buffer_rsrc_t data,
                                          __amdgpu_buffer_rsrc_t scales, int rowb, int nsc, int K,
                                          int k0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < chunks_of<ROWS>(); ++j) {
    const int c = t + kThreads * j;
    const int row = c >> 3, ch = c & 7;
    const int kc = k0 + 32 * ch;
    // (SCALE_VEC implies K % 256 == 0: no chunk of a stage is past K)
    r.d[j] = __builtin_amdgcn_raw_buffer_load_b128(
        data, (SCALE_VEC || kc < K) ? row * rowb + kc / 2 : kOutOfRange, 0, 0);
  }
  constexpr int bs = MX ? 32 : 16;
  constexpr int spr = Cfg<MX>::kScaleRow;
  const int kb = k0 / bs;
  const int sr = t % ROWS;   // scale row (threads past ROWS repeat rows: same bytes, same place)
  if (SCALE_VEC) {   // K % 256 == 0 and 16-byte aligned scale rows
    if (MX) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(scales, sr * nsc + kb, 0, 0);
      r.s[0] = v.x;
      r.s[1] = v.y;
    } else {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(scales, sr * nsc + kb, 0, 0);
      r.s[0] = v.x;
      r.s[1] = v.y;
      r.s[2] = v.z;
      r.s[3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < spr / 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = kb + 4 * q + i;
        v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(scales, b < nsc ? sr * nsc + b : kOutOfRange,
                                                             0, 0) << (8 * i);
      }
      r.s[q] = v;
    }
  }
}

// tile: the operand's 32 KB tile in the stage buffer; sc: its scale rows
template <bool MX, int ROWS>
__device__ __forceinline__ void store_part(const StageRegs<MX, ROWS>& r, uint8_t* __restrict__ tile,
                                           uint8_t* __restrict__ sc) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < chunks_of<ROWS>(); ++j) {
    const int c = t + kThreads * j;
    *reinterpret_cast<u32x4*>(tile + swz(c >> 3, c & 7)) = r.d[j];
  }
  uint8_t* sp = sc + (t % ROWS) * Cfg<MX>::kScaleRow;
  if (MX)
    *reinterpret_cast<u32x2*>(sp) = u32x2{r.s[0], r.s[1]};
  else
    *reinterpret_cast<u32x4*>(sp) = u32x4{r.s[0], r.s[1], r.s[2], r.s[3]};
}

// --------------------------------------------------------- NV fragment dequant --
// f16 pair (h, h), h = E4M3 value * 2^-8 exactly: the byte's exponent and
// mantissa fields drop into the f16 fields (bias 7 against 15 gives the 2^-8;
// E4M3 subnormals land on f16 subnormals), its sign on the sign.  Bytes
// 0x7f / 0xff (NaN) read as +-480; quantizers never emit them.
__device__ __forceinline__ v2h e4m3_h2(uint32_t byte) {
  const uint32_t h = ((byte & 0x80u) << 8) | ((byte & 0x7fu) << 7);
  return __builtin_bit_cast(v2h, h | (h << 16));
}

// The 8 values E2M1(code) * E4M3 of one dword of codes: the conversion scales by
// 2^8 (exact) and the f16 product with E4M3 * 2^-8 is exact (at most 6
// significant bits, magnitude in [2^-10, 2688]).
__device__ __forceinline__ v8h dq8(uint32_t codes, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// ------------------------------------------------------------------ kernel --
template <bool MX, bool OUT_BF16, bool SCALE_VEC>
__global__ void __launch_bounds__(kThreads, 1)
    k_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ as,
           const uint8_t* __restrict__ W, const uint8_t* __restrict__ ws,
           const float* __restrict__ g_a, const float* __restrict__ g_b, float g_d, int M, int N,
           int K, void* __restrict__ D, int tiles_m, int tiles_n, bool vec_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r16 = lane & 15, g = lane >> 4;
  constexpr int spr = Cfg<MX>::kScaleRow;
  constexpr int bs = MX ? 32 : 16;
  const int rowb = K / 2, nsc = K / bs;

  __amdgpu_buffer_rsrc_t src_a, src_w, src_as, src_ws;
  {
    const int rows_a = min(BM, M - m0), rows_w = min(BN, N - n0);
    src_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A) + (int64_t)m0 * rowb, 0,
                                              rows_a * rowb, kBufferWord3);
    src_w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W) + (int64_t)n0 * rowb, 0,
                                              rows_w * rowb, kBufferWord3);
    src_as = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(as) + (int64_t)m0 * nsc, 0,
                                               rows_a * nsc, kBufferWord3);
    src_ws = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ws) + (int64_t)n0 * nsc, 0,
                                               rows_w * nsc, kBufferWord3);
  }

  v4f acc[kTN][kTM];   // [W tile][A tile]: rows n, columns m of the MFMA
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + BK - 1) / BK;
  constexpr int kStage = Cfg<MX>::kStageBytes;
  // stage buffer layout: A tile | W tile | A scale rows | W scale rows
  auto tile_a = [&](int b) { return smem + b * kStage; };
  auto tile_w = [&](int b) { return smem + b * kStage + kTileA; };
  auto sc_a = [&](int b) { return smem + b * kStage + kTileA + kTileW; };
  auto sc_w = [&](int b) { return smem + b * kStage + kTileA + kTileW + Cfg<MX>::kScaleA; };
  StageRegs<MX, BM> st;
  StageRegs<MX, BN> st2;
  load_part<MX, SCALE_VEC, BM>(st, src_a, src_as, rowb, nsc, K, 0);
  store_part<MX, BM>(st, tile_a(0), sc_a(0));
  load_part<MX, SCALE_VEC, BN>(st2, src_w, src_ws, rowb, nsc, K, 0);
  store_part<MX, BN>(st2, tile_w(0), sc_w(0));
  __syncthreads();

  // The loop body has no branch (a branch lets the compiler sink the MFMAs past
  // the stores and the barrier): after the last stage the next-stage loads read
  // through empty descriptors (zeros, no memory traffic) into the buffer nobody
  // reads again.
  const __amdgpu_buffer_rsrc_t none =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A), 0, 0, kBufferWord3);
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    const int nb = (kt + 1) & 1;
    // the next stage's loads are issued first; A is stored after k-step 0, W
    // after k-step 1
    load_part<MX, SCALE_VEC, BM>(st, more ? src_a : none, more ? src_as : none, rowb, nsc, K,
                                 (kt + 1) * BK);
    load_part<MX, SCALE_VEC, BN>(st2, more ? src_w : none, more ? src_ws : none, rowb, nsc, K,
                                 (kt + 1) * BK);
    const uint8_t* la = tile_a(kt & 1);
    const uint8_t* lw = tile_w(kt & 1);
    const uint8_t* lsa = sc_a(kt & 1);
    const uint8_t* lsw = sc_w(kt & 1);
    const int ra0 = wm * 16 * kTM + r16, rw0 = wn * 16 * kTN + r16;
    // this lane's scale bytes for the stage, one dword per tile
    uint32_t sa[kTM], sw[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      sa[i] = MX ? *reinterpret_cast<const uint16_t*>(lsa + (ra0 + 16 * i) * spr + 2 * g)
                 : *reinterpret_cast<const uint32_t*>(lsa + (ra0 + 16 * i) * spr + 4 * g);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
      sw[i] = MX ? *reinterpret_cast<const uint16_t*>(lsw + (rw0 + 16 * i) * spr + 2 * g)
                 : *reinterpret_cast<const uint32_t*>(lsw + (rw0 + 16 * i) * spr + 4 * g);
    // MXFP4: both k-steps' fragments are read up front, so the second k-step's
    // LDS reads are in flight while the first k-step's MFMAs run (one wave per
    // SIMD has no other wave to hide them behind).  The MFMA's scale byte
    // select must be a constant, hence the k-step template.
    auto read_frags = [&](auto ks_c, u32x4 (&fa)[kTM], u32x4 (&fw)[kTN]) {
      constexpr int ks = decltype(ks_c)::value;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(la + swz(ra0 + 16 * i, 2 * g + ks));
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        fw[i] = *reinterpret_cast<const u32x4*>(lw + swz(rw0 + 16 * i, 2 * g + ks));
    };
    auto mx_kstep = [&](auto ks_c, const u32x4 (&fa)[kTM], const u32x4 (&fw)[kTN]) {
      constexpr int ks = decltype(ks_c)::value;
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        const v8i wv = {(int)fw[i].x, (int)fw[i].y, (int)fw[i].z, (int)fw[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
          const v8i av = {(int)fa[j].x, (int)fa[j].y, (int)fa[j].z, (int)fa[j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wv, av, acc[i][j], 4, 4, ks, (int)sw[i], ks, (int)sa[j]);
        }
      }
    };
    auto nv_kstep = [&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      // (a loop, not unrolled: keeps the accumulators in place in the AGPRs)
#pragma unroll 1
      for (int s4 = 0; s4 < 4; ++s4) {
        // dword s4 of the fragment: 8 values of NV block 4g + 2ks + s4 / 2
        const int sh = 8 * (2 * ks + (s4 >> 1));
        v8h da[kTM], dw[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          const uint32_t ca = *reinterpret_cast<const uint32_t*>(la + swz(ra0 + 16 * i, 2 * g + ks) + 4 * s4);
          da[i] = dq8(ca, e4m3_h2((sa[i] >> sh) & 0xffu));
        }
#pragma unroll
        for (int i = 0; i < kTN; ++i) {
          const uint32_t cw = *reinterpret_cast<const uint32_t*>(lw + swz(rw0 + 16 * i, 2 * g + ks) + 4 * s4);
          dw[i] = dq8(cw, e4m3_h2((sw[i] >> sh) & 0xffu));
        }
#pragma unroll
        for (int i = 0; i < kTN; ++i)
#pragma unroll
          for (int j = 0; j < kTM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dw[i], da[j], acc[i][j], 0, 0, 0);
      }
    };
    // scheduling barriers keep each part's LDS store after the k-step that hides
    // its loads (the compiler would otherwise hoist the stores, and the wait
    // for their loads, above the MFMAs)
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    if constexpr (MX) {
      u32x4 fa0[kTM], fw0[kTN], fa1[kTM], fw1[kTN];
      read_frags(K0{}, fa0, fw0);
      read_frags(K1{}, fa1, fw1);
      mx_kstep(K0{}, fa0, fw0);
      __builtin_amdgcn_sched_barrier(0);
      store_part<MX, BM>(st, tile_a(nb), sc_a(nb));
      __builtin_amdgcn_sched_barrier(0);
      mx_kstep(K1{}, fa1, fw1);
    } else {
      nv_kstep(K0{});
      __builtin_amdgcn_sched_barrier(0);
      store_part<MX, BM>(st, tile_a(nb), sc_a(nb));
      __builtin_amdgcn_sched_barrier(0);
      nv_kstep(K1{});
    }
    __builtin_amdgcn_sched_barrier(0);
    store_part<MX, BN>(st2, tile_w(nb), sc_w(nb));
    __syncthreads();
  }

  // epilogue: lane holds D[m][n .. n+3] for each tile pair; D = acc * ((g_a * g_b) * g_d)
  float alpha = g_d;
  if (!MX) alpha = ((*g_a) * (*g_b)) * g_d;
#pragma unroll
  for (int j = 0; j < kTM; ++j) {
    const int m = m0 + wm * 16 * kTM + 16 * j + r16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n0 + wn * 16 * kTN + 16 * i + 4 * g;
      const v4f v = acc[i][j] * alpha;
      if (OUT_BF16) {
        uint16_t* row = reinterpret_cast<uint16_t*>(D) + (int64_t)m * N;
        if (vec_out && n + 3 < N) {
          *reinterpret_cast<u32x2*>(row + n) =
              u32x2{f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16), f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16)};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) row[n + q] = (uint16_t)f32_to_bf16(v[q]);
        }
      } else {
        float* row = reinterpret_cast<float*>(D) + (int64_t)m * N;
        if (vec_out && n + 3 < N) {
          *reinterpret_cast<v4f*>(row + n) = v;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) row[n + q] = v[q];
        }
      }
    }
  }
}

template <bool MX, bool OUT_BF16, bool SCALE_VEC>
hipError_t launch_t(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K, void* D,
                    hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  constexpr int lds = Cfg<MX>::kLdsBytes;
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<MX, OUT_BF16, SCALE_VEC>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // 4 outputs per store when every row start is aligned to 4 outputs
  const bool vec_out = N % 4 == 0 && reinterpret_cast<uintptr_t>(D) % (OUT_BF16 ? 8 : 16) == 0;
  hipLaunchKernelGGL((k_gemm<MX, OUT_BF16, SCALE_VEC>), dim3(tiles_m * tiles_n), dim3(kThreads), lds,
                     stream, A, as, W, ws, g_a, g_b, g_d, M, N, K, D, tiles_m, tiles_n, vec_out);
  return hipGetLastError();
}

template <bool MX, bool OUT_BF16>
hipError_t launch_s(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K, void* D,
                    hipStream_t stream) {
  const bool vec = K % BK == 0 && (reinterpret_cast<uintptr_t>(as) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
  return vec ? launch_t<MX, OUT_BF16, true>(A, as, W, ws, g_a, g_b, g_d, M, N, K, D, stream)
             : launch_t<MX, OUT_BF16, false>(A, as, W, ws, g_a, g_b, g_d, M, N, K, D, stream);
}

}  // namespace

namespace fp4impl {

hipError_t launch_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales, const float* g_a,
                       const uint8_t* W, const uint8_t* w_scales, const float* g_b, float g_d,
                       int64_t M, int64_t N, int64_t K, void* D, bool d_bf16, hipStream_t stream) {
  // buffer ranges cover one 256-row tile of an operand: 256 * K / 2 < 2^31
  if (M > (1 << 30) || N > (1 << 30) || K >= (1 << 23)) return hipErrorInvalidValue;
  if (mx) {
    return d_bf16 ? launch_s<true, true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                         (int)K, D, stream)
                  : launch_s<true, false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                          (int)K, D, stream);
  }
  return d_bf16 ? launch_s<false, true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                        (int)K, D, stream)
                : launch_s<false, false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                         (int)K, D, stream);
}

}  // namespace fp4impl
