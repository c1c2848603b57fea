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
// its own 8 x 8 block of 16x16 MFMA tiles (accumulators in AGPRs); the plain
// MXFP4 launch runs 2 x 4 waves of 8 x 4 tiles instead (k_gemm_mx8, below).
// Plain launches are persistent (one workgroup per CU walks several tiles, its
// loads running on from one tile into the next).  K advances 256 values
// (128 bytes per row) per stage in two k-steps of 128; stages are
// double-buffered in LDS and filled by buffer loads that write LDS directly
// (no register staging, no LDS store instructions), one barrier per stage.
// MXFP4 runs the loads two stages ahead and reads the next k-step's operand
// fragments while the current k-step's MFMAs run, one MFMA row at a time, so
// no MFMA waits on LDS after a barrier.  A 16-byte chunk c of tile row r is
// stored at chunk position c ^ ((r >> 1) & 7): the 16 rows of a fragment read
// then cover all 64 banks.  Inside a stage, lane group g (lane / 16) takes values
// [64g + 32ks, +32) in k-step ks, identically for both operands (the MFMA sum
// does not depend on the K order), so a lane's scale bytes for the stage are
// contiguous: 2 bytes (MXFP4, byte ks selected by the MFMA) or 4 (NVFP4).
// The MFMA's first operand is the W fragment, so each lane ends with 4
// consecutive columns of one output row (one 4-, 8- or 16-byte store for an
// E4M3, bf16 or float32 output).  The E4M3 output (section 五's scaled-mm
// example writes float8_e4m3fn) is the float32 result's sign bit followed by
// the nearest E4M3 magnitude, ties to the even code, saturating at 448.
// Workgroup -> tile map: workgroups are dealt round-robin to the 8 XCDs, so
// each XCD is given a contiguous range of tiles; tiles are visited in groups
// of 8 row-tiles so concurrently running workgroups of an XCD share operand
// rows in its L2.  A persistent workgroup w takes tiles w, w + G, ... with G a
// multiple of 8, so it stays on one XCD and the ranges hold.
#include <atomic>
#include <type_traits>
#include <utility>

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
// the stage loads below assume 256-row tiles of both operands, one scale row per thread
static_assert(BM == 256 && BN == 256 && kThreads == 256, "stage loads assume 256-row tiles");
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
// Workgroup bid -> tile t in [0, T): the hardware deals workgroups round-robin
// to the kXcds XCDs, so XCD x runs workgroups x, x + kXcds, ...; of those below
// T it takes the contiguous tiles [start_x, start_x + n_x).  A bijection on
// [0, T) for any T; false for bid >= T.
__device__ __forceinline__ bool xcd_tile(int bid, int T, int& t) {
  if (bid >= T) return false;
  const int x = bid % kXcds, k = bid / kXcds;
  const int q = T / kXcds, rem = T % kXcds;
  t = x * q + min(x, rem) + k;
  return true;
}

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  int t;
  xcd_tile(bid, tiles_m * tiles_n, t);   // callers pass bid < tiles_m * tiles_n
  const int in_group = kGroupM * tiles_n;
  const int group = t / in_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int r = t - group * in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Grouped GEMM (one launch over E groups, e.g. the experts of an MoE layer).
// Group e's rows are goff[e] .. goff[e+1] (clamped into [0, M], so rows never
// leave A or D); it has ceil(rows / BM) row tiles.  Each wave walks the
// offsets 64 groups at a time with a lane prefix sum; the waves of a
// workgroup reach the same results, so no barrier is needed.

// Tile count of the groups c .. c + 63 held one per lane: (first row, one past
// the last row, row tiles) of lane's group, and the inclusive prefix sum.
__device__ __forceinline__ void group_chunk(const int32_t* __restrict__ goff, int ngroups, int M,
                                            int c, int& l0, int& l1, int& tl, int& inc) {
  const int lane = threadIdx.x & 63;
  const int e = c + lane;
  l0 = l1 = tl = 0;
  if (e < ngroups) {
    l0 = min(max(goff[e], 0), M);
    l1 = min(max(goff[e + 1], l0), M);
    tl = (l1 - l0 + BM - 1) / BM;
  }
  inc = tl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d, 64);
    if ((threadIdx.x & 63) >= d) inc += v;
  }
}

// Total row tiles over all groups.
__device__ __forceinline__ int group_row_tiles(const int32_t* __restrict__ goff, int ngroups, int M) {
  int total = 0;
  for (int c = 0; c < ngroups; c += 64) {
    int l0, l1, tl, inc;
    group_chunk(goff, ngroups, M, c, l0, l1, tl, inc);
    total += __shfl(inc, 63, 64);
  }
  return total;
}

// Row tile `row_tile` -> group e, its first row lo, one past its last row hi,
// and the tile's index tm inside the group.  False past the last group's tiles.
__device__ __forceinline__ bool group_tile_of(const int32_t* __restrict__ goff, int ngroups, int M,
                                              int row_tile, int& e_out, int& tm, int& lo, int& hi) {
  int base = 0;
  for (int c = 0; c < ngroups; c += 64) {
    int l0, l1, tl, inc;
    group_chunk(goff, ngroups, M, c, l0, l1, tl, inc);
    const int start = base + inc - tl;
    const uint64_t hit = __ballot(c + (int)(threadIdx.x & 63) < ngroups && row_tile >= start &&
                                  row_tile < start + tl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      e_out = c + src;
      tm = row_tile - __shfl(start, src, 64);
      lo = __shfl(l0, src, 64);
      hi = __shfl(l1, src, 64);
      return true;
    }
    base += __shfl(inc, 63, 64);
  }
  return false;
}

// D += W x A with block scales, FP4 operands (16 bytes of codes per lane):
// v_mfma_scale_f32_16x16x128_f8f6f4, accumulating in place in AGPRs.  SW / SA
// select the scale byte of sw / sa.  Written as inline asm because the
// compiler, with all 256 AGPRs holding accumulators, moves accumulators
// between AGPRs and VGPRs around its own MFMAs (hundreds of copies per stage).
// The compiler does not apply MFMA hazard rules to inline asm, so the callers
// keep them: operands come straight from LDS reads (waited on by the
// compiler), each group of MFMAs starts after 2 wait states (s_nop 1, for a
// vector-ALU write of an operand just before), and results are read only
// after mfma_drain.
template <int SW, int SA>
__device__ __forceinline__ void mfma_fp4(v4f& acc, const u32x4& w, const u32x4& a, uint32_t sw,
                                         uint32_t sa) {
  asm volatile(
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] "
      "cbsz:4 blgp:4"
      : "+a"(acc)
      : "v"(w), "v"(a), "v"(sw), "v"(sa), "n"(SW & 1), "n"(SA & 1), "n"(SW >> 1), "n"(SA >> 1));
}
// D += W x A, fp16 operands (8 values per lane each): v_mfma_f32_16x16x32_f16
// in place in AGPRs, under the same rules as mfma_fp4.
__device__ __forceinline__ void mfma_f16(v4f& acc, const v8h& w, const v8h& a) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(w), "v"(a));
}
// 2 wait states before a group of MFMAs (vector-ALU write -> MFMA read); no
// instruction is scheduled across it
__device__ __forceinline__ void mfma_lead() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}
// wait states after the last MFMA before its result is read (24 >= what a
// 4-pass MFMA result needs before a vector-ALU or accvgpr read)
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// Wait until this wave's buffer loads, including those that write LDS
// directly, have completed (vmcnt(0); the lgkm and exp counters are left
// alone).  The compiler orders a wave's direct-to-LDS loads only before that
// wave's own later LDS reads, never before another wave's, so each barrier
// that publishes such loads to the workgroup is preceded by this.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// lgkmcnt(0): LDS and scalar-memory operations of this wave have completed
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{})
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int swz(int row, int chunk) {   // byte offset in a tile
  return row * kRowBytes + 16 * (chunk ^ ((row >> 1) & 7));
}

// ------------------------------------------------------------- stage loads --
// Operand tiles go from global memory straight into LDS (buffer loads with the
// LDS flag): one instruction moves 64 x 16 bytes, lane l's 16 bytes landing at
// LDS base + 16 l.  A 256-row tile is 32 such 1 KB blocks (8 rows each); wave
// w loads blocks w, w + 4, ...  Lane l of block b fills tile row 8b + l / 8 at
// chunk position l % 8, so it fetches the chunk that the swizzle puts there.
// Reads go through per-tile buffer descriptors whose range is the tile's rows
// that exist: rows past the matrix and chunks past K land in LDS as zeros
// (value 0; the scale bytes of such rows never reach an output).
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBlocksPerWave = 256 * kRowBytes / 1024 / (kThreads / 64);   // 8
static_assert(kThreads == 256, "blocks are dealt to 4 waves");

// Block q (of kBlocksPerWave) of this wave's share of an operand tile.
template <bool SCALE_VEC>
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t src, uint8_t* tile, int rowb, int K,
                                          int k0, int q) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block b = wave + 4q holds rows 8b .. 8b + 7; the swizzle of those rows
  // depends only on the parity of b, which is the parity of the wave
  const int row0 = 8 * wave + (lane >> 3);
  const int ch = (lane & 7) ^ ((row0 >> 1) & 7);   // logical chunk stored at position lane % 8
  const int kc = k0 + 32 * ch;
  lds_void* dst = (lds_void*)(tile + 1024 * (wave + 4 * q));
  if (SCALE_VEC)   // K % 256 == 0: no chunk of a stage is past K; the block's row offset is scalar
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, row0 * rowb + kc / 2, 32 * q * rowb, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, kc < K ? (row0 + 32 * q) * rowb + kc / 2 : kOutOfRange,
                                             0, 0, 0);
}

template <bool SCALE_VEC>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t src, uint8_t* tile, int rowb, int K,
                                         int k0) {
#pragma unroll
  for (int q = 0; q < kBlocksPerWave; ++q) dma_block<SCALE_VEC>(src, tile, rowb, K, k0, q);
}

// One operand's scale bytes of a stage, in registers between their global load
// and their LDS store: thread t holds row t's 8 (MXFP4) or 16 (NVFP4) bytes.
template <bool MX>
struct StageScales {
  uint32_t s[MX ? 2 : 4];
};

template <bool MX, bool SCALE_VEC>
__device__ __forceinline__ void load_scales(StageScales<MX>& r, __amdgpu_buffer_rsrc_t scales, int nsc,
                                            int k0) {
  constexpr int bs = MX ? 32 : 16;
  constexpr int spr = Cfg<MX>::kScaleRow;
  const int kb = k0 / bs;
  const int sr = threadIdx.x;
  if (SCALE_VEC) {   // K % 256 == 0 and 16-byte aligned scale rows
    if constexpr (MX) {
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

// LDS scale layout of an operand: entry (h, g, r16, i) holds the bytes that lane
// group g of MFMA tile i of wave half h needs for tile row r16 (MXFP4: 2 bytes,
// one per k-step; NVFP4: 4 bytes, one per 16 values).  The 8 tiles' entries of
// (h, g, r16) are contiguous, so a lane fetches its whole stage's scales with
// one (MXFP4) or two (NVFP4) 16-byte reads.  Thread t holds scale row t, which
// is row r16 = t % 16 of tile t / 16 = 8 h + i of the 256-row operand tile.
template <bool MX>
__device__ __forceinline__ void store_scales(const StageScales<MX>& r, uint8_t* __restrict__ sc) {
  const int t = threadIdx.x, h = t >> 7, i = (t >> 4) & 7, r16 = t & 15;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int e = ((h * 4 + g) * 16 + r16) * 8 + i;
    if (MX)
      reinterpret_cast<uint16_t*>(sc)[e] = (uint16_t)(r.s[g >> 1] >> (16 * (g & 1)));
    else
      reinterpret_cast<uint32_t*>(sc)[e] = r.s[g];
  }
}

// ---------------------------------------------------------------- epilogue --
// Writes a wave's outputs: lane (r16, g) holds D[mb + 16 j][nb + 16 i .. +3]
// (before the multiply by alpha) in acc[i][j].  EDGE: the tile may cross M or
// N, or rows may not take whole 4-output stores; otherwise every store is
// whole and unconditional.
template <int OUT, bool EDGE, int TN = kTN, int TM = kTM>
__device__ __forceinline__ void store_outputs(v4f (&acc)[TN][TM], float alpha, float s_glob,
                                              int mb, int nb, int M, int N, void* __restrict__ D,
                                              uint8_t* __restrict__ d_scales, bool vec_out, int r16,
                                              int g) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = mb + 16 * j;
    if (EDGE && m >= M) continue;
    if constexpr (OUT == 0) {
      // NVFP4.  The 16 columns of block (m, i) are held by the lanes r16 + 16 g'
      // (g' = 0..3), which share m.  Per group of 4 tiles the lanes reduce the
      // 4 block maxima, lane g computes the scale of block i4 + g (as the
      // quantizer does) and stores its byte, and every lane takes each block's
      // multiplier from the lane that computed it.
      uint8_t* qrow = reinterpret_cast<uint8_t*>(D) + (int64_t)m * ((N + 1) / 2);
      uint8_t* srow = d_scales + (int64_t)m * ((N + 15) / 16);
#pragma unroll
      for (int i4 = 0; i4 < TN; i4 += 4) {
        v4f x[4];
        float a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // (keeps the accumulator in its AGPRs until here: read tile by tile,
          // the epilogue needs a few VGPRs, not 256)
          asm volatile("" : "+a"(acc[i4 + k][j]));
          x[k] = acc[i4 + k][j] * alpha;
          if (EDGE) {
            const int n = nb + 16 * (i4 + k);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q >= N) x[k][q] = 0.0f;
          }
          a[k] = fmaxf(fmaxf(fabsf(x[k].x), fabsf(x[k].y)), fmaxf(fabsf(x[k].z), fabsf(x[k].w)));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = fmaxf(a[k], __shfl_xor(a[k], 16, 64));
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = fmaxf(a[k], __shfl_xor(a[k], 32, 64));
        const float ab = g == 0 ? a[0] : g == 1 ? a[1] : g == 2 ? a[2] : a[3];
        uint32_t sc;
        float r;
        nv_block_scale(ab, s_glob, sc, r);
        const int nblk = nb + 12 * g + 16 * i4;   // first column of block i4 + g
        if (!EDGE || nblk < N) srow[nblk / 16] = (uint8_t)sc;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float rk = __shfl(r, r16 + 16 * k, 64);
          uint32_t c = e2m1_pack2<0>(0u, x[k].x * rk, x[k].y * rk);
          c = e2m1_pack2<1>(c, x[k].z * rk, x[k].w * rk);
          const int n = nb + 16 * (i4 + k);
          if (!EDGE || (vec_out && n + 3 < N)) {
            *reinterpret_cast<uint16_t*>(qrow + n / 2) = (uint16_t)c;
          } else {
            if (n < N) qrow[n / 2] = (uint8_t)c;
            if (n + 2 < N) qrow[n / 2 + 1] = (uint8_t)(c >> 8);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = nb + 16 * i;
        asm volatile("" : "+a"(acc[i][j]));
        const v4f v = acc[i][j] * alpha;
        const bool whole = !EDGE || (vec_out && n + 3 < N);
        if constexpr (OUT == 2) {
          uint16_t* row = reinterpret_cast<uint16_t*>(D) + (int64_t)m * N;
          const u32x2 h = u32x2{bf16_pack2(v.x, v.y), bf16_pack2(v.z, v.w)};
          if (whole) {
            *reinterpret_cast<u32x2*>(row + n) = h;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < N) row[n + q] = (uint16_t)(h[q >> 1] >> (16 * (q & 1)));
          }
        } else if constexpr (OUT == 1) {
          uint8_t* row = reinterpret_cast<uint8_t*>(D) + (int64_t)m * N;
          const uint32_t c = e4m3_pack4_signed(v.x, v.y, v.z, v.w);
          if (whole) {
            *reinterpret_cast<uint32_t*>(row + n) = c;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < N) row[n + q] = (uint8_t)(c >> (8 * q));
          }
        } else {
          float* row = reinterpret_cast<float*>(D) + (int64_t)m * N;
          if (whole) {
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
}

// ------------------------------------------------------------------ kernel --
// GROUPED: A and D hold the groups' rows back to back (group e: rows goff[e] ..
// goff[e+1]), W and w_scales one [N, K] operand per group, g_b one tensor
// scale per group; the grid is an upper bound on the groups' tiles.
template <bool MX, int OUT, bool SCALE_VEC, bool GROUPED>
__global__ void __launch_bounds__(kThreads, 1)
    k_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ as,
           const uint8_t* __restrict__ W, const uint8_t* __restrict__ ws,
           const float* __restrict__ g_a, const float* __restrict__ g_b, float g_d, int M, int N,
           int K, void* __restrict__ D, uint8_t* __restrict__ d_scales,
           const float* __restrict__ d_amax, float* __restrict__ d_gscale, int tiles_m, int tiles_n,
           bool vec_out, const int32_t* __restrict__ goff, int ngroups) {
  static_assert(!GROUPED || OUT != 0, "grouped launches write float32, bf16 or E4M3");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // Plain launches are persistent: at most one workgroup per CU, workgroup w
  // taking tiles w, w + G, ... (G a multiple of the XCD count), with the load
  // schedule running on across tiles as in k_gemm_mx8 (the last stage of a
  // tile loads the next tile's first two stages; the tile's output stores
  // drain while the next tile computes; a tile's stages are padded to an even
  // count).  Grouped launches take one tile per workgroup (their group lookup
  // inside the tile loop would not fit the registers without spills).
  constexpr bool kPersist = !GROUPED;
  const int G = gridDim.x;
  // grouped: the groups' tiles (the grid is an upper bound) dealt to the XCDs
  // in contiguous ranges; the column tile runs fastest, so the workgroups of an
  // XCD share the row tile of A in its L2
  const int T = GROUPED ? group_row_tiles(goff, ngroups, M) * tiles_n : tiles_m * tiles_n;
  int bid = blockIdx.x;
  if (bid >= T) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r16 = lane & 15, g = lane >> 4;
  constexpr int bs = MX ? 32 : 16;
  const int rowb = K / 2, nsc = K / bs;

  // Tile b: its first row of A (a_row) and of W (w_row, group included), the
  // rows of each that exist, its origin inside its group (m0, n0), the group's
  // rows (m_rows) and the group (e).  Past the last tile: no rows, so loads
  // through its empty ranges read zeros and touch no memory.
  struct TileRows {
    int64_t a_row, w_row;
    int rows_a, rows_w, m0, n0, m_rows, e;
  };
  auto tile_rows = [&](int b) {
    TileRows t{0, 0, 0, 0, 0, 0, 0, 0};
    if (b >= T) return t;
    int tm = 0, tn = 0, lo = 0;
    t.m_rows = M;
    if constexpr (GROUPED) {
      int tt, hi;
      xcd_tile(b, T, tt);
      if (!group_tile_of(goff, ngroups, M, tt / tiles_n, t.e, tm, lo, hi)) return t;
      tn = tt % tiles_n;
      t.m_rows = hi - lo;
    } else {
      tile_of(b, tiles_m, tiles_n, tm, tn);
    }
    t.m0 = tm * BM;
    t.n0 = tn * BN;
    t.a_row = (int64_t)lo + t.m0;
    t.w_row = (int64_t)t.e * N + t.n0;
    t.rows_a = min(BM, t.m_rows - t.m0);
    t.rows_w = min(BN, N - t.n0);
    return t;
  };
  auto rsrc_a = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A) + t.a_row * rowb, 0,
                                             t.rows_a * rowb, kBufferWord3);
  };
  auto rsrc_w = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W) + t.w_row * rowb, 0,
                                             t.rows_w * rowb, kBufferWord3);
  };
  auto rsrc_as = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(as) + t.a_row * nsc, 0,
                                             t.rows_a * nsc, kBufferWord3);
  };
  auto rsrc_ws = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ws) + t.w_row * nsc, 0,
                                             t.rows_w * nsc, kBufferWord3);
  };
  // A grouped workgroup's one tile is looked up once.  Plain launches carry
  // the coordinates (tile row, tile column; -1 past the last tile) of the
  // current and the next tile from tile to tile, and derive the rest where it
  // is needed (few scalar registers, no division inside the loop).
  const TileRows tile0 = tile_rows(bid);
  auto rows_of = [&](int tm, int tn) {
    TileRows t{0, 0, 0, 0, 0, 0, M, 0};
    if (tm >= 0) {
      t.m0 = tm * BM;
      t.n0 = tn * BN;
      t.a_row = t.m0;
      t.w_row = t.n0;
      t.rows_a = min(BM, M - t.m0);
      t.rows_w = min(BN, N - t.n0);
    }
    return t;
  };
  auto coords = [&](int b, int& tm, int& tn) {
    tm = tn = -1;
    if (b < T) tile_of(b, tiles_m, tiles_n, tm, tn);
  };
  int ctm = -1, ctn = -1, xtm = -1, xtn = -1;
  if constexpr (kPersist) {
    coords(bid, ctm, ctn);
    coords(bid + G, xtm, xtn);
  }
  auto tile_at = [&](bool next) {
    if constexpr (kPersist) return next ? rows_of(xtm, xtn) : rows_of(ctm, ctn);
    else return next ? TileRows{0, 0, 0, 0, 0, 0, 0, 0} : tile0;
  };

  v4f acc[kTN][kTM];   // [W tile][A tile]: rows n, columns m of the MFMA
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + BK - 1) / BK, nk2 = (nk + 1) & ~1;
  // The loads of stage kt + 2 of the current tile: from this tile, from the
  // next tile past the (padded) end, or nothing for a padding stage.
  auto load_tile = [&](int kt, int& k_ld) {
    const int kl = kt + 2;
    const bool nx = kl >= nk2;
    k_ld = (nx ? kl - nk2 : kl) * BK;
    TileRows t = tile_at(nx);
    if (!nx && kl >= nk) t.rows_a = t.rows_w = 0;
    return t;
  };
  // LDS layout: A scales of buffers 0, 1 | W scales 0, 1 | A tiles 0, 1 | W tiles 0, 1
  // (every access of one kind differs from the others by a 16-bit LDS offset)
  constexpr int kScA = Cfg<MX>::kScaleA, kScW = Cfg<MX>::kScaleW;
  constexpr int kTiles = 2 * (kScA + kScW);
  auto sc_a = [&](int b) { return smem + b * kScA; };
  auto sc_w = [&](int b) { return smem + 2 * kScA + b * kScW; };
  auto tile_a = [&](int b) { return smem + kTiles + b * kTileA; };
  auto tile_w = [&](int b) { return smem + kTiles + 2 * kTileA + b * kTileW; };
  // an empty range: loads through it read zeros and touch no memory
  const __amdgpu_buffer_rsrc_t none =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A), 0, 0, kBufferWord3);
  const int ra0 = wm * 16 * kTM + r16, rw0 = wn * 16 * kTN + r16;

  // this lane's scale bytes of a stage (layout at store_scales).  MXFP4: tile i's
  // two bytes are bytes 2 (i & 1) + ks of dword i / 2 (the MFMA selects the
  // byte); NVFP4: dword i, byte 2 ks + s4 / 2 for dword s4 of k-step ks.
  constexpr int kScDw = MX ? 4 : 8;   // dwords per lane per operand
  auto read_scales = [&](int b, uint32_t (&sa)[kScDw], uint32_t (&sw)[kScDw]) {
    const u32x4* lsa = reinterpret_cast<const u32x4*>(sc_a(b)) + ((wm * 4 + g) * 16 + r16) * (kScDw / 4);
    const u32x4* lsw = reinterpret_cast<const u32x4*>(sc_w(b)) + ((wn * 4 + g) * 16 + r16) * (kScDw / 4);
#pragma unroll
    for (int q = 0; q < kScDw / 4; ++q) {
      const u32x4 va = lsa[q], vw = lsw[q];
      sa[4 * q] = va.x; sa[4 * q + 1] = va.y; sa[4 * q + 2] = va.z; sa[4 * q + 3] = va.w;
      sw[4 * q] = vw.x; sw[4 * q + 1] = vw.y; sw[4 * q + 2] = vw.z; sw[4 * q + 3] = vw.w;
    }
  };
  // MXFP4 operand fragment: 32 FP4 values (16 bytes) of a tile row per lane
  auto frag = [&](const uint8_t* tile, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(tile + swz(row, chunk));
  };
  auto read_frags = [&](int b, auto ks_c, u32x4 (&fa)[kTM], u32x4 (&fw)[kTN]) {
    constexpr int ks = decltype(ks_c)::value;
#pragma unroll
    for (int i = 0; i < kTM; ++i) fa[i] = frag(tile_a(b), ra0 + 16 * i, 2 * g + ks);
#pragma unroll
    for (int i = 0; i < kTN; ++i) fw[i] = frag(tile_w(b), rw0 + 16 * i, 2 * g + ks);
  };
  // row i of k-step ks: W tile i against the kTM A tiles.  The MFMA's scale
  // byte select must be a constant, hence the templates.
  auto mx_row = [&](auto i_c, auto ks_c, const u32x4 (&fa)[kTM], const u32x4 (&fw)[kTN],
                    const uint32_t (&sa)[kScDw], const uint32_t (&sw)[kScDw]) {
    constexpr int i = decltype(i_c)::value;
    constexpr int ks = decltype(ks_c)::value;
    static_for<kTM>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      mfma_fp4<2 * (i & 1) + ks, 2 * (j & 1) + ks>(acc[i][j], fw[i], fa[j], sw[i >> 1], sa[j >> 1]);
    });
  };
  // NVFP4 sub-step u (k-step u / 4, dword u % 4 of the lane's 16-byte chunk):
  // one dword of codes per tile (8 values of NV block 4g + 2 (u / 4) + (u % 4) / 2),
  // dequantized to fp16, then 64 fp16 MFMAs.
  auto raw_dw = [&](const uint8_t* tile, int row, int u) {
    return *reinterpret_cast<const uint32_t*>(tile + swz(row, 2 * g + (u >> 2)) + 4 * (u & 3));
  };
  // f16 pair (h(b0), h(b1)) of the two E4M3 scale bytes of k-step ks in a tile's
  // scale dword, h(b) = E4M3(b) * 2^-8: one v_cvt_scalef32_pk_f16_fp8 with the
  // scale 2^-8 (exact for every finite E4M3 byte, subnormals included; a NaN
  // byte gives NaN)
  auto scale_pair = [&](uint32_t scale_dw, int ks) {
    const v2h p = ks ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_dw, 0x1p-8f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_dw, 0x1p-8f, false);
    return __builtin_bit_cast(uint32_t, p);
  };
  // values 2k, 2k + 1 (k = part) of the 8 dequantized values of sub-step u: the
  // E2M1 codes scaled by 2^8, times the scale of block half (u % 4) / 2
  auto dq_part = [&](v8h& d, uint32_t codes, uint32_t pair, auto part_c, int u) {
    constexpr int part = decltype(part_c)::value;
    const v2h t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, part);
    const v2h h = __builtin_bit_cast(v2h, pair);
    const v2h r = t * (((u & 3) >> 1) ? v2h{h.y, h.y} : v2h{h.x, h.x});
    d[2 * part] = r.x;
    d[2 * part + 1] = r.y;
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;

  // epilogue of tile t: lane holds D[m][n .. n+3] for each tile pair;
  // D = acc * ((g_a * g_b) * g_d)
  float s_glob = 1.0f;   // NVFP4 output: tensor scale of D from its given amax, as the quantizer's
  if (OUT == 0) {
    s_glob = nv_global_scale(*d_amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *d_gscale = s_glob;
  }
  auto epilogue = [&](const TileRows& t) {
    float alpha = g_d;
    if (!MX) alpha = ((*g_a) * g_b[t.e]) * g_d;
    // a grouped tile writes the rows of its group, which start at row a_row - m0
    void* Dt = reinterpret_cast<uint8_t*>(D) + (t.a_row - t.m0) * N * OUT;
    const int mb = t.m0 + wm * 16 * kTM + r16, nb = t.n0 + wn * 16 * kTN + 4 * g;
    if (vec_out && t.m0 + BM <= t.m_rows && t.n0 + BN <= N)
      store_outputs<OUT, false>(acc, alpha, s_glob, mb, nb, t.m_rows, N, Dt, d_scales, true, r16, g);
    else
      store_outputs<OUT, true>(acc, alpha, s_glob, mb, nb, t.m_rows, N, Dt, d_scales, vec_out, r16, g);
  };
  // next tile: zero the accumulators (compile-time indices keep them in registers)
  auto next_tile = [&]() {
    if constexpr (!kPersist) return false;
    bid += G;
    if (bid >= T) return false;
    ctm = xtm;
    ctn = xtn;
    coords(bid + G, xtm, xtn);
    static_for<kTN>([&](auto i_c) {
      static_for<kTM>([&](auto j_c) {
        acc[decltype(i_c)::value][decltype(j_c)::value] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      });
    });
    return true;
  };
  // Every loop body below is branch-free (a branch lets the compiler sink the
  // MFMAs past the stores and the barrier): stages past the last one are loaded
  // through the empty range (zeros into a buffer that is never read again).
  StageScales<MX> ssa, ssw;   // a later stage's scale bytes, from global load to LDS store
  if constexpr (MX) {
    // Stage s lives in buffer s & 1.  Loads run two stages ahead: stage kt + 2
    // is issued right after the barrier of iteration kt, into the buffer stage
    // kt has finished with, and must land by the next barrier.  The operand
    // fragments of the first k-step of stage kt + 1 are read during the second
    // k-step's MFMAs of stage kt, so no MFMA waits for LDS after a barrier.
    load_scales<MX, SCALE_VEC>(ssa, rsrc_as(tile0), nsc, 0);
    load_scales<MX, SCALE_VEC>(ssw, rsrc_ws(tile0), nsc, 0);
    dma_tile<SCALE_VEC>(rsrc_a(tile0), tile_a(0), rowb, K, 0);
    dma_tile<SCALE_VEC>(rsrc_w(tile0), tile_w(0), rowb, K, 0);
    store_scales<MX>(ssa, sc_a(0));
    store_scales<MX>(ssw, sc_w(0));
    const bool two = nk > 1;
    load_scales<MX, SCALE_VEC>(ssa, two ? rsrc_as(tile0) : none, nsc, BK);
    load_scales<MX, SCALE_VEC>(ssw, two ? rsrc_ws(tile0) : none, nsc, BK);
    dma_tile<SCALE_VEC>(two ? rsrc_a(tile0) : none, tile_a(1), rowb, K, BK);
    dma_tile<SCALE_VEC>(two ? rsrc_w(tile0) : none, tile_w(1), rowb, K, BK);
    wait_dma();
    __syncthreads();
    uint32_t sa0[kScDw], sw0[kScDw], sa1[kScDw], sw1[kScDw];
    u32x4 fa0[kTM], fw0[kTN], fa1[kTM], fw1[kTN];
    read_scales(0, sa0, sw0);
    read_frags(0, K0{}, fa0, fw0);
    // nothing but LDS reads outstanding on the LDS/scalar counter from here on
    // (a pending scalar load would turn every LDS wait in the loop into a full drain)
    wait_lgkm();
    static_assert(kTM == 8 && kTN == 8 && kBlocksPerWave == 8, "one load slot per W tile row");
    // One stage: buffer CB holds stage kt (scales sa / sw); the scales of stage
    // kt + 1 are read into sa_n / sw_n.  Fragment reads are spread over the
    // MFMA rows in the order the next k-step consumes them (its first row needs
    // every A fragment and W fragment 0).
    auto mx_stage = [&](auto cb_c, int kt, const uint32_t (&sa)[kScDw], const uint32_t (&sw)[kScDw],
                        uint32_t (&sa_n)[kScDw], uint32_t (&sw_n)[kScDw]) {
      constexpr int cb = decltype(cb_c)::value, nb = cb ^ 1;
      // k-step 0 of stage kt, reading the fragments of k-step 1
      mfma_lead();
      static_for<kTN>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        mx_row(i_c, K0{}, fa0, fw0, sa, sw);
        if constexpr (i < 4) {
          fa1[2 * i] = frag(tile_a(cb), ra0 + 32 * i, 2 * g + 1);
          fa1[2 * i + 1] = frag(tile_a(cb), ra0 + 32 * i + 16, 2 * g + 1);
        } else {
          fw1[2 * i - 8] = frag(tile_w(cb), rw0 + 32 * i - 128, 2 * g + 1);
          fw1[2 * i - 7] = frag(tile_w(cb), rw0 + 32 * i - 112, 2 * g + 1);
        }
      });
      store_scales<MX>(ssa, sc_a(nb));   // stage kt + 1
      store_scales<MX>(ssw, sc_w(nb));
      wait_dma();        // stage kt + 1 (issued during the previous stage) has landed
      __syncthreads();   // stage kt + 1 is in buffer nb; nobody reads buffer cb any more
      // k-step 1 of stage kt, issuing one block of each operand's stage kt + 2
      // loads per row and reading the fragments of stage kt + 1, k-step 0
      int k_ld;
      const TileRows lt = load_tile(kt, k_ld);
      const __amdgpu_buffer_rsrc_t la = rsrc_a(lt), lw = rsrc_w(lt);
      load_scales<MX, SCALE_VEC>(ssa, rsrc_as(lt), nsc, k_ld);
      load_scales<MX, SCALE_VEC>(ssw, rsrc_ws(lt), nsc, k_ld);
      mfma_lead();
      static_for<kTN>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        mx_row(i_c, K1{}, fa1, fw1, sa, sw);
        if constexpr (i == 0) read_scales(nb, sa_n, sw_n);
        dma_block<SCALE_VEC>(la, tile_a(cb), rowb, K, k_ld, i);
        dma_block<SCALE_VEC>(lw, tile_w(cb), rowb, K, k_ld, i);
        if constexpr (i < 4) {
          fa0[2 * i] = frag(tile_a(nb), ra0 + 32 * i, 2 * g);
          fa0[2 * i + 1] = frag(tile_a(nb), ra0 + 32 * i + 16, 2 * g);
        } else {
          fw0[2 * i - 8] = frag(tile_w(nb), rw0 + 32 * i - 128, 2 * g);
          fw0[2 * i - 7] = frag(tile_w(nb), rw0 + 32 * i - 112, 2 * g);
        }
      });
      // the accumulators are read after the loop: 24 wait states after the last MFMA
      mfma_drain();
    };
    // Two stages per iteration, so the scale registers alternate without
    // copies.  With an odd stage count the last iteration's second stage is
    // one past the end: it was loaded through the empty range (FP4 codes 0,
    // scale bytes 0) and adds exact zeros.
    do {
      for (int kt = 0; kt < nk2; kt += 2) {
        mx_stage(std::integral_constant<int, 0>{}, kt, sa0, sw0, sa1, sw1);
        mx_stage(std::integral_constant<int, 1>{}, kt + 1, sa1, sw1, sa0, sw0);
      }
      epilogue(tile_at(false));
    } while (next_tile());
  } else {
    // Stage s lives in buffer s & 1.  A stage is 8 sub-steps; in sub-step u the
    // 64 MFMAs run on the fp16 operands of u while the codes of u + 1 are
    // dequantized and those of u + 2 read from LDS (one tile row of each after
    // each MFMA row), all double-buffered in registers.  The barrier comes after
    // sub-step 5, once this stage's last codes have been read: sub-steps 6 and 7
    // then issue the loads of stage kt + 2 (into this stage's buffer) and read
    // and dequantize the first codes of stage kt + 1, so no MFMA waits at a
    // stage boundary.
    load_scales<MX, SCALE_VEC>(ssa, rsrc_as(tile0), nsc, 0);
    load_scales<MX, SCALE_VEC>(ssw, rsrc_ws(tile0), nsc, 0);
    dma_tile<SCALE_VEC>(rsrc_a(tile0), tile_a(0), rowb, K, 0);
    dma_tile<SCALE_VEC>(rsrc_w(tile0), tile_w(0), rowb, K, 0);
    store_scales<MX>(ssa, sc_a(0));
    store_scales<MX>(ssw, sc_w(0));
    const bool two = nk > 1;
    load_scales<MX, SCALE_VEC>(ssa, two ? rsrc_as(tile0) : none, nsc, BK);
    load_scales<MX, SCALE_VEC>(ssw, two ? rsrc_ws(tile0) : none, nsc, BK);
    dma_tile<SCALE_VEC>(two ? rsrc_a(tile0) : none, tile_a(1), rowb, K, BK);
    dma_tile<SCALE_VEC>(two ? rsrc_w(tile0) : none, tile_w(1), rowb, K, BK);
    wait_dma();
    __syncthreads();
    uint32_t sa0[kScDw], sw0[kScDw], sa1[kScDw], sw1[kScDw];
    uint32_t ra[2][kTM], rw[2][kTN];   // codes of sub-steps u (parity u & 1)
    v8h da[2][kTM], dw[2][kTN];        // fp16 operands of sub-steps u (parity u & 1)
    uint32_t pa[2][kTM], pw[2][kTN];   // scale pairs of k-steps 0 and 1 of a stage
    read_scales(0, sa0, sw0);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      ra[0][i] = raw_dw(tile_a(0), ra0 + 16 * i, 0);
      ra[1][i] = raw_dw(tile_a(0), ra0 + 16 * i, 1);
      rw[0][i] = raw_dw(tile_w(0), rw0 + 16 * i, 0);
      rw[1][i] = raw_dw(tile_w(0), rw0 + 16 * i, 1);
    }
    wait_lgkm();
    static_for<kTM>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      pa[0][i] = scale_pair(sa0[i], 0);
      pw[0][i] = scale_pair(sw0[i], 0);
      static_for<4>([&](auto k_c) {
        dq_part(da[0][i], ra[0][i], pa[0][i], k_c, 0);
        dq_part(dw[0][i], rw[0][i], pw[0][i], k_c, 0);
      });
    });
    // Each MFMA is issued with its share of the other work in a slot of its
    // own (no instruction crosses a slot), so the vector ALU work runs while
    // the MFMA pipe is busy: per MFMA row i, slot j dequantizes dword j % 4 of
    // the next sub-step's A (j < 4) or W (j >= 4) tile i; slots 0 and 4 read
    // the codes two sub-steps ahead; sub-step 2 forms the scale pairs of
    // k-step 1, sub-step 6 those of the next stage's k-step 0 (rows 4-7) and
    // issues one block of each operand's loads per row.
    auto nv_stage = [&](auto cb_c, int kt, const uint32_t (&sa)[kScDw], const uint32_t (&sw)[kScDw],
                        uint32_t (&sa_n)[kScDw], uint32_t (&sw_n)[kScDw]) {
      constexpr int cb = decltype(cb_c)::value, nb = cb ^ 1;
      int k_ld;
      const TileRows lt = load_tile(kt, k_ld);
      const __amdgpu_buffer_rsrc_t la = rsrc_a(lt), lw = rsrc_w(lt);
      static_for<8>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int p = u & 1, q = p ^ 1;
        constexpr int un = (u + 1) & 7;          // sub-step dequantized here (next stage's 0 after 7)
        constexpr int kn = un >> 2;              // its k-step
        if constexpr (u == 6) {
          // every wave has read this stage's last codes (sub-step 7, read in 5)
          store_scales<MX>(ssa, sc_a(nb));   // stage kt + 1
          store_scales<MX>(ssw, sc_w(nb));
          wait_dma();        // stage kt + 1 (issued during the previous stage) has landed
          __syncthreads();   // stage kt + 1 is in buffer nb; buffer cb is free
          load_scales<MX, SCALE_VEC>(ssa, rsrc_as(lt), nsc, k_ld);
          load_scales<MX, SCALE_VEC>(ssw, rsrc_ws(lt), nsc, k_ld);
          read_scales(nb, sa_n, sw_n);
        }
        mfma_lead();
        static_for<kTN>([&](auto i_c) {
          constexpr int i = decltype(i_c)::value;
          static_for<kTM>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            mfma_f16(acc[i][j], dw[p][i], da[p][j]);
            if constexpr (j < 4)
              dq_part(da[q][i], ra[q][i], pa[kn][i], std::integral_constant<int, j>{}, un);
            else
              dq_part(dw[q][i], rw[q][i], pw[kn][i], std::integral_constant<int, j - 4>{}, un);
            if constexpr (j == 0) {   // codes of sub-step u + 2 (the next stage's 0, 1 after the barrier)
              if constexpr (u + 2 < 8) ra[p][i] = raw_dw(tile_a(cb), ra0 + 16 * i, u + 2);
              else ra[p][i] = raw_dw(tile_a(nb), ra0 + 16 * i, u - 6);
            }
            if constexpr (j == 4) {
              if constexpr (u + 2 < 8) rw[p][i] = raw_dw(tile_w(cb), rw0 + 16 * i, u + 2);
              else rw[p][i] = raw_dw(tile_w(nb), rw0 + 16 * i, u - 6);
            }
            if constexpr (u == 2 && j == 1) pa[1][i] = scale_pair(sa[i], 1);
            if constexpr (u == 2 && j == 5) pw[1][i] = scale_pair(sw[i], 1);
            if constexpr (u == 6 && i >= 4 && j == 1) {
              pa[0][2 * i - 8] = scale_pair(sa_n[2 * i - 8], 0);
              pa[0][2 * i - 7] = scale_pair(sa_n[2 * i - 7], 0);
            }
            if constexpr (u == 6 && i >= 4 && j == 5) {
              pw[0][2 * i - 8] = scale_pair(sw_n[2 * i - 8], 0);
              pw[0][2 * i - 7] = scale_pair(sw_n[2 * i - 7], 0);
            }
            if constexpr (u == 6 && j == 2) dma_block<SCALE_VEC>(la, tile_a(cb), rowb, K, k_ld, i);
            if constexpr (u == 6 && j == 6) dma_block<SCALE_VEC>(lw, tile_w(cb), rowb, K, k_ld, i);
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      });
      // the accumulators are read after the loop: 24 wait states after the last MFMA
      mfma_drain();
    };
    // two stages per iteration (scale registers alternate); an odd stage count
    // runs one stage past the end, loaded through the empty range (codes 0,
    // scale bytes 0: exact zeros)
    do {
      for (int kt = 0; kt < nk2; kt += 2) {
        nv_stage(std::integral_constant<int, 0>{}, kt, sa0, sw0, sa1, sw1);
        nv_stage(std::integral_constant<int, 1>{}, kt + 1, sa1, sw1, sa0, sw0);
      }
      epilogue(tile_at(false));
    } while (next_tile());
  }
}

// ------------------------------------------------ MXFP4 kernel, 8 waves --
// The MXFP4 GEMM with 8 waves (2 per SIMD) on the same 256 x 256 tile: a
// 2 x 4 wave grid, each wave 128 x 64 outputs (8 A tiles by 4 W tiles of
// 16 x 16, 128 accumulator registers).  Stages, tile swizzle, load schedule,
// A's scale layout and the epilogue are those of k_gemm.  With two waves on a
// SIMD, one wave's MFMAs run while the other is held up issuing its
// direct-to-LDS loads, reading LDS or at the stage barrier.  A wave reads 8 A
// and 4 W fragments per k-step, so a CU reads 96 KB of fragments per k-step
// (64 KB with 4 waves of 128 x 128).  W's scale layout follows the wave
// quarters: entry (q, g, r16, i) holds the two bytes (k-steps 0 and 1) of lane
// group g for row r16 of MFMA tile i of W quarter q, so a lane reads its 4
// tiles' bytes with one 8-byte read.
constexpr int kThreads8 = 512;
constexpr int kW8N = 4;                          // waves along W (2 along A)
constexpr int kT8N = 4;                          // W tiles per wave (kTM A tiles)
static_assert(16 * kTM * 2 == BM && 16 * kT8N * kW8N == BN, "the 8-wave grid covers the tile");

// Block q (of 4) of this wave's share of an operand tile: block b = wave + 8q
// holds rows 8b .. 8b + 7 (their swizzle depends only on b's parity, the
// wave's), filled as in dma_block.
template <bool SCALE_VEC>
__device__ __forceinline__ void dma_block8(__amdgpu_buffer_rsrc_t src, uint8_t* tile, int rowb, int K,
                                           int k0, int q) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = 8 * wave + (lane >> 3);
  const int ch = (lane & 7) ^ ((row0 >> 1) & 7);
  const int kc = k0 + 32 * ch;
  lds_void* dst = (lds_void*)(tile + 1024 * (wave + 8 * q));
  if (SCALE_VEC)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, row0 * rowb + kc / 2, 64 * q * rowb, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, kc < K ? (row0 + 64 * q) * rowb + kc / 2 : kOutOfRange,
                                             0, 0, 0);
}

template <bool SCALE_VEC>
__device__ __forceinline__ void dma_tile8(__amdgpu_buffer_rsrc_t src, uint8_t* tile, int rowb, int K,
                                          int k0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) dma_block8<SCALE_VEC>(src, tile, rowb, K, k0, q);
}

// Threads 0..255 hold A's scale row t of a stage, threads 256..511 W's row
// t - 256 (8 bytes each).
__device__ __forceinline__ bool holds_a_scales() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4;
}

template <bool SCALE_VEC>
__device__ __forceinline__ void load_scales8(StageScales<true>& r, __amdgpu_buffer_rsrc_t sa,
                                             __amdgpu_buffer_rsrc_t sw, int nsc, int k0) {
  const __amdgpu_buffer_rsrc_t src = holds_a_scales() ? sa : sw;
  const int kb = k0 / 32;
  const int sr = threadIdx.x & 255;
  if (SCALE_VEC) {   // K % 256 == 0 and 16-byte aligned scale rows
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(src, sr * nsc + kb, 0, 0);
    r.s[0] = v.x;
    r.s[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = kb + 4 * q + i;
        v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(src, b < nsc ? sr * nsc + b : kOutOfRange,
                                                             0, 0) << (8 * i);
      }
      r.s[q] = v;
    }
  }
}

__device__ __forceinline__ void store_scales8(const StageScales<true>& r, uint8_t* __restrict__ sc_a,
                                              uint8_t* __restrict__ sc_w) {
  const int t = threadIdx.x & 255, r16 = t & 15;
  const bool a = holds_a_scales();
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint16_t v = (uint16_t)(r.s[g >> 1] >> (16 * (g & 1)));
    if (a)   // A: (half h, g, r16, tile i of 8), as store_scales
      reinterpret_cast<uint16_t*>(sc_a)[(((t >> 7) * 4 + g) * 16 + r16) * 8 + ((t >> 4) & 7)] = v;
    else     // W: (quarter q, g, r16, tile i of 4)
      reinterpret_cast<uint16_t*>(sc_w)[(((t >> 6) * 4 + g) * 16 + r16) * 4 + ((t >> 4) & 3)] = v;
  }
}

// Persistent: the grid is at most one workgroup per CU, and workgroup w takes
// tiles w, w + G, w + 2G, ... (G = grid size, a multiple of the XCD count, so
// a workgroup stays on one XCD and tile_of's XCD ranges hold).  The load
// schedule runs on across tiles: the last stage of a tile loads the first two
// stages of the next one, and the tile's output stores drain while the next
// tile computes (with one tile per workgroup launch, every tile's stores and
// load fill stood between two tiles' MFMAs: ~15% of the 8192 x 28672 x 8192
// GEMM).  A tile's stages are padded to an even count (two per loop
// iteration); a padding stage loads nothing and adds exact zeros.
template <int OUT, bool SCALE_VEC>
__global__ void __launch_bounds__(kThreads8, 1)
    k_gemm_mx8(const uint8_t* __restrict__ A, const uint8_t* __restrict__ as,
               const uint8_t* __restrict__ W, const uint8_t* __restrict__ ws, float g_d, int M,
               int N, int K, void* __restrict__ D, uint8_t* __restrict__ d_scales,
               const float* __restrict__ d_amax, float* __restrict__ d_gscale, int tiles_m,
               int tiles_n, bool vec_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int T = tiles_m * tiles_n, G = gridDim.x;
  int bid = blockIdx.x;
  if (bid >= T) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kW8N, wn = wave % kW8N;
  const int r16 = lane & 15, g = lane >> 4;
  const int rowb = K / 2, nsc = K / 32;

  // tile b's origin and rows that exist (none past the last tile: loads
  // through its empty ranges read zeros and touch no memory)
  struct TileRows {
    int m0, n0, rows_a, rows_w;
  };
  auto tile_rows = [&](int b) {
    TileRows t{0, 0, 0, 0};
    if (b < T) {
      int tm, tn;
      tile_of(b, tiles_m, tiles_n, tm, tn);
      t.m0 = tm * BM;
      t.n0 = tn * BN;
      t.rows_a = min(BM, M - t.m0);
      t.rows_w = min(BN, N - t.n0);
    }
    return t;
  };
  auto rsrc_a = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A) + (int64_t)t.m0 * rowb, 0,
                                             t.rows_a * rowb, kBufferWord3);
  };
  auto rsrc_w = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W) + (int64_t)t.n0 * rowb, 0,
                                             t.rows_w * rowb, kBufferWord3);
  };
  auto rsrc_as = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(as) + (int64_t)t.m0 * nsc, 0,
                                             t.rows_a * nsc, kBufferWord3);
  };
  auto rsrc_ws = [&](const TileRows& t) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ws) + (int64_t)t.n0 * nsc, 0,
                                             t.rows_w * nsc, kBufferWord3);
  };

  v4f acc[kT8N][kTM];   // [W tile][A tile]
#pragma unroll
  for (int i = 0; i < kT8N; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + BK - 1) / BK, nk2 = (nk + 1) & ~1;
  // LDS layout as k_gemm's MXFP4 layout
  constexpr int kScA = Cfg<true>::kScaleA, kScW = Cfg<true>::kScaleW;
  constexpr int kTiles = 2 * (kScA + kScW);
  auto sc_a = [&](int b) { return smem + b * kScA; };
  auto sc_w = [&](int b) { return smem + 2 * kScA + b * kScW; };
  auto tile_a = [&](int b) { return smem + kTiles + b * kTileA; };
  auto tile_w = [&](int b) { return smem + kTiles + 2 * kTileA + b * kTileW; };
  const __amdgpu_buffer_rsrc_t none =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A), 0, 0, kBufferWord3);
  const int ra0 = wm * 16 * kTM + r16, rw0 = wn * 16 * kT8N + r16;

  // this lane's scale bytes of a stage: A tile j's two bytes are bytes
  // 2 (j & 1) + ks of dword j / 2 of sa, W tile i's of dword i / 2 of sw
  auto read_scales = [&](int b, uint32_t (&sa)[4], uint32_t (&sw)[2]) {
    const u32x4 va = *reinterpret_cast<const u32x4*>(sc_a(b) + ((wm * 4 + g) * 16 + r16) * 16);
    const u32x2 vw = *reinterpret_cast<const u32x2*>(sc_w(b) + ((wn * 4 + g) * 16 + r16) * 8);
    sa[0] = va.x; sa[1] = va.y; sa[2] = va.z; sa[3] = va.w;
    sw[0] = vw.x; sw[1] = vw.y;
  };
  auto frag = [&](const uint8_t* tile, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(tile + swz(row, chunk));
  };
  // row i of k-step ks: W tile i against the kTM A tiles
  auto mx_row = [&](auto i_c, auto ks_c, const u32x4 (&fa)[kTM], const u32x4 (&fw)[kT8N],
                    const uint32_t (&sa)[4], const uint32_t (&sw)[2]) {
    constexpr int i = decltype(i_c)::value;
    constexpr int ks = decltype(ks_c)::value;
    static_for<kTM>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      mfma_fp4<2 * (i & 1) + ks, 2 * (j & 1) + ks>(acc[i][j], fw[i], fa[j], sw[i >> 1], sa[j >> 1]);
    });
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;

  TileRows cur = tile_rows(bid), nxt = tile_rows(bid + G);
  // Stage s of a tile lives in buffer s & 1 (nk2 is even, so every tile starts
  // in buffer 0); loads run two stages ahead as in k_gemm's MXFP4 loop, every
  // loop body branch-free.
  StageScales<true> ss;
  load_scales8<SCALE_VEC>(ss, rsrc_as(cur), rsrc_ws(cur), nsc, 0);
  dma_tile8<SCALE_VEC>(rsrc_a(cur), tile_a(0), rowb, K, 0);
  dma_tile8<SCALE_VEC>(rsrc_w(cur), tile_w(0), rowb, K, 0);
  store_scales8(ss, sc_a(0), sc_w(0));
  const bool two = nk > 1;
  load_scales8<SCALE_VEC>(ss, two ? rsrc_as(cur) : none, two ? rsrc_ws(cur) : none, nsc, BK);
  dma_tile8<SCALE_VEC>(two ? rsrc_a(cur) : none, tile_a(1), rowb, K, BK);
  dma_tile8<SCALE_VEC>(two ? rsrc_w(cur) : none, tile_w(1), rowb, K, BK);
  wait_dma();
  __syncthreads();
  uint32_t sa0[4], sw0[2], sa1[4], sw1[2];
  u32x4 fa0[kTM], fw0[kT8N], fa1[kTM], fw1[kT8N];
  read_scales(0, sa0, sw0);
#pragma unroll
  for (int i = 0; i < kTM; ++i) fa0[i] = frag(tile_a(0), ra0 + 16 * i, 2 * g);
#pragma unroll
  for (int i = 0; i < kT8N; ++i) fw0[i] = frag(tile_w(0), rw0 + 16 * i, 2 * g);
  wait_lgkm();
  // One stage: buffer CB holds stage kt (scales sa / sw); row i of a k-step
  // also reads A fragments 2i, 2i + 1 and W fragment i of the next k-step (the
  // order the next k-step's first row needs them in).  The loads of stage
  // kt + 2 come from this tile, or past its (padded) end from the next tile.
  auto mx_stage = [&](auto cb_c, int kt, const uint32_t (&sa)[4], const uint32_t (&sw)[2],
                      uint32_t (&sa_n)[4], uint32_t (&sw_n)[2]) {
    constexpr int cb = decltype(cb_c)::value, nb = cb ^ 1;
    mfma_lead();
    static_for<kT8N>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      mx_row(i_c, K0{}, fa0, fw0, sa, sw);
      fa1[2 * i] = frag(tile_a(cb), ra0 + 32 * i, 2 * g + 1);
      fa1[2 * i + 1] = frag(tile_a(cb), ra0 + 32 * i + 16, 2 * g + 1);
      fw1[i] = frag(tile_w(cb), rw0 + 16 * i, 2 * g + 1);
    });
    store_scales8(ss, sc_a(nb), sc_w(nb));   // the next stage
    wait_dma();        // the next stage (issued during the previous stage) has landed
    __syncthreads();   // it is in buffer nb; nobody reads buffer cb any more
    const int kl = kt + 2;
    const bool nx = kl >= nk2;                   // stage kl - nk2 of the next tile
    const bool live = nx || kl < nk;
    const int k_ld = (nx ? kl - nk2 : kl) * BK;
    TileRows lt = nx ? nxt : cur;
    if (!live) lt.rows_a = lt.rows_w = 0;        // a padding stage: empty ranges
    const __amdgpu_buffer_rsrc_t la = rsrc_a(lt), lw = rsrc_w(lt);
    load_scales8<SCALE_VEC>(ss, rsrc_as(lt), rsrc_ws(lt), nsc, k_ld);
    mfma_lead();
    static_for<kT8N>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      mx_row(i_c, K1{}, fa1, fw1, sa, sw);
      if constexpr (i == 0) read_scales(nb, sa_n, sw_n);
      dma_block8<SCALE_VEC>(la, tile_a(cb), rowb, K, k_ld, i);
      dma_block8<SCALE_VEC>(lw, tile_w(cb), rowb, K, k_ld, i);
      fa0[2 * i] = frag(tile_a(nb), ra0 + 32 * i, 2 * g);
      fa0[2 * i + 1] = frag(tile_a(nb), ra0 + 32 * i + 16, 2 * g);
      fw0[i] = frag(tile_w(nb), rw0 + 16 * i, 2 * g);
    });
    mfma_drain();
  };

  float s_glob = 1.0f;
  if (OUT == 0) {
    s_glob = nv_global_scale(*d_amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *d_gscale = s_glob;
  }
  for (;;) {
    for (int kt = 0; kt < nk2; kt += 2) {
      mx_stage(std::integral_constant<int, 0>{}, kt, sa0, sw0, sa1, sw1);
      mx_stage(std::integral_constant<int, 1>{}, kt + 1, sa1, sw1, sa0, sw0);
    }
    const int m0 = cur.m0, n0 = cur.n0;
    const int mb = m0 + wm * 16 * kTM + r16, nb = n0 + wn * 16 * kT8N + 4 * g;
    if (vec_out && m0 + BM <= M && n0 + BN <= N)
      store_outputs<OUT, false, kT8N, kTM>(acc, g_d, s_glob, mb, nb, M, N, D, d_scales, true, r16, g);
    else
      store_outputs<OUT, true, kT8N, kTM>(acc, g_d, s_glob, mb, nb, M, N, D, d_scales, vec_out, r16, g);
    bid += G;
    if (bid >= T) break;
    cur = nxt;
    nxt = tile_rows(bid + G);
    // (compile-time indices: the accumulators stay in registers)
    static_for<kT8N>([&](auto i_c) {
      static_for<kTM>([&](auto j_c) {
        acc[decltype(i_c)::value][decltype(j_c)::value] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      });
    });
  }
}

// Output of one GEMM call: D, plus the NVFP4 scale bytes, given amax and
// written tensor scale when D holds NVFP4 codes.
struct OutArgs {
  void* D;
  uint8_t* d_scales;
  const float* d_amax;
  float* d_gscale;
};

// Groups of a grouped launch: ngroups > 0 selects the grouped kernel.
struct Groups {
  const int32_t* offsets;
  int ngroups;
};

template <bool MX, int OUT, bool SCALE_VEC, bool GROUPED = false>
hipError_t launch_t(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K,
                    const OutArgs& o, hipStream_t stream, const Groups& gr = Groups{nullptr, 0}) {
  const int tiles_n = (N + BN - 1) / BN;
  // grouped: each group adds at most one partial row tile to ceil(M / BM)
  const int tiles_m = (M + BM - 1) / BM + (GROUPED ? gr.ngroups : 0);
  constexpr int lds = Cfg<MX>::kLdsBytes;
  // MXFP4: the 8-wave kernel (grouped launches: k_gemm, whose group lookup
  // would not fit the 8-wave kernel's 256 registers without spills); NVFP4: k_gemm
  constexpr bool kMx8 = MX && !GROUPED;
  const void* fn = kMx8 ? reinterpret_cast<const void*>(&k_gemm_mx8<OUT, SCALE_VEC>)
                        : reinterpret_cast<const void*>(&k_gemm<MX, OUT, SCALE_VEC, GROUPED>);
  static std::atomic<uint64_t> lds_set{0};   // devices on which this kernel's LDS limit is set
  const hipError_t e = fp4impl::set_lds_limit_once(lds_set, fn, lds);
  if (e != hipSuccess) return e;
  // 4 outputs per store when every row start is aligned to 4 outputs
  // (NVFP4: 4 outputs are 2 bytes)
  const bool vec_out =
      N % 4 == 0 && reinterpret_cast<uintptr_t>(o.D) % (OUT == 0 ? 2 : 4 * OUT) == 0;
  // persistent kernels: at most one workgroup per CU, a multiple of the XCD
  // count when there are more tiles than CUs (grouped: tiles_m * tiles_n is an
  // upper bound on the tiles)
  const int T = tiles_m * tiles_n, ncu = fp4impl::num_cus();
  const int grid = GROUPED || T <= ncu ? T : (ncu >= kXcds ? ncu / kXcds * kXcds : ncu);
  if constexpr (kMx8) {
    hipLaunchKernelGGL((k_gemm_mx8<OUT, SCALE_VEC>), dim3(grid), dim3(kThreads8), lds, stream, A,
                       as, W, ws, g_d, M, N, K, o.D, o.d_scales, o.d_amax, o.d_gscale, tiles_m,
                       tiles_n, vec_out);
  } else {
    hipLaunchKernelGGL((k_gemm<MX, OUT, SCALE_VEC, GROUPED>), dim3(grid),
                       dim3(kThreads), lds, stream, A, as, W, ws, g_a, g_b, g_d, M, N, K, o.D,
                       o.d_scales, o.d_amax, o.d_gscale, tiles_m, tiles_n, vec_out, gr.offsets,
                       gr.ngroups);
  }
  return hipGetLastError();
}

template <bool MX, int OUT>
hipError_t launch_s(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K,
                    const OutArgs& o, hipStream_t stream) {
  const bool vec = K % BK == 0 && (reinterpret_cast<uintptr_t>(as) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
  return vec ? launch_t<MX, OUT, true>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream)
             : launch_t<MX, OUT, false>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream);
}

// d_bytes: 4 float32, 2 bf16, 1 E4M3, 0 NVFP4 codes
template <bool MX>
hipError_t launch_o(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                    const float* g_a, const float* g_b, float g_d, int M, int N, int K,
                    const OutArgs& o, int d_bytes, hipStream_t stream) {
  switch (d_bytes) {
    case 4: return launch_s<MX, 4>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream);
    case 2: return launch_s<MX, 2>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream);
    case 1: return launch_s<MX, 1>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream);
    case 0: return launch_s<MX, 0>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool MX>
hipError_t launch_grouped_o(const uint8_t* A, const uint8_t* as, const uint8_t* W, const uint8_t* ws,
                            const float* g_a, const float* g_b, float g_d, int M, int N, int K,
                            void* D, int d_bytes, const Groups& gr, hipStream_t stream) {
  const bool vec = K % BK == 0 && (reinterpret_cast<uintptr_t>(as) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
  const OutArgs o{D, nullptr, nullptr, nullptr};
#define FP4_GG(OUTV)                                                                          \
  return vec ? launch_t<MX, OUTV, true, true>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream, gr) \
             : launch_t<MX, OUTV, false, true>(A, as, W, ws, g_a, g_b, g_d, M, N, K, o, stream, gr)
  switch (d_bytes) {
    case 4: FP4_GG(4);
    case 2: FP4_GG(2);
    case 1: FP4_GG(1);
    default: return hipErrorInvalidValue;
  }
#undef FP4_GG
}

__global__ void k_global_scale(const float* __restrict__ amax, float* __restrict__ out) {
  if (threadIdx.x == 0) *out = nv_global_scale(*amax);
}

}  // namespace

namespace fp4impl {

hipError_t launch_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales, const float* g_a,
                       const uint8_t* W, const uint8_t* w_scales, const float* g_b, float g_d,
                       int64_t M, int64_t N, int64_t K, void* D, int d_bytes, hipStream_t stream) {
  return launch_gemm_nvfp4_out(mx, A, a_scales, g_a, W, w_scales, g_b, g_d, M, N, K, D, d_bytes,
                               nullptr, nullptr, nullptr, stream);
}

hipError_t launch_gemm_nvfp4_out(bool mx, const uint8_t* A, const uint8_t* a_scales,
                                 const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                                 const float* g_b, float g_d, int64_t M, int64_t N, int64_t K,
                                 void* D, int d_bytes, uint8_t* d_scales, const float* d_amax,
                                 float* d_gscale, hipStream_t stream) {
  // buffer ranges cover one 256-row tile of an operand: 256 * K / 2 < 2^31
  if (M > (1 << 30) || N > (1 << 30) || K >= (1 << 23)) return hipErrorInvalidValue;
  if (d_bytes == 0 && (d_scales == nullptr || d_amax == nullptr || d_gscale == nullptr))
    return hipErrorInvalidValue;
  const OutArgs o{D, d_scales, d_amax, d_gscale};
  return mx ? launch_o<true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N, (int)K, o,
                             d_bytes, stream)
            : launch_o<false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N, (int)K, o,
                              d_bytes, stream);
}

hipError_t launch_grouped_gemm(bool mx, const uint8_t* A, const uint8_t* a_scales,
                               const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                               const float* g_b, float g_d, int64_t ngroups,
                               const int32_t* offsets, int64_t M, int64_t N, int64_t K, void* D,
                               int d_bytes, hipStream_t stream) {
  // buffer ranges cover one 256-row tile of an operand: 256 * K / 2 < 2^31
  if (M > (1 << 30) || N > (1 << 30) || K >= (1 << 23) || ngroups > (1 << 20))
    return hipErrorInvalidValue;
  if (((M + BM - 1) / BM + ngroups) * ((N + BN - 1) / BN) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const Groups gr{offsets, (int)ngroups};
  return mx ? launch_grouped_o<true>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N, (int)K,
                                     D, d_bytes, gr, stream)
            : launch_grouped_o<false>(A, a_scales, W, w_scales, g_a, g_b, g_d, (int)M, (int)N,
                                      (int)K, D, d_bytes, gr, stream);
}

hipError_t launch_nv_global_scale(const float* amax, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_global_scale, dim3(1), dim3(64), 0, stream, amax, out);
  return hipGetLastError();
}

}  // namespace fp4impl
