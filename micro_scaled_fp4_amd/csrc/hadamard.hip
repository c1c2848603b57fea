// Fused Walsh-Hadamard rotation + NVFP4 quantization for gfx950.
//
// "NVIDIA NVFP4 与 Micro-Scaling" article, section 4.1: activations are rotated
// by an orthogonal Hadamard matrix (x @ H, H H^T = I, fast Walsh-Hadamard)
// before quantization; "FP4" wiki, 技術實現與量化方法: Hadamard transform and
// stochastic rounding as NVFP4 quantization options.
//
// Layout: a 128-channel group is held by 4 adjacent lanes (an aligned DPP quad),
// 32 contiguous channels per lane, i.e. two whole NVFP4 blocks per lane.
// Butterfly stages h = 1..16 run inside a lane; h = 32 and h = 64 exchange
// registers with the lane at xor distance 1 and 2 through DPP quad
// permutations.  Every stage computes (a, b) -> (a + b, a - b) in float32 on the
// same operand pairs as the plain transform, so the result is bit-identical
// whatever lane holds which value.
//
// Pass 1 (dynamic amax only) rotates and reduces max|y|; pass 2 rotates again
// and encodes, so the rotated tensor never touches HBM.
#include "fp4_device.h"
#include "fp4_internal.h"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 2048;
constexpr int kPer = 32;             // channels per lane
constexpr float kNorm = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128)) = 0.0883883461...

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

// 16-byte vectors of one slot (32 channels) -> float32
template <bool BF16>
__device__ __forceinline__ void unpack32(const u32x4* w, float (&v)[kPer]) {
  if (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = bf16_lo(a[j]);
        v[8 * k + 2 * j + 1] = bf16_hi(a[j]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[4 * k] = __uint_as_float(w[k].x);
      v[4 * k + 1] = __uint_as_float(w[k].y);
      v[4 * k + 2] = __uint_as_float(w[k].z);
      v[4 * k + 3] = __uint_as_float(w[k].w);
    }
  }
}

// DPP quad permutations: lane ^ 1 and lane ^ 2 inside each group of 4 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

// Orthonormal 128-point FWHT of the group held by this lane's quad; p = lane's
// position (0..3) in the quad.
// Stages h = 1 ... 16: the lane's own 32 channels.
__device__ __forceinline__ void fwht_in_lane(float (&v)[kPer]) {
#pragma unroll
  for (int h = 1; h < kPer; h <<= 1) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

__device__ __forceinline__ void fwht128(float (&v)[kPer], int p) {
  fwht_in_lane(v);
  // h = 32: partner lane p ^ 1.  Lower lane keeps a + b, upper lane a - b,
  // computed as partner + (-own) (the same IEEE operation as a - b).
  {
    const uint32_t neg = (p & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float other = dpp_f<kQuadXor1>(v[j]);
      v[j] = other + __uint_as_float(__float_as_uint(v[j]) ^ neg);
    }
  }
  {
    const uint32_t neg = (p & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float other = dpp_f<kQuadXor2>(v[j]);
      v[j] = other + __uint_as_float(__float_as_uint(v[j]) ^ neg);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = v[j] * kNorm;
}

// max |y| over the lane's 32 outputs of the 128-point transform BEFORE the
// final multiply by kNorm (the multiply is monotone, so the caller scales the
// maximum once: max fl(|y| c) = fl(max|y| c)).  Stages up to h = 32 as in
// fwht128.  At h = 64 only magnitudes are needed: of the two outputs a + b and
// a - b of a lane pair, the larger magnitude is |a| + |b| exactly before
// rounding, so max(|fl(a + b)|, |fl(a - b)|) = fl(|a| + |b|), computed by both
// lanes of the pair.
__device__ __forceinline__ float fwht128_absmax_unscaled(float (&v)[kPer], int p) {
  fwht_in_lane(v);
  const uint32_t neg = (p & 1) ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float other = dpp_f<kQuadXor1>(v[j]);
    v[j] = other + __uint_as_float(__float_as_uint(v[j]) ^ neg);
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) m = fmaxf(m, fabsf(dpp_f<kQuadXor2>(v[j])) + fabsf(v[j]));
  return m;
}

// ---------------------------------------------------------- Philox4x32-10 --
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
// (SC'11): 10 rounds of two 32x32->64 multiplies with the Philox constants,
// the round key bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one 32x32->64 multiply per product (v_mad_u64_u32: both halves at once)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Stochastic E2M1 codes of eight values q (value j in nibble j) given the four
// Philox words of their counter: value j takes the 16 bits u_j of word j / 2
// (low half for even j).  For lo <= |q| < hi adjacent E2M1 magnitudes and
// f = (|q| - lo) / (hi - lo), the code rounds up iff
// floor(f * 2^22) + 64 u_j >= 2^22 (|q| >= 6 gives 6, the sign is q's).
// v_cvt_scalef32_sr_pk_fp4_f32 rounds exactly so: it adds 22 bits of its
// random operand (bits 10..31 for the pair's first value, 9..30 for the
// second) to the 22 bits of |q| below the code and keeps the carry.  Each
// value gets an operand of its own, u_j in the top 16 of its 22 bits and zeros
// below, with 0 in the pair's other slot (code 0), so the two values of a pair
// never share random bits.  The instruction leaves the destination's other
// bytes undefined, so only byte 0 of each result is used.
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e2m1_pack8_sr(const float (&q)[8], const uint32_t (&ctr)[4]) {
  uint32_t out = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t r0 = ctr[p] << 16;                 // low half at bits 16..31, 10..15 zero
    const uint32_t r1 = (ctr[p] >> 1) & 0x7fff8000u;  // high half at bits 15..30, 9..14 zero
    const uint32_t a = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2v{q[2 * p], 0.0f}, r0, 1.0f, 0);
    const uint32_t b = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2v{0.0f, q[2 * p + 1]}, r1, 1.0f, 0);
    out |= ((a & 0x0fu) | (b & 0xf0u)) << (8 * p);
  }
  return out;
}

// ------------------------------------------------------------------ kernels --
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
    k_had_amax(const void* __restrict__ x, int64_t nslots, uint32_t* __restrict__ partials) {
  constexpr int VPB = BF16 ? 4 : 8;
  __shared__ u32x4 lds[VPB * (kThreads + 1)];
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int p = threadIdx.x & 3;
  uint32_t m = 0;
  // nslots and the chunk bases are multiples of 4, so the lanes of a quad are
  // all active or all idle (DPP partners are always active).  The next chunk's
  // loads are in flight while this chunk is rotated.
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto chunk_nb = [&](int64_t b) { return (int)(nslots - b < kThreads ? nslots - b : kThreads); };
  u32x4 raw[VPB];
  int64_t base = (int64_t)blockIdx.x * kThreads;
  if (base < nslots) chunk_load<VPB, kThreads>(xv, base, chunk_nb(base), raw);
  for (; base < nslots; base += stride) {
    const int nb = chunk_nb(base);
    u32x4 w[VPB];
    chunk_deal<VPB, kThreads>(raw, nb, lds, w);
    if (base + stride < nslots) chunk_load<VPB, kThreads>(xv, base + stride, chunk_nb(base + stride), raw);
    if ((int)threadIdx.x >= nb) continue;
    float v[kPer];
    unpack32<BF16>(w, v);
    m = umax(m, __float_as_uint(fwht128_absmax_unscaled(v, p)));
  }
  m = block_max_u32(m);   // non-negative floats order as their bit patterns
  if (threadIdx.x == 0) partials[blockIdx.x] = __float_as_uint(__uint_as_float(m) * kNorm);
}

template <bool BF16, bool SR>
__global__ void __launch_bounds__(kThreads)
    k_had_quant(const void* __restrict__ x, int64_t nslots, uint64_t seed, uint8_t* __restrict__ q,
                uint8_t* __restrict__ scales, const float* __restrict__ amax_in,
                const uint32_t* __restrict__ partials, int npart, float* __restrict__ amax_out,
                float* __restrict__ scale_out) {
  float G;
  if (partials == nullptr) {
    G = *amax_in;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npart; i += kThreads) m = umax(m, partials[i]);
    G = __uint_as_float(block_max_u32(m));
  }
  const float s_global = nv_global_scale(G);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) *amax_out = G;
    *scale_out = s_global;
  }
  constexpr int VPB = BF16 ? 4 : 8;
  __shared__ u32x4 lds[VPB * (kThreads + 1)];
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int p = threadIdx.x & 3;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  // the next chunk's loads are in flight while this chunk is rotated and encoded
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto chunk_nb = [&](int64_t b) { return (int)(nslots - b < kThreads ? nslots - b : kThreads); };
  u32x4 raw[VPB];
  int64_t base = (int64_t)blockIdx.x * kThreads;
  if (base < nslots) chunk_load<VPB, kThreads>(xv, base, chunk_nb(base), raw);
  for (; base < nslots; base += stride) {
    const int nb = chunk_nb(base);
    u32x4 wv[VPB];
    chunk_deal<VPB, kThreads>(raw, nb, lds, wv);
    if (base + stride < nslots) chunk_load<VPB, kThreads>(xv, base + stride, chunk_nb(base + stride), raw);
    if ((int)threadIdx.x >= nb) continue;
    const int64_t s = base + threadIdx.x;
    float v[kPer];
    unpack32<BF16>(wv, v);
    fwht128(v, p);
    uint32_t w[4];
    uint32_t sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // max |v| of the block (float max of magnitudes: the abs folds into the
      // max instruction's operand modifiers)
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(v[16 * blk + j]));
      float r;
      nv_block_scale(am, s_global, sc[blk], r);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int base = 16 * blk + 8 * half;
        if (SR) {
          // elements 32s + base .. +7 share Philox counter (32s + base) / 8
          const uint64_t g = (uint64_t)(4 * s + 2 * blk + half);
          uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
          philox4x32_10(ctr, k0, k1);
          float qv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) qv[j] = v[base + j] * r;
          w[2 * blk + half] = e2m1_pack8_sr(qv, ctr);
        } else {
          float qv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) qv[j] = v[base + j] * r;
          w[2 * blk + half] = e2m1_pack8(qv);
        }
      }
    }
    // (non-temporal stores: written once, read by another kernel)
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(q) + s);
    __builtin_nontemporal_store((uint16_t)(sc[0] | (sc[1] << 8)), reinterpret_cast<uint16_t*>(scales) + s);
  }
}

// Writes the VPB vectors out[] of slot base + t (t = threadIdx.x < nb) to
// dst through LDS, so each store instruction covers consecutive 16-byte
// vectors (the inverse of chunk_deal's exchange).  Every thread must call it.
template <int VPB, int NT>
__device__ __forceinline__ void chunk_store(const u32x4 (&out)[VPB], int nb, u32x4* lds,
                                            u32x4* __restrict__ dst, int64_t base) {
  if ((int)threadIdx.x < nb) {
#pragma unroll
    for (int k = 0; k < VPB; ++k) lds[k * (NT + 1) + threadIdx.x] = out[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < VPB; ++k) {
    const int i = threadIdx.x + NT * k;
    if (i < VPB * nb)
      __builtin_nontemporal_store(lds[(i % VPB) * (NT + 1) + i / VPB], dst + base * VPB + i);
  }
  __syncthreads();
}

// y = x H per 128-channel group (the rotation alone), float32 or bf16 out.
template <bool BF16, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads)
    k_had_rotate(const void* __restrict__ x, int64_t nslots, void* __restrict__ y) {
  constexpr int VPB = BF16 ? 4 : 8;
  constexpr int VPO = OUT_BF16 ? 4 : 8;
  __shared__ u32x4 lds[(VPB > VPO ? VPB : VPO) * (kThreads + 1)];
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int p = threadIdx.x & 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto chunk_nb = [&](int64_t b) { return (int)(nslots - b < kThreads ? nslots - b : kThreads); };
  u32x4 raw[VPB];
  int64_t base = (int64_t)blockIdx.x * kThreads;
  if (base < nslots) chunk_load<VPB, kThreads>(xv, base, chunk_nb(base), raw);
  for (; base < nslots; base += stride) {
    const int nb = chunk_nb(base);
    u32x4 w[VPB];
    chunk_deal<VPB, kThreads>(raw, nb, lds, w);
    if (base + stride < nslots) chunk_load<VPB, kThreads>(xv, base + stride, chunk_nb(base + stride), raw);
    u32x4 out[VPO];
    if ((int)threadIdx.x < nb) {
      float v[kPer];
      unpack32<BF16>(w, v);
      fwht128(v, p);
#pragma unroll
      for (int k = 0; k < VPO; ++k) {
        if (OUT_BF16) {
          out[k] = u32x4{bf16_pack2(v[8 * k], v[8 * k + 1]), bf16_pack2(v[8 * k + 2], v[8 * k + 3]),
                         bf16_pack2(v[8 * k + 4], v[8 * k + 5]), bf16_pack2(v[8 * k + 6], v[8 * k + 7])};
        } else {
          out[k] = u32x4{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                         __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
        }
      }
    }
    chunk_store<VPO, kThreads>(out, nb, lds, reinterpret_cast<u32x4*>(y), base);
  }
}

// Rotation + MXFP4: the 32 rotated channels a lane holds are one MXFP4 block,
// so there is no cross-lane work after the FWHT and no global amax (one pass).
template <bool BF16, bool SR>
__global__ void __launch_bounds__(kThreads)
    k_had_quant_mx(const void* __restrict__ x, int64_t nslots, uint64_t seed,
                   uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  constexpr int VPB = BF16 ? 4 : 8;
  __shared__ u32x4 lds[VPB * (kThreads + 1)];
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int p = threadIdx.x & 3;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto chunk_nb = [&](int64_t b) { return (int)(nslots - b < kThreads ? nslots - b : kThreads); };
  u32x4 raw[VPB];
  int64_t base = (int64_t)blockIdx.x * kThreads;
  if (base < nslots) chunk_load<VPB, kThreads>(xv, base, chunk_nb(base), raw);
  for (; base < nslots; base += stride) {
    const int nb = chunk_nb(base);
    u32x4 wv[VPB];
    chunk_deal<VPB, kThreads>(raw, nb, lds, wv);
    if (base + stride < nslots) chunk_load<VPB, kThreads>(xv, base + stride, chunk_nb(base + stride), raw);
    if ((int)threadIdx.x >= nb) continue;
    const int64_t s = base + threadIdx.x;
    float v[kPer];
    unpack32<BF16>(wv, v);
    fwht128(v, p);
    float am = 0.0f;   // max |v| (abs folded into the max instruction)
#pragma unroll
    for (int j = 0; j < kPer; ++j) am = fmaxf(am, fabsf(v[j]));
    const uint32_t sc = e8m0_code(__float_as_uint(am));
    const float inv = e8m0_inv(sc);
    uint32_t w[4];
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) {
      float qv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = v[8 * g8 + j] * inv;     // exact power-of-two multiply
      if (SR) {
        // elements 32 s + 8 g8 .. +7 share Philox counter 4 s + g8
        const uint64_t g = (uint64_t)(4 * s + g8);
        uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
        philox4x32_10(ctr, k0, k1);
        w[g8] = e2m1_pack8_sr(qv, ctr);
      } else {
        w[g8] = e2m1_pack8(qv);
      }
    }
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(q) + s);
    __builtin_nontemporal_store((uint8_t)sc, scales + s);
  }
}

inline int grid_for(int64_t slots) {
  int64_t g = (slots + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (int)(g < kMaxGrid ? g : kMaxGrid);
}

}  // namespace

namespace fp4impl {

hipError_t launch_hadamard_amax(const void* x, bool bf16, int64_t rows, int64_t cols,
                                uint32_t* partials, int* npart, hipStream_t stream) {
  const int64_t nslots = rows * cols / kPer;
  int g = grid_for(nslots);
  if (g > kAmaxPartials) g = kAmaxPartials;
  *npart = g;
  if (bf16)
    hipLaunchKernelGGL(k_had_amax<true>, dim3(g), dim3(kThreads), 0, stream, x, nslots, partials);
  else
    hipLaunchKernelGGL(k_had_amax<false>, dim3(g), dim3(kThreads), 0, stream, x, nslots, partials);
  return hipGetLastError();
}

hipError_t launch_hadamard_quant(const void* x, bool bf16, int64_t rows, int64_t cols, bool sr,
                                 uint64_t seed, uint8_t* q, uint8_t* scales, const float* amax_in,
                                 const uint32_t* partials, int npart, float* amax_out,
                                 float* scale_out, hipStream_t stream) {
  const int64_t nslots = rows * cols / kPer;
  const int g = grid_for(nslots);
#define FP4_HAD_LAUNCH(B, S)                                                                  \
  hipLaunchKernelGGL((k_had_quant<B, S>), dim3(g), dim3(kThreads), 0, stream, x, nslots, seed, q, \
                     scales, amax_in, partials, npart, amax_out, scale_out)
  if (bf16) {
    if (sr) FP4_HAD_LAUNCH(true, true); else FP4_HAD_LAUNCH(true, false);
  } else {
    if (sr) FP4_HAD_LAUNCH(false, true); else FP4_HAD_LAUNCH(false, false);
  }
#undef FP4_HAD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_hadamard_rotate(const void* x, bool bf16, int64_t rows, int64_t cols, void* y,
                                  bool y_bf16, hipStream_t stream) {
  const int64_t nslots = rows * cols / kPer;
  const int g = grid_for(nslots);
#define FP4_ROT_LAUNCH(B, O) \
  hipLaunchKernelGGL((k_had_rotate<B, O>), dim3(g), dim3(kThreads), 0, stream, x, nslots, y)
  if (bf16) {
    if (y_bf16) FP4_ROT_LAUNCH(true, true); else FP4_ROT_LAUNCH(true, false);
  } else {
    if (y_bf16) FP4_ROT_LAUNCH(false, true); else FP4_ROT_LAUNCH(false, false);
  }
#undef FP4_ROT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_hadamard_quant_mx(const void* x, bool bf16, int64_t rows, int64_t cols, bool sr,
                                    uint64_t seed, uint8_t* q, uint8_t* scales,
                                    hipStream_t stream) {
  const int64_t nslots = rows * cols / kPer;
  const int g = grid_for(nslots);
#define FP4_HMX_LAUNCH(B, S)                                                                     \
  hipLaunchKernelGGL((k_had_quant_mx<B, S>), dim3(g), dim3(kThreads), 0, stream, x, nslots, seed, \
                     q, scales)
  if (bf16) {
    if (sr) FP4_HMX_LAUNCH(true, true); else FP4_HMX_LAUNCH(true, false);
  } else {
    if (sr) FP4_HMX_LAUNCH(false, true); else FP4_HMX_LAUNCH(false, false);
  }
#undef FP4_HMX_LAUNCH
  return hipGetLastError();
}

}  // namespace fp4impl
