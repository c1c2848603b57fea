/*
 * fp4.h -- C ABI of libfp4.so: NVFP4 / MXFP4 micro-scaled FP4 on AMD Instinct
 * MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller.  The library never
 *    allocates or frees memory and never synchronizes: the work is enqueued on
 *    `stream` (NULL = the null stream) and the call returns.
 *  - Tensors are row-major and contiguous.  Blocks of 16 (NVFP4) or 32 (MXFP4)
 *    values run along the last dimension ("cols", the GEMM's K); a last partial
 *    block covers the remaining columns.
 *  - Packed FP4: a row of C values takes ceil(C/2) bytes; value 2j sits in the
 *    low nibble of byte j, value 2j+1 in the high nibble; the high nibble of an
 *    odd row's last byte is 0.  FP4 code = sign<<3 | E2M1 magnitude code, values
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6} ("FP4" wiki, 技術原理: ONNX FLOAT4E2M1 rule and
 *    packing; 10100.com data-type article, "nvFP4的数据结构设计").
 *  - Argument checks (NULL, shape, dtype, alignment, workspace size) run on the
 *    host before anything is enqueued; on failure the call returns the status
 *    and enqueues nothing.  A launch failure returns FP4_ERR_HIP.  Device faults
 *    surface at the caller's next synchronization (HIP semantics).
 *  - The device must be gfx950; anything else returns FP4_ERR_ARCH (no silent
 *    fallback to another precision).
 *  - Non-finite inputs, |x| >= 2^126 and tensors whose amax is below ~1e-30 are
 *    outside the contract: no fault, outputs unspecified.
 *  - Calls on distinct streams with distinct buffers are independent; the
 *    library keeps no device state between calls.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_ERR_NULL = 1,      /* a required pointer is NULL                        */
  FP4_ERR_SHAPE = 2,     /* negative size, K not a multiple of the block, ... */
  FP4_ERR_DTYPE = 3,     /* unknown dtype / format / rounding enum            */
  FP4_ERR_ALIGN = 4,     /* a pointer misses the alignment the call states    */
  FP4_ERR_ARCH = 5,      /* current device is not gfx950                      */
  FP4_ERR_WORKSPACE = 6, /* workspace missing or smaller than required        */
  FP4_ERR_HIP = 7,       /* a HIP runtime call or kernel launch failed        */
  FP4_ERR_ALIAS = 8      /* an output aliases an input the call reads         */
} fp4_status;

/* FP4_E4M3 (one FP8 E4M3 byte per value) is valid only as fp4_scaled_gemm's output. */
typedef enum { FP4_F32 = 0, FP4_BF16 = 1, FP4_E4M3 = 2 } fp4_dtype;
typedef enum { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;
typedef enum { FP4_RNE = 0, FP4_SR = 1 } fp4_rounding;

/* Bytes of workspace that nvfp4_quantize / hadamard_quantize need when the
 * global amax is computed on the device (amax_given == 0): per-workgroup
 * partial maxima of the first pass. */
#define FP4_AMAX_WORKSPACE_BYTES 4096

/* Size limits of the contractions.  The GEMM kernels address one 256-row tile
 * of an operand, and the GEMV one 16-row strip of W, with 32-bit byte offsets;
 * shapes beyond these return FP4_ERR_SHAPE before anything is launched.  The
 * quantizers, the dequantizer and the rotations index in 64 bits and have no
 * limit of their own. */
#define FP4_GEMM_MAX_MN (1LL << 30)           /* M, N (M_total) of the GEMMs */
#define FP4_GEMM_MAX_K ((1LL << 23) - 32)     /* K of the GEMMs */
#define FP4_GROUPED_MAX_GROUPS (1LL << 20)    /* num_groups of fp4_grouped_gemm */
#define FP4_GEMV_MAX_N (1LL << 30)
#define FP4_GEMV_MAX_K (1LL << 30)

/*
 * nvfp4_quantize -- two-level NVFP4 quantization of x [rows, cols].
 *
 * "low-precision floats" blog, section "FP4 / MXFP4 / NVFP4" (s_global and
 * s_block equations): s_global = amax / (6 * 448); per 16 values
 * s_block = (block_amax / 6) / s_global stored as FP8 E4M3; each value is
 * Q_E2M1(x / (s_global * s_block)).  NVIDIA "Introducing NVFP4" blog: one E4M3
 * scale per 16-value micro-block plus one FP32 scale per tensor.
 * Float32 operation order (exact contract, bit-identical to the CPU oracle):
 *   G = max|x| (or *global_amax when amax_given); s_global = G / 2688 (1 if G == 0)
 *   t = (A_b / 6) / s_global -> E4M3, nearest-even, saturating at 448, subnormals kept
 *   s_b = s_global * E4M3(t);  r_b = 1 / s_b (0 if s_b == 0)
 *   code_i = E2M1(x_i * r_b): nearest, ties to even, saturating at 6, sign of x_i kept
 *
 *  x            [rows, cols], FP4_F32 or FP4_BF16 (xt)
 *  q            out [rows, ceil(cols/2)] packed codes
 *  scales       out [rows, ceil(cols/16)] E4M3 bytes
 *  global_amax  amax_given != 0: read (static / calibrated amax, one float);
 *               amax_given == 0: written with the computed amax
 *  global_scale out, one float: s_global (the g_a / g_b of fp4_scaled_gemm)
 *  workspace    >= FP4_AMAX_WORKSPACE_BYTES bytes when amax_given == 0, else may be NULL
 * rows == 0 or cols == 0 writes G = 0 and s_global = 1 only.
 */
fp4_status nvfp4_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols,
                          uint8_t* q, uint8_t* scales, float* global_amax, int amax_given,
                          float* global_scale, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * nvfp4_quantize_no_workspace -- nvfp4_quantize without the workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The caller still owns
 * x, q, scales, global_amax and global_scale; with amax_given == 0 the first
 * pass writes its partial maxima into an array the library keeps on each device
 * it runs on (FP4_AMAX_WORKSPACE_BYTES, held until the process ends) instead of
 * a workspace.  The call allocates nothing and calls no allocating routine.
 * That array is shared by every call on a device and keeps the last call's
 * contents: calls that overlap on one device (concurrent streams, or host
 * threads enqueuing on different streams) race and must be serialized by the
 * caller.  Every size fits (the first pass uses at most 1024 workgroups, one
 * partial each, and writes every partial the second pass reads, so nothing has
 * to start at zero).  Arguments, outputs and errors as nvfp4_quantize, with a
 * failed lookup of the array returning FP4_ERR_HIP; the outputs are
 * bit-identical to nvfp4_quantize's.
 */
fp4_status nvfp4_quantize_no_workspace(const void* x, fp4_dtype xt, int64_t rows, int64_t cols,
                                       uint8_t* q, uint8_t* scales, float* global_amax,
                                       int amax_given, float* global_scale, hipStream_t stream);

/* Widest scale search of nvfp4_quantize_ex: +-126 codes covers every finite E4M3 byte. */
#define FP4_MAX_SCALE_SEARCH 126

/*
 * nvfp4_quantize_ex -- nvfp4_quantize with a choice of block size and of how the
 * E4M3 block scale is picked.
 *  block         8, 16 or 32 values per E4M3 scale along cols ("NVIDIA NVFP4 与
 *                Micro-Scaling" article, section 3.1 table: smaller blocks restore
 *                local range better at a higher scale overhead); scales is
 *                [rows, ceil(cols/block)].
 *  scale_search  0: the amax rule of nvfp4_quantize (code0 = E4M3(t)).  W > 0: the
 *                bytes code0 + d, d = -1, +1, -2, +2, ..., -W, +W inside 0..126, are
 *                tried in that order, and one replaces the current choice only when
 *                its float32 squared error is strictly smaller (NVIDIA "Introducing
 *                NVFP4" blog, 高精度缩放: the E4M3 scale can be the one that makes the
 *                block's summed error smallest).  The error of byte c, in float32
 *                with s_b = s_global * E4M3(c), r = 1 / s_b (0 if s_b == 0):
 *                  E = sum over the block, in index order, of (x_i - s_b * E2M1(x_i * r))^2
 *                each product, difference, square and sum rounded to float32.
 *                0 <= W <= FP4_MAX_SCALE_SEARCH.
 * Everything else (global amax, element encode, outputs, workspace) as
 * nvfp4_quantize; block 16 with scale_search 0 is nvfp4_quantize.  An invalid
 * block or scale_search returns FP4_ERR_SHAPE.
 */
fp4_status nvfp4_quantize_ex(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int block,
                             int scale_search, uint8_t* q, uint8_t* scales, float* global_amax,
                             int amax_given, float* global_scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_quantize -- MXFP4: E2M1 values with one E8M0 power-of-two scale per 32
 * values and no tensor scale (10100.com data-type article, "mxFP4的技术局限";
 * NVIDIA blog Table 1).  Scale = the smallest 2^e with 6 * 2^e >= block amax,
 * the rounded-up power of two of the "low-precision floats" blog (1.99 -> 2,
 * 2.01 -> 4); byte = clamp(e + 127, 0, 254), 0 for an all-zero block.
 * code_i = E2M1(x_i * 2^-e) (exact multiply).
 *  q       out [rows, ceil(cols/2)];  scales out [rows, ceil(cols/32)] E8M0 bytes
 */
fp4_status mxfp4_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols,
                          uint8_t* q, uint8_t* scales, hipStream_t stream);

/*
 * fp4_dequantize -- x_hat = s * v ("low-precision floats" blog: x_hat =
 * s_global * s_block * Q(.)).
 *  NVFP4: x_hat = (s_global * E4M3(byte)) * v in float32 (two roundings, the
 *         first product identical to the quantizer's s_b); global_scale is the
 *         device float written by nvfp4_quantize.
 *  MXFP4: x_hat = v * 2^(byte-127) (exact); global_scale must be NULL.
 *  y      out [rows, cols] float32, or bf16 rounded to nearest-even from the float32 value.
 */
fp4_status fp4_dequantize(fp4_format fmt, const uint8_t* q, const uint8_t* scales,
                          const float* global_scale, int64_t rows, int64_t cols,
                          void* y, fp4_dtype yt, hipStream_t stream);

/*
 * nvfp4_dequantize_ex -- fp4_dequantize of NVFP4 data written by
 * nvfp4_quantize_ex with blocks of `block` (8, 16 or 32) values: scales is
 * [rows, ceil(cols/block)].  An invalid block returns FP4_ERR_SHAPE.
 */
fp4_status nvfp4_dequantize_ex(const uint8_t* q, const uint8_t* scales, const float* global_scale,
                               int64_t rows, int64_t cols, int block, void* y, fp4_dtype yt,
                               hipStream_t stream);

/*
 * fp4_scaled_gemm -- D = g_d * ((g_a s_a . A) @ (g_b s_b . W)^T), fp32 accumulate.
 *
 * "NVIDIA NVFP4 与 Micro-Scaling" article, section 三 (scaled GEMM equation) and
 * section 五 (operand layouts A_fp4 [M, K/2], a_scale [M, K/16]; the concept API
 * passes W [N, K] as W.t()).  Both operands are K-major packed FP4:
 *   A [M, K/2], a_scales [M, K/bs];  W [N, K/2], w_scales [N, K/bs]
 * bs = 16 with E4M3 bytes (NVFP4) or 32 with E8M0 bytes (MXFP4).
 *   g_a, g_b  device floats: NVFP4 -> the global_scale written by nvfp4_quantize;
 *             MXFP4 -> must be NULL (tensor scale 1).
 *   g_d       host float output multiplier.
 *   D         out [M, N], float32, bf16 (nearest-even from the float32 result) or
 *             FP8 E4M3 bytes (FP4_E4M3): the sign of the float32 result, then its
 *             magnitude to the nearest E4M3 value, ties to the even code, saturating
 *             at 448 (section 五's scaled-mm example writes its output as
 *             float8_e4m3fn after g_d, fusing the next layer's input cast).
 * Each block product s_a * s_w * sum_k v_a v_w is exact; blocks are summed in
 * float32; |D - D_ref| <= 1e-5 * |g_d| * sum_k |A_hat_mk W_hat_nk| (+ one bf16
 * rounding for bf16 output).  K must be a multiple of bs (FP4_ERR_SHAPE);
 * A, W must be 16-byte aligned and K a multiple of 32 (FP4_ERR_ALIGN / SHAPE).
 * M == 0 or N == 0 is a no-op; K == 0 writes D = 0 without reading the operands.
 * M, N <= FP4_GEMM_MAX_MN and K <= FP4_GEMM_MAX_K, else FP4_ERR_SHAPE.
 */
fp4_status fp4_scaled_gemm(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                           const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                           const float* g_b, float g_d, int64_t M, int64_t N, int64_t K,
                           void* D, fp4_dtype dt, hipStream_t stream);

/*
 * fp4_scaled_gemm_nvfp4_out -- the same GEMM with its output requantized to
 * NVFP4 in the epilogue: the next layer's input quantization fused into this
 * layer's GEMM (article of fp4_scaled_gemm, section 三: the output is rescaled by
 * g_d and stored at low precision; section 五: the scales come from calibration).
 *   A .. g_d, M, N, K  as for fp4_scaled_gemm.
 *   d_amax    in: device float, the given (calibrated) tensor amax G of D; the
 *             tensor scale has to be known before any output block is encoded,
 *             so it is not computed from D.
 *   Dq        out [M, ceil(N/2)] packed E2M1 codes (low nibble first; for odd N
 *             the last high nibble is 0);
 *   d_scales  out [M, ceil(N/16)] E4M3 block-scale bytes, blocks of 16 along N
 *             (the last block partial when N % 16 != 0);
 *   d_global_scale out: device float s_global = G / 2688 (1 when G == 0), the g
 *             of D for the next GEMM.
 * Dq, d_scales and d_global_scale are exactly what nvfp4_quantize with
 * amax_given writes for the float32 result D = fl(acc * alpha) that
 * fp4_scaled_gemm produces for the same operands, bit for bit.  d_amax must not
 * alias d_global_scale (FP4_ERR_ALIAS).  M == 0 or N == 0 is a no-op; K == 0 encodes D = 0
 * (codes 0, scale bytes 0) without reading the operands.  Errors as for
 * fp4_scaled_gemm; NULL d_amax, d_scales or d_global_scale -> FP4_ERR_NULL.
 */
fp4_status fp4_scaled_gemm_nvfp4_out(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                                     const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                                     const float* g_b, float g_d, int64_t M, int64_t N, int64_t K,
                                     uint8_t* Dq, uint8_t* d_scales, const float* d_amax,
                                     float* d_global_scale, hipStream_t stream);

/*
 * fp4_grouped_gemm -- many GEMMs with one K and N in one launch, e.g. the expert
 * FFNs of a mixture-of-experts layer, whose weights the "NVIDIA NVFP4 与
 * Micro-Scaling" article (section 6.1) names as the first NVFP4 candidates.
 * Group e (0 <= e < num_groups) computes, as fp4_scaled_gemm does,
 *   D[r, :] = g_d * (A_hat[r, :] @ W_hat_e^T)   for r in [offsets[e], offsets[e+1])
 * where the rows of all groups are stored back to back (tokens sorted by group).
 *   A [M_total, K/2], a_scales [M_total, K/bs]; g_a one device float (NVFP4: the
 *       s_global of the whole A) or NULL (MXFP4);
 *   W [num_groups, N, K/2], w_scales [num_groups, N, K/bs]; g_b device floats
 *       [num_groups] (NVFP4: each group's s_global) or NULL (MXFP4);
 *   offsets  device int32 [num_groups + 1], non-decreasing, offsets[0] = 0,
 *       offsets[num_groups] = M_total.  Read on the device (no host sync, so the
 *       call can be captured in a graph).  Offsets outside that contract are
 *       clamped into [0, M_total]: no memory outside A, W and D is touched, but
 *       D is then unspecified;
 *   D  out [M_total, N], FP4_F32, FP4_BF16 or FP4_E4M3 (as fp4_scaled_gemm).
 * Each group's result equals fp4_scaled_gemm of its rows, bit for bit.  Rows
 * of D outside every group are not written.  num_groups >= 1; K % 32 == 0;
 * A, W 16-byte aligned.  M_total == 0 or N == 0 is a no-op; K == 0 writes D = 0.
 * M_total, N <= FP4_GEMM_MAX_MN, K <= FP4_GEMM_MAX_K, num_groups <=
 * FP4_GROUPED_MAX_GROUPS and (ceil(M_total/256) + num_groups) * ceil(N/256) <
 * 2^31 (the launch's tile bound), else FP4_ERR_SHAPE.
 */
fp4_status fp4_grouped_gemm(fp4_format fmt, const uint8_t* A, const uint8_t* a_scales,
                            const float* g_a, const uint8_t* W, const uint8_t* w_scales,
                            const float* g_b, float g_d, int64_t num_groups,
                            const int32_t* offsets, int64_t M_total, int64_t N, int64_t K,
                            void* D, fp4_dtype dt, hipStream_t stream);

/* Bytes of workspace fp4_gemv_batched needs for a batch of B rows of length K. */
size_t fp4_gemv_workspace_bytes(int64_t B, int64_t K);

/*
 * fp4_gemv_batched -- decode-time batched GEMV y = g_d * x_hat @ W_hat^T
 * (10100.com data-type article: "FP4 batch GEMV", written here from the scaled
 * GEMM of the ybb.press article, section 三).
 *   x   [B, K] float32 or bf16, quantized to NVFP4 on the fly with ONE dynamic
 *       tensor scale over all of [B, K], bit-identical to nvfp4_quantize;
 *   W   NVFP4 [N, K/2] + w_scales [N, K/16] + g_w (device float);
 *   y   out [B, N] float32 or bf16.  1 <= B <= 16, K % 32 == 0.
 *   workspace  >= fp4_gemv_workspace_bytes(B, K) bytes (holds quantized x).
 * N == 0 is a no-op; K == 0 writes y = 0 without reading x, W or the workspace.
 * x, W and workspace must be 16-byte aligned, w_scales 2-byte aligned (FP4_ERR_ALIGN).
 * N <= FP4_GEMV_MAX_N and K <= FP4_GEMV_MAX_K, else FP4_ERR_SHAPE.
 * Accuracy as for fp4_scaled_gemm.
 */
fp4_status fp4_gemv_batched(const void* x, fp4_dtype xt, int64_t B, const uint8_t* W,
                            const uint8_t* w_scales, const float* g_w, int64_t N, int64_t K,
                            float g_d, void* y, fp4_dtype yt, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * hadamard_quantize -- rotate every `group` (= 128) contiguous channels by the
 * orthonormal Walsh-Hadamard matrix, then NVFP4-quantize the rotated tensor
 * ("NVIDIA NVFP4 与 Micro-Scaling" article, section 4.1: x @ H with H H^T = I by
 * a fast Walsh-Hadamard transform; "FP4" wiki, 技術實現與量化方法: Hadamard
 * transform and stochastic rounding as NVFP4 quantization options).
 * Transform: Sylvester order, butterfly stages h = 1, 2, ..., 64 in float32
 * ((a, b) -> (a + b, a - b)), then one multiply by fl32(1/sqrt(128)).
 * The global amax is that of the rotated tensor (computed unless amax_given).
 *   mode FP4_RNE: as nvfp4_quantize.
 *   mode FP4_SR:  element codes rounded stochastically (scales stay nearest):
 *     for lo <= |q| < hi adjacent E2M1 magnitudes and f = (|q| - lo) / (hi - lo),
 *     round up iff floor(f * 2^22) + 64 * u16 >= 2^22 (probability
 *     floor(f * 2^16) / 2^16; |q| >= 6 gives 6), where u16 are 16 bits of
 *     Philox4x32-10 (Salmon et al., SC'11) with key (seed low, seed high) and
 *     counter (i/8 low, i/8 high, 0, 0) for flat element index i, taking word
 *     (i%8)/2, low half for even i%8, high half for odd.
 *   cols % group == 0; group must be 128.  x and q must be 16-byte aligned,
 *   scales 2-byte aligned (FP4_ERR_ALIGN).
 * Outputs and workspace as nvfp4_quantize.
 */
fp4_status hadamard_quantize(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                             fp4_rounding mode, uint64_t seed, uint8_t* q, uint8_t* scales,
                             float* global_amax, int amax_given, float* global_scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * hadamard_quantize_mx -- the rotation of hadamard_quantize, then MXFP4 as
 * mxfp4_quantize does (E8M0 per 32 rotated values, no tensor scale).  The
 * article of hadamard_quantize (section 4.1) rotates so that a block's absmax is
 * no longer set by one outlier channel; MXFP4's power-of-two block scales gain
 * from that, and the rotation can be absorbed into the adjacent layer's
 * weights: the GEMM of hadamard_quantize_mx(x) and hadamard_quantize_mx(W)
 * approximates x W^T, since (x H)(W H)^T = x W^T.
 *   mode FP4_SR: element codes of q = y * 2^-e rounded stochastically with the
 *   random bits of hadamard_quantize (same seed and element index -> same bits).
 *   q out [rows, cols/2]; scales out [rows, cols/32] E8M0 bytes.
 * One pass (no global amax, no workspace).  cols % group == 0, group == 128;
 * x and q 16-byte aligned (FP4_ERR_ALIGN).  rows == 0 or cols == 0 is a no-op.
 */
fp4_status hadamard_quantize_mx(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                                fp4_rounding mode, uint64_t seed, uint8_t* q, uint8_t* scales,
                                hipStream_t stream);

/*
 * hadamard_rotate -- y = x H for every `group` (= 128) contiguous channels,
 * the rotation of hadamard_quantize alone (same float32 steps), so that a
 * weight can be rotated once, offline, and stored (W H), or H absorbed into a
 * neighbouring layer (article of hadamard_quantize, section 4.1).
 *   x [rows, cols] FP4_F32 or FP4_BF16;  y out [rows, cols] FP4_F32 or FP4_BF16
 *   (nearest-even from the float32 result).  cols % group == 0, group == 128,
 *   x and y 16-byte aligned.  rows == 0 or cols == 0 is a no-op.
 */
fp4_status hadamard_rotate(const void* x, fp4_dtype xt, int64_t rows, int64_t cols, int group,
                           void* y, fp4_dtype yt, hipStream_t stream);

/* Human-readable text of a status (static storage). */
const char* fp4_status_string(fp4_status s);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char* fp4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
