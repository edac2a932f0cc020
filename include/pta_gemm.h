/*
 * libpta quantized GEMM operators (gfx950).
 *
 * The TACO-LLM pages list quantized GEMM operators next to the attention
 * kernels (17173xz.com article, section "TACO-LLM如何实现降本增效?": W4A8,
 * W4A16, W8A16 and W8A8 operators; 618zxw.cn article, section
 * "LLM量子化技術による推論コストの削減": weight-aware rearrangement, task
 * scheduling, fast dequantisation and integer scales for the GEMM and
 * attention operators; design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践",
 * section "5. 支持 Quantization（模型量化）": weights held as INT8/FP8 to cut
 * storage and bandwidth, run on low-precision matrix instructions).
 *
 * Computed (rounding aside), with A [M][K] the activations (one row per token)
 * and W [N][K] the weights (one row per output channel):
 *   W8A8:   Y[m][n] = a_scale[m] * w_scale[n] * sum_k A[m][k] * W[n][k],
 *           A and W OCP fp8 e4m3fn codes, scales float32.
 *   W4A16:  Y[m][n] = sum_k A[m][k] * q[n][k] * w_scale[n][k / group],
 *           A bf16, q signed 4-bit integers (-8..7), scales float32 per
 *           (output channel, group of `group` consecutive k).
 *   W8A16:  Y[m][n] = w_scale[n] * sum_k A[m][k] * W[n][k],
 *           A bf16, W fp8 e4m3fn codes, one float32 scale per output channel.
 *   W4A8:   Y[m][n] = a_scale[m] * sum_k A[m][k] * q[n][k] * w_scale[n][k / group],
 *           A signed 8-bit integers, q and w_scale as W4A16.
 * Y is bf16 [M][N] row-major, rounded to nearest even from float32.
 *
 * Conventions as in pta.h: device pointers, caller-owned buffers, work
 * enqueued asynchronously on `stream`, errors returned as pta_status before
 * any HIP call when they can be checked on the host.
 */
#ifndef PTA_GEMM_H
#define PTA_GEMM_H

#include <stddef.h>
#include <stdint.h>

#include "pta.h"

#ifdef __cplusplus
extern "C" {
#endif

/* fp8 x fp8 GEMM on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4),
 * float32 accumulation, per-row activation and per-output-channel weight
 * scales applied to the float32 sums.
 *   a        uint8 [M][K]  e4m3fn codes, row-major, 16-byte aligned
 *   a_scale  float [M]
 *   w        uint8 [N][K]  e4m3fn codes, row-major, 16-byte aligned
 *   w_scale  float [N]
 *   y        bf16  [M][N]  row-major (written; every element)
 * M >= 1, N >= 1, K a positive multiple of 64, M and N rounded up to multiples
 * of 256, each times K, below 2^32
 * (else PTA_ERR_BAD_DIMS); NULL pointers PTA_ERR_NULL_PTR; a failed launch
 * PTA_ERR_HIP.  NaN codes propagate to the affected outputs. */
pta_status taco_gemm_w8a8(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y,
                          int32_t M, int32_t N, int32_t K, void* stream);

/* bf16 x group-scaled int4 GEMM on the bf16 matrix cores
 * (v_mfma_f32_32x32x16_bf16).  Every int4 weight is converted exactly to bf16;
 * each group's products are summed in float32 and scaled by w_scale in
 * float32.
 *   a        bf16  [M][K]      row-major, 16-byte aligned
 *   w        uint8 [N][K / 2]  row-major, 16-byte aligned; byte j of a row holds
 *                              k = 2 j in its low nibble and k = 2 j + 1 in its
 *                              high nibble, two's complement
 *   w_scale  float [N][K / group], 4-byte aligned
 *   y        bf16  [M][N]      row-major (written; every element)
 * M >= 1, N >= 1, K a positive multiple of 64, group a multiple of 64 that
 * divides K; M rounded up to a multiple of 128 (64 when M <= 64) times 2 K,
 * N rounded up to a multiple of 128 times K / 2 and times 4 K / group, below
 * 2^32 (else PTA_ERR_BAD_DIMS); NULL pointers PTA_ERR_NULL_PTR; a failed launch
 * PTA_ERR_HIP.  NaN activations propagate to the affected outputs. */
pta_status taco_gemm_w4a16(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N,
                           int32_t K, int32_t group, void* stream);

/* Weight-aware rearrangement of W4A16 weights (the 618zxw.cn article, section
 * "LLM量子化技術による推論コストの削減", lists weight rearrangement among the
 * quantized operators' techniques): the int4 weights of taco_gemm_w4a16 laid
 * out in the GEMM's load order, so that each 64-k step of a 128-column tile is
 * one contiguous 4 KiB block (whole cache lines) instead of 32 bytes of each
 * of 128 rows.  Done once per weight matrix, outside the per-token path.
 *   taco_gemm_w4a16_tiled_bytes: size of the rearranged buffer for N x K
 *     weights (N rounded up to 128 columns, zero filled), 0 when N < 1, K is
 *     not a positive multiple of 64 or the size reaches 2^32.
 *   taco_gemm_w4a16_pack: w (row-major [N][K / 2], as taco_gemm_w4a16) into
 *     w_tiled (that many bytes, caller-allocated); both 16-byte aligned, else
 *     PTA_ERR_BAD_DIMS; bad N or K PTA_ERR_BAD_DIMS; NULL pointers
 *     PTA_ERR_NULL_PTR; asynchronous on stream.  Block (t, s) of w_tiled, at
 *     byte (t * K / 64 + s) * 4096, holds at byte 32 r + 16 p the 16 bytes of
 *     column 128 t + r at k-bytes 32 s + 16 (p ^ ((r >> 3) & 1)).
 *   taco_gemm_w4a16_tiled: taco_gemm_w4a16 on the rearranged weights (same
 *     arguments, limits, errors and results, bit for bit). */
size_t taco_gemm_w4a16_tiled_bytes(int32_t N, int32_t K);
pta_status taco_gemm_w4a16_pack(const void* w, void* w_tiled, int32_t N, int32_t K, void* stream);
pta_status taco_gemm_w4a16_tiled(const void* a, const void* w_tiled, const float* w_scale, void* y, int32_t M,
                                 int32_t N, int32_t K, int32_t group, void* stream);

/* bf16 x fp8 GEMM on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16): the
 * W8A16 operator the 17173xz.com article lists ("TACO-LLM如何实现降本增效?").
 * Every weight code is decoded exactly to bf16, the products are summed in
 * float32, and the channel scale multiplies the float32 sum.
 *   a        bf16  [M][K]  row-major, 16-byte aligned
 *   w        uint8 [N][K]  e4m3fn codes, row-major, 16-byte aligned
 *   w_scale  float [N], 4-byte aligned
 *   y        bf16  [M][N]  row-major (written; every element)
 * M >= 1, N >= 1, K a positive multiple of 64; M rounded up to a multiple of
 * 128 (64 when M <= 64) times 2 K, and N rounded up to a multiple of 128 times
 * K, below 2^32 (else PTA_ERR_BAD_DIMS); misaligned pointers PTA_ERR_BAD_DIMS;
 * NULL pointers PTA_ERR_NULL_PTR; a failed launch PTA_ERR_HIP.  NaN codes and
 * activations propagate to the affected outputs. */
pta_status taco_gemm_w8a16(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N,
                           int32_t K, void* stream);

/* Weight-aware rearrangement of W8A16 weights (as for W4A16 above): the fp8
 * codes of taco_gemm_w8a16 laid out in the GEMM's load order, so each 64-k
 * step of a 128-column tile is one contiguous 8 KiB block instead of 64 bytes
 * (half a cache line) of each of 128 rows.
 *   taco_gemm_w8a16_tiled_bytes: size of the rearranged buffer for N x K
 *     weights (N rounded up to 128 columns, zero filled), 0 when N < 1, K is
 *     not a positive multiple of 64 or the size reaches 2^32.
 *   taco_gemm_w8a16_pack: w (row-major [N][K]) into w_tiled (that many
 *     bytes, caller-allocated); both 16-byte aligned, else PTA_ERR_BAD_DIMS;
 *     bad N or K PTA_ERR_BAD_DIMS; NULL pointers PTA_ERR_NULL_PTR;
 *     asynchronous on stream.  Block (t, s) of w_tiled, at byte
 *     (t * K / 64 + s) * 8192, holds at byte 64 r + 16 p the 16 bytes of column
 *     128 t + r at k-bytes 64 s + 16 (p ^ ((r >> 2) & 3)).
 *   taco_gemm_w8a16_tiled: taco_gemm_w8a16 on the rearranged weights (same
 *     arguments, limits, errors and results, bit for bit). */
size_t taco_gemm_w8a16_tiled_bytes(int32_t N, int32_t K);
pta_status taco_gemm_w8a16_pack(const void* w, void* w_tiled, int32_t N, int32_t K, void* stream);
pta_status taco_gemm_w8a16_tiled(const void* a, const void* w_tiled, const float* w_scale, void* y, int32_t M,
                                 int32_t N, int32_t K, void* stream);

/* taco_gemm_w8a8 on weights rearranged by taco_gemm_w8a16_pack (the same fp8
 * codes and the same layout: each block is also the W8A8 kernels' image of a
 * 64-k stage of 128 columns).  Same arguments, limits, errors and results as
 * taco_gemm_w8a8, bit for bit; past 256 rows it runs the 64-k-step kernel
 * where taco_gemm_w8a8 runs the 128-k-step one (the sums are the same). */
pta_status taco_gemm_w8a8_tiled(const void* a, const float* a_scale, const void* w_tiled, const float* w_scale,
                                void* y, int32_t M, int32_t N, int32_t K, void* stream);

/* int8 x group-scaled int4 GEMM on the integer matrix cores
 * (v_mfma_i32_32x32x32_i8): the W4A8 operator the 17173xz.com article lists
 * ("TACO-LLM如何实现降本增效?"), with 8-bit integer activations (int4 weights
 * widen to int8 exactly).  Each group's products are summed exactly in int32,
 * scaled by w_scale in float32, and the float32 total multiplied by a_scale.
 *   a        int8  [M][K]      two's complement, row-major, 16-byte aligned
 *   a_scale  float [M], 4-byte aligned
 *   w        uint8 [N][K / 2]  as taco_gemm_w4a16 (low nibble = even k), 16-byte aligned
 *   w_scale  float [N][K / group], 4-byte aligned
 *   y        bf16  [M][N]      row-major (written; every element)
 * M >= 1, N >= 1, K a positive multiple of 64, group a multiple of 64 that
 * divides K; M rounded up to a multiple of 128 (64 when M <= 64) times K, N
 * rounded up to a multiple of 128 times K / 2 and times 4 K / group, below
 * 2^32 (else PTA_ERR_BAD_DIMS); misaligned pointers PTA_ERR_BAD_DIMS; NULL
 * pointers PTA_ERR_NULL_PTR; a failed launch PTA_ERR_HIP. */
pta_status taco_gemm_w4a8(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y,
                          int32_t M, int32_t N, int32_t K, int32_t group, void* stream);

/* taco_gemm_w4a8 on weights rearranged by taco_gemm_w4a16_pack (the same
 * nibble codes, so the same rearranged buffer serves both GEMMs): same
 * arguments, limits, errors and results, bit for bit. */
pta_status taco_gemm_w4a8_tiled(const void* a, const float* a_scale, const void* w_tiled, const float* w_scale,
                                void* y, int32_t M, int32_t N, int32_t K, int32_t group, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PTA_GEMM_H */
