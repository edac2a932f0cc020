/*
 * libpta measurement helpers: what this GPU actually delivers, measured with
 * kernels of this library, to put beside the published peaks.
 *
 * The pages judge an inference step by comparing the time its memory traffic
 * needs at the device's bandwidth with the time its arithmetic needs at the
 * device's peak (design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践",
 * section "TACO-LLM 如何解决大模型推理瓶颈?", the 10B-model example).  These
 * two calls measure both ceilings on the device at hand: a streaming read of
 * HBM and a bf16 matrix-core loop.  They are not part of the attention path.
 *
 * Conventions as in pta.h: device pointers, caller-owned buffers, work
 * enqueued asynchronously on `stream`, errors returned as pta_status.
 */
#ifndef PTA_CALIB_H
#define PTA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "pta.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf (device, 16-byte aligned, bytes a positive
 * multiple of 16 KiB) once with 16-byte vector loads: each workgroup of 256
 * lanes reads contiguous 16 KiB pieces in a grid-stride loop, four loads per
 * lane in flight.  workgroups in [1, 65535]; sink: device uint32[workgroups],
 * written only in the (practically impossible) case that the XOR of all data
 * read by a workgroup equals 0x9E3779B9, which keeps every load alive.
 * Errors: PTA_ERR_NULL_PTR, PTA_ERR_BAD_DIMS (size, alignment or workgroups),
 * PTA_ERR_HIP. */
pta_status taco_pta_calib_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                      void* stream);

/* bf16 matrix-core loop: every wave of `workgroups` workgroups of 4 waves
 * issues iters rounds of four independent v_mfma_f32_32x32x16_bf16 products
 * (32 * 32 * 16 * 2 = 32768 flops each), so a launch does
 * workgroups * 4 * iters * 4 * 32768 flops.  workgroups in [1, 65535],
 * iters in [1, 2^24]; sink: device float[workgroups], written only when the
 * accumulated sum is exactly 1234.5 (keeps the products alive).
 * Errors: PTA_ERR_NULL_PTR, PTA_ERR_BAD_DIMS, PTA_ERR_HIP. */
pta_status taco_pta_calib_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PTA_CALIB_H */
