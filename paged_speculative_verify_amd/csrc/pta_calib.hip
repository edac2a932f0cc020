// Measurement kernels (include/pta_calib.h): a streaming HBM read and a bf16
// matrix-core loop, the two ceilings the pages' roofline argument compares
// (design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践", section
// "TACO-LLM 如何解决大模型推理瓶颈?").
#include "../../include/pta_calib.h"
#include "pta_device.h"

using namespace pta;

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;                                   // 16-byte loads per lane in flight
constexpr int64_t kReadPiece = (int64_t)kReadThreads * kReadUnroll;   // 16-byte units per piece (16 KiB)

// Workgroup w reads pieces w, w + gridDim.x, ...; lane l of a piece reads
// units l, l + 256, l + 512, l + 768 (each load instruction covers 4 KiB
// contiguous across the workgroup).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kReadThreads) void calib_read_kernel(const u32x4* __restrict__ buf, int64_t pieces,
                                                                   uint32_t* sink) {
  uint32_t acc = 0;
  for (int64_t p = blockIdx.x; p < pieces; p += gridDim.x) {
    const u32x4* src = buf + p * kReadPiece + threadIdx.x;
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = __builtin_nontemporal_load(src + k * kReadThreads);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (acc == 0x9E3779B9u && (threadIdx.x & 63) == 0) sink[blockIdx.x] = acc;
}

// Four independent accumulation chains per wave so the matrix core never
// waits on a previous product; operands derive from the lane index so nothing
// folds at compile time.
__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    y[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, x, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, y, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

pta_status taco_pta_calib_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                      void* stream) {
  if (buf == nullptr || sink == nullptr) return PTA_ERR_NULL_PTR;
  if (bytes == 0 || bytes % (size_t)(kReadPiece * 16) != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
      workgroups < 1 || workgroups > 65535)
    return PTA_ERR_BAD_DIMS;
  const int64_t pieces = (int64_t)(bytes / (size_t)(kReadPiece * 16));
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const u32x4*>(buf), pieces, sink);
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

pta_status taco_pta_calib_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (sink == nullptr) return PTA_ERR_NULL_PTR;
  if (workgroups < 1 || workgroups > 65535 || iters < 1 || iters > (1 << 24)) return PTA_ERR_BAD_DIMS;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

}  // extern "C"
