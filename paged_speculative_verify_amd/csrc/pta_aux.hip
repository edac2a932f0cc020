// KV append and contract validation kernels.
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

// ---------------------------------------------------------------- KV append
// One wave per (token, KV head); slot = block * 16 + offset, negative = skip.
// Pages are filled as tokens arrive (design talk section
// "4. 支持 Paged Attention"); fp8 caches store RNE-saturated e4m3fn codes of
// x / scale with the block's own scale.
template <typename NT, typename KT>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int n = blockIdx.x, hk = blockIdx.y, lane = threadIdx.x;
  const int64_t slot = a.slots[n];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / kPage, off = slot % kPage;
  const int64_t src = ((int64_t)n * a.Hkv + hk) * a.D;
  const int64_t dst = ((blk * a.Hkv + hk) * kPage + off) * a.D;
  for (int which = 0; which < 2; ++which) {
    const void* in = which == 0 ? a.k_new : a.v_new;
    void* cache = which == 0 ? a.k_cache : a.v_cache;
    if constexpr (KT::bytes == 1) {
      const float scl = (which == 0 ? a.k_scale : a.v_scale)[blk * a.Hkv + hk];
      for (int d = lane; d < a.D; d += 64) {
        float x;
        if constexpr (NT::bytes == 4) x = reinterpret_cast<const float*>(in)[src + d];
        else x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(in)[src + d] << 16);
        reinterpret_cast<uint8_t*>(cache)[dst + d] = (uint8_t)f32_to_e4m3fn_sat(__fdiv_rn(x, scl));
      }
    } else {
      using S = typename KT::storage;
      for (int d = lane; d < a.D; d += 64)
        reinterpret_cast<S*>(cache)[dst + d] = reinterpret_cast<const S*>(in)[src + d];
    }
  }
}

hipError_t launch_append(const AppendArgs& p, int new_dtype, int kv_dtype, hipStream_t s) {
  const dim3 grid((unsigned)p.N, (unsigned)p.Hkv);
  if (p.N == 0) return hipSuccess;
  if (kv_dtype == 0 && new_dtype == 0) hipLaunchKernelGGL((append_kernel<F32, F32>), grid, dim3(64), 0, s, p);
  else if (kv_dtype == 1 && new_dtype == 1) hipLaunchKernelGGL((append_kernel<BF16, BF16>), grid, dim3(64), 0, s, p);
  else if (kv_dtype == 2 && new_dtype == 0) hipLaunchKernelGGL((append_kernel<F32, FP8>), grid, dim3(64), 0, s, p);
  else if (kv_dtype == 2 && new_dtype == 1) hipLaunchKernelGGL((append_kernel<BF16, FP8>), grid, dim3(64), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------- validation
__global__ __launch_bounds__(64) void clear_flag_kernel(int32_t* f) {
  if (threadIdx.x == 0) *f = 0;
}

__global__ __launch_bounds__(64) void validate_kernel(ValidateArgs v) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int C = v.ctx[b], q = v.qlen[b];
  int flags = 0;
  if (q < 1 || q > v.Qmax) flags |= 1;
  if (C < q || C > v.max_ctx) flags |= 2;
  if (C > v.page * v.MBS) flags |= 4;
  const int pages = min((max(C, 0) + v.page - 1) / v.page, v.MBS);
  for (int p = lane; p < pages; p += 64) {
    const int32_t blk = v.tables[(int64_t)b * v.MBS + p];
    if (blk < 0 || (int64_t)blk >= v.num_blocks) flags |= 8;
  }
  if (flags) atomicOr(v.flags, flags);
}

hipError_t launch_validate(const ValidateArgs& v, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(64), 0, s, v.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || v.B == 0) return e;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)v.B), dim3(64), 0, s, v);
  return hipGetLastError();
}

}  // namespace pta
