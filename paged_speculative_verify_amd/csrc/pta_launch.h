// Internal launch entry points of the kernel files (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pta {

struct AttnArgs;

// dtype codes follow pta_dtype: 0 f32, 1 bf16, 2 fp8 e4m3fn
hipError_t launch_valu(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int rows_pow2,
                       dim3 grid, hipStream_t s);
hipError_t launch_stream(const AttnArgs& a, int kv_dtype, int head_dim, int rb, int nw, dim3 grid,
                         hipStream_t s);
// Persistent work-balanced matrix-core stream kernel (rows per KV head <= 32):
// workgroups of nw = 4 waves, one page slice per wave.  With a == nullptr, *nwg
// receives the grid size (workgroups) for the current device; otherwise *nwg
// workgroups are launched.
hipError_t stream_balanced(const AttnArgs* a, int kv_dtype, int head_dim, int rb, int nw, int B, int* nwg,
                           hipStream_t s);
// Matrix-core shared-tile kernel (rows per KV head 33..256): nwr waves of 32 rows.
hipError_t launch_tile(const AttnArgs& a, int kv_dtype, int head_dim, int nwr, dim3 grid, hipStream_t s);
// Persistent work-balanced shared-tile kernel (bf16 KV, rows per KV head
// 33..256): workgroups of nwr in {2, 4} waves, ceil(rows / (32 nwr)) row groups
// per slice.  With a == nullptr, *nwg receives the workgroups that fit the
// device at once; otherwise *nwg workgroups are launched.
hipError_t tile_balanced(const AttnArgs* a, int head_dim, int nwr, int B, int* nwg, hipStream_t s);
// The same grid with the 32x32x16-product pipeline (pta_wide.hip), nwr in
// {2, 4, 8}; needs every bf16 cache tensor below 4 GiB (32-bit buffer offsets).
hipError_t wide_balanced(const AttnArgs* a, int head_dim, int nwr, int B, int* nwg, hipStream_t s);
// Second launch of both balanced grids: merge of the slice partials (bf16 out),
// NS = slices of the attention launch.
hipError_t launch_slice_merge(const AttnArgs& a, int head_dim, int NS, hipStream_t s);

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  const float* k_scale;
  const float* v_scale;
  int32_t N, Hkv, D;
  int64_t num_slots;        // num_blocks * page_size
};
hipError_t launch_append(const AppendArgs& p, int new_dtype, int kv_dtype, hipStream_t s);

struct AcceptArgs {
  const int32_t* ctx;
  const int32_t* qlen;
  const uint8_t* mask;
  const int32_t* cand;
  const int32_t* target;
  const int32_t* target_prev;
  const int32_t* tables;
  void* k;
  void* v;
  const float* k_scale;
  const float* v_scale;
  int32_t* n_acc;
  int32_t* path;
  int32_t* bonus;
  int32_t* new_ctx;
  int32_t B, Hkv, D, Qmax, MBS;
};
hipError_t launch_accept(const AcceptArgs& p, int kv_dtype, hipStream_t s);

struct ValidateArgs {
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* qlen;
  int32_t* flags;
  int32_t B, Qmax, MBS, max_ctx, page;
  int64_t num_blocks;
};
hipError_t launch_validate(const ValidateArgs& v, hipStream_t s);

}  // namespace pta
