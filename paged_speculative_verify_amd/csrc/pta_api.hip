// C ABI of libpta: host-side argument checks, path selection and launches.
// All checks run before any HIP call; no allocation, no synchronisation.
#include "../../include/pta.h"
#include "pta_device.h"
#include "pta_launch.h"

#include <math.h>

using namespace pta;

namespace {

constexpr int kMaxQLen = 64;
constexpr int kPiecePad = 32;        // wide balanced grid: page-line padding per unit
constexpr int kValuMaxRows = 8;     // largest G * max_q_len of the vector-ALU path
constexpr int kMfmaMaxRows = 256;   // 8 waves x 32 rows
constexpr int kStreamMaxRows = 32;  // largest G * max_q_len of the streaming matrix-core path

bool dtype_ok(int q, int kv) {
  return (q == PTA_F32 && kv == PTA_F32) || (q == PTA_BF16 && (kv == PTA_BF16 || kv == PTA_FP8_E4M3FN));
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

pta_status check_dims(const pta_dims* d) {
  if (d == nullptr) return PTA_ERR_NULL_PTR;
  if (d->num_seqs < 0 || d->num_seqs > 65535 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_kv_heads > 65535 || d->num_q_heads % d->num_kv_heads != 0)
    return PTA_ERR_BAD_DIMS;
  if (d->head_dim != 64 && d->head_dim != 128) return PTA_ERR_BAD_DIMS;
  if (d->page_size != kPage) return PTA_ERR_BAD_DIMS;
  if (d->max_q_len < 1 || d->max_q_len > kMaxQLen) return PTA_ERR_BAD_DIMS;
  if (d->max_blocks_per_seq < 1 || d->max_ctx_len < 1 ||
      (int64_t)d->max_ctx_len > (int64_t)d->page_size * d->max_blocks_per_seq)
    return PTA_ERR_BAD_DIMS;
  if (d->num_blocks < 1) return PTA_ERR_BAD_DIMS;
  if ((d->flags & ~PTA_FLAG_SHARED_PAGES) != 0) return PTA_ERR_BAD_DIMS;
  if (!dtype_ok(d->q_dtype, d->kv_dtype)) return PTA_ERR_BAD_DTYPE;
  if (d->path < PTA_PATH_AUTO || d->path > PTA_PATH_TILE16) return PTA_ERR_BAD_DIMS;
  return PTA_OK;
}

// Kernel families:
//   VALU    vector-ALU page stream, any q dtype, rows per KV head <= 8
//   STREAM  matrix-core page stream (bf16 q), rows per KV head <= 32: each wave
//           walks its own pages with no barrier
//   TILE    matrix-core shared-tile kernel (bf16 q), rows per KV head <= 256:
//           one wave per 32 rows, K/V tiles shared through LDS
enum Family { FAM_VALU, FAM_STREAM, FAM_TILE };

struct Plan {
  Family fam;
  int rows_pow2;   // VALU
  int rb;          // STREAM: 16-row blocks
  int nw;          // STREAM / TILE: waves per workgroup
};

pta_status plan_for(const pta_dims* d, Plan* p) {
  const int G = d->num_q_heads / d->num_kv_heads;
  const int rows = G * d->max_q_len;
  const bool valu_ok = rows <= kValuMaxRows;
  const bool mfma_ok = d->q_dtype == PTA_BF16 && rows <= kMfmaMaxRows;
  bool mfma;
  p->rows_pow2 = pow2_at_least(rows);
  if (d->path == PTA_PATH_TILE || d->path == PTA_PATH_TILE16) {
    if (!mfma_ok) return PTA_ERR_UNSUPPORTED;
    p->fam = FAM_TILE;
    p->nw = max(2, pow2_at_least((rows + 31) / 32));
    return PTA_OK;
  }
  if (d->path == PTA_PATH_VALU) {
    if (!valu_ok) return PTA_ERR_UNSUPPORTED;
    mfma = false;
  } else if (d->path == PTA_PATH_MFMA) {
    if (!mfma_ok) return PTA_ERR_UNSUPPORTED;
    mfma = true;
  } else {
    if (mfma_ok) mfma = true;
    else if (valu_ok) mfma = false;
    else return PTA_ERR_UNSUPPORTED;
  }
  p->rows_pow2 = pow2_at_least(rows);
  if (!mfma) {
    p->fam = FAM_VALU;
    p->nw = 4;
  } else if (rows <= kStreamMaxRows) {
    p->fam = FAM_STREAM;
    p->rb = rows <= 16 ? 1 : 2;
    p->nw = 4;
  } else {
    p->fam = FAM_TILE;
    p->nw = pow2_at_least((rows + 31) / 32);     // 2, 4 or 8 waves of 32 rows
  }
  return PTA_OK;
}

pta_status check_attn_ptrs(const pta_dims* d, const void* q, const void* k, const void* v,
                           const float* ks, const float* vs, const int32_t* tables,
                           const int32_t* ctx, const int32_t* ql, const uint8_t* mask,
                           const void* out) {
  if (!q || !k || !v || !tables || !ctx || !ql || !out) return PTA_ERR_NULL_PTR;
  if (d->max_q_len > 1 && !mask) return PTA_ERR_NULL_PTR;
  if (d->kv_dtype == PTA_FP8_E4M3FN && (!ks || !vs)) return PTA_ERR_NULL_PTR;
  return PTA_OK;
}

AttnArgs make_args(const pta_dims* d, const void* q, const void* k, const void* v,
                   const float* ks, const float* vs, const int32_t* tables, const int32_t* ctx,
                   const int32_t* ql, const uint8_t* mask, float scale, void* out, float* lse) {
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.k_scale = ks; a.v_scale = vs;
  a.tables = tables; a.ctx = ctx; a.qlen = ql;
  a.mask = d->max_q_len > 1 ? mask : nullptr;
  a.out = out; a.lse = lse;
  a.scale_log2 = scale * kLog2e;
  a.B = d->num_seqs; a.Hq = d->num_q_heads; a.Hkv = d->num_kv_heads;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.Qmax = d->max_q_len; a.MBS = d->max_blocks_per_seq;
  a.num_blocks = d->num_blocks;
  a.stream_pages = (d->flags & PTA_FLAG_SHARED_PAGES) == 0;
  return a;
}

pta_status run_attn(const pta_dims* d, const AttnArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)a.num_parts, (unsigned)a.Hkv, (unsigned)a.B);
  hipError_t e;
  switch (p.fam) {
    case FAM_STREAM: e = launch_stream(a, d->kv_dtype, d->head_dim, p.rb, p.nw, grid, s); break;
    case FAM_TILE: e = launch_tile(a, d->kv_dtype, d->head_dim, p.nw, grid, s); break;
    default: e = launch_valu(a, d->q_dtype, d->kv_dtype, d->head_dim, p.rows_pow2, grid, s); break;
  }
  return e == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

struct SplitLayout {
  int64_t parts;
  size_t o_off, lse_off, total;
};

// Workspace: [counters int32 B*Hkv | partial O float B*Hq*Qmax*P*D | partial LSE float B*Hq*Qmax*P],
// each region 256-byte aligned.  Only the counters must be zero on entry; the call leaves them zero.
bool split_layout(const pta_dims* d, int32_t T, SplitLayout* L) {
  if (T <= 0 || T % 32 != 0) return false;
  L->parts = ((int64_t)d->max_ctx_len + T - 1) / T;
  const int64_t rows = (int64_t)d->num_seqs * d->num_q_heads * d->max_q_len * L->parts;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L->o_off = up((size_t)d->num_seqs * d->num_kv_heads * sizeof(int32_t));
  L->lse_off = L->o_off + up((size_t)rows * d->head_dim * sizeof(float));
  L->total = L->lse_off + up((size_t)rows * sizeof(float));
  return true;
}

// Balanced mode: [partial O float S*Mmax*D | partial LSE float S*Mmax]
// with Mmax = G * max_q_len rows per slot.
//   stream family: no counters, S = workgroups * nw + B*Hkv partial slots (one slice
//     per wave, nw = 4 waves per workgroup; a second launch merges).
//   tile family (bf16 KV): nw waves of 32 rows per workgroup (2 or 4), rg row groups per
//     slice, ns slices (a multiple of 8 with ns * rg workgroups fitting the device at
//     once); no counters (a second launch merges), S = ns + B*Hkv slots.
struct BalancedLayout {
  int nwg, nw, rg;
  size_t o_off, lse_off, total;
};


constexpr int kBalancedMaxSeqs = 16383;   // sequence page prefix lives in LDS

// The balanced shared-tile grid runs the 32x32x16-product kernel (pta_wide.hip)
// unless the caller holds it to the 16x16x32 one or a cache tensor is too large
// for its 32-bit buffer offsets (the tile past the last one must still be
// addressable: offsets stay below 2^32).
bool wide_tiles(const pta_dims* d) {
  const uint64_t tile = (uint64_t)kPage * (uint64_t)d->head_dim * 2u;
  return d->path != PTA_PATH_TILE16 &&
         (uint64_t)d->num_blocks * (uint64_t)d->num_kv_heads * tile + tile <= 0xFFFFFFFFull;
}

hipError_t balanced_tiles(const pta_dims* d, const AttnArgs* a, int nw, int* nwg, hipStream_t s) {
  return wide_tiles(d) ? wide_balanced(a, d->head_dim, nw, d->num_seqs, nwg, s)
                       : tile_balanced(a, d->head_dim, nw, d->num_seqs, nwg, s);
}

pta_status tile_balanced_layout(const pta_dims* d, BalancedLayout* L) {
  const int rows = (d->num_q_heads / d->num_kv_heads) * d->max_q_len;
  const int waves = (rows + 31) / 32;
  // at most 4 waves per row group: two 4-wave workgroups per compute unit overlap one's
  // barrier waits with the other's work (one 8-wave workgroup of 256 rows per compute
  // unit, which loads every page tile into LDS once, measured no faster on the widest tree)
  const int nw = waves <= 2 ? 2 : 4;
  const int rg = (waves + nw - 1) / nw;
  int fit = 0;
  if (balanced_tiles(d, nullptr, nw, &fit, nullptr) != hipSuccess) return PTA_ERR_HIP;
  const int ns = (fit / rg) & ~7;
  if (ns < 8) return PTA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)d->num_seqs * d->num_kv_heads;
  const int64_t slot_rows = ((int64_t)ns + units) * rows;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L->nwg = ns * rg;
  L->nw = nw;
  L->rg = rg;
  L->o_off = 0;
  L->lse_off = L->o_off + up((size_t)slot_rows * d->head_dim * sizeof(float));
  L->total = L->lse_off + up((size_t)slot_rows * sizeof(float));
  return PTA_OK;
}

pta_status balanced_layout(const pta_dims* d, const Plan& p, BalancedLayout* L) {
  if (d->num_seqs > kBalancedMaxSeqs) return PTA_ERR_UNSUPPORTED;
  if ((int64_t)d->num_seqs * d->max_blocks_per_seq >= ((int64_t)1 << 31)) return PTA_ERR_UNSUPPORTED;
  if ((int64_t)d->num_kv_heads * d->num_seqs * d->max_blocks_per_seq >= ((int64_t)1 << 31))
    return PTA_ERR_UNSUPPORTED;
  if (p.fam == FAM_TILE && d->kv_dtype == PTA_BF16) return tile_balanced_layout(d, L);
  if (p.fam != FAM_STREAM) return PTA_ERR_UNSUPPORTED;
  const int nw = 4;                                   // waves per workgroup, one slice each
  int nwg = 0;
  if (stream_balanced(nullptr, d->kv_dtype, d->head_dim, p.rb, nw, d->num_seqs, &nwg, nullptr) != hipSuccess)
    return PTA_ERR_HIP;
  const int64_t units = (int64_t)d->num_seqs * d->num_kv_heads;
  const int64_t slots = (int64_t)nwg * nw + units;
  const int64_t rows = slots * (d->num_q_heads / d->num_kv_heads) * d->max_q_len;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L->nwg = nwg;
  L->nw = nw;
  L->rg = 1;
  L->o_off = 0;
  L->lse_off = L->o_off + up((size_t)rows * d->head_dim * sizeof(float));
  L->total = L->lse_off + up((size_t)rows * sizeof(float));
  return PTA_OK;
}

// ---- allocation-free balanced entry: the workspace lives in this file-scope
// device array, one copy per GPU (each device that loads the library holds it
// until the process ends).  Host code never passes `scratch` itself to a
// kernel (its host-side name is only a handle): the device address of the
// current device's copy is looked up with hipGetSymbolAddress, once per device
// with that device current, and that pointer is what the kernels receive.
static __device__ __align__(256) char scratch[PTA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];     // device address of each device's copy, or null

pta_status scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PTA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return PTA_ERR_UNSUPPORTED;
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    // every thread that races here gets the same address, so storing it twice is harmless
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PTA_ERR_HIP;
    __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
  }
  *out = p;
  return PTA_OK;
}

// Balanced entry body: workspace from the caller, or (noalloc) this device's
// copy of `scratch`, whose size is the limit; k_new / v_new (bf16 rows) set by
// the fused-append entry, which only the 32x32x16 grid serves.
pta_status balanced_call(const pta_dims* d, const void* q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_tables,
                         const int32_t* ctx_lens, const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                         void* out, float* lse, void* workspace, size_t workspace_bytes, bool noalloc,
                         hipStream_t stream, const void* k_new = nullptr, const void* v_new = nullptr) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (!isfinite(scale)) return PTA_ERR_BAD_DIMS;
  Plan p;
  st = plan_for(d, &p);
  if (st != PTA_OK) return st;
  if (p.fam != FAM_STREAM && !(p.fam == FAM_TILE && d->kv_dtype == PTA_BF16)) return PTA_ERR_UNSUPPORTED;
  if (k_new != nullptr && !(p.fam == FAM_TILE && wide_tiles(d))) return PTA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0) return PTA_OK;
  st = check_attn_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                       tree_mask, out);
  if (st != PTA_OK) return st;
  if (!noalloc) {
    if (workspace == nullptr) return PTA_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PTA_ERR_BAD_DIMS;
  }
  BalancedLayout L;
  st = balanced_layout(d, p, &L);
  if (st != PTA_OK) return st;
  if (workspace_bytes < L.total) return PTA_ERR_WORKSPACE_TOO_SMALL;
  if (noalloc) {
    st = scratch_for_current_device(&workspace);
    if (st != PTA_OK) return st;
  }
  AttnArgs a = make_args(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                         tree_mask, scale, out, lse);
  a.k_new = k_new;
  a.v_new = v_new;
  // the wide grid's slices even out pages plus a fixed cost per unit piece (each piece
  // refills the copy pipeline and stores its rows, 12-14 us per extra piece measured on the
  // wide-tree calls; 32 pages of padding measured best of 8, 16, 32 and 48)
  a.slice_pad = p.fam == FAM_TILE && wide_tiles(d) ? kPiecePad : 0;
  char* ws = reinterpret_cast<char*>(workspace);
  a.counters = nullptr;                  // both balanced grids merge in a second launch
  a.part_o = reinterpret_cast<float*>(ws + L.o_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.lse_off);
  a.total_waves = L.nwg * L.nw;
  int nwg = L.nwg;
  if (p.fam == FAM_TILE) return balanced_tiles(d, &a, L.nw, &nwg, stream) == hipSuccess ? PTA_OK : PTA_ERR_HIP;
  return stream_balanced(&a, d->kv_dtype, d->head_dim, p.rb, L.nw, d->num_seqs, &nwg, stream) == hipSuccess
             ? PTA_OK
             : PTA_ERR_HIP;
}

}  // namespace

extern "C" {

pta_status taco_paged_tree_attn(const pta_dims* d, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* ctx_lens,
                                const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                                void* out, float* lse, void* stream) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (!isfinite(scale)) return PTA_ERR_BAD_DIMS;
  Plan p;
  st = plan_for(d, &p);
  if (st != PTA_OK) return st;
  if (d->num_seqs == 0) return PTA_OK;
  st = check_attn_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                       tree_mask, out);
  if (st != PTA_OK) return st;
  AttnArgs a = make_args(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                         tree_mask, scale, out, lse);
  a.part_tokens = 0;
  a.num_parts = 1;
  return run_attn(d, a, p, (hipStream_t)stream);
}

pta_status taco_paged_tree_attn_append(const pta_dims* d, const void* q, const void* k_new,
                                       const void* v_new, int32_t new_dtype, void* k_cache, void* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, const int32_t* ctx_lens,
                                       const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                                       void* out, float* lse, void* stream) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (!isfinite(scale)) return PTA_ERR_BAD_DIMS;
  if (d->kv_dtype == PTA_FP8_E4M3FN) {
    if (new_dtype != PTA_F32 && new_dtype != PTA_BF16) return PTA_ERR_BAD_DTYPE;
  } else if (new_dtype != d->kv_dtype) {
    return PTA_ERR_BAD_DTYPE;
  }
  Plan p;
  st = plan_for(d, &p);
  if (st != PTA_OK) return st;
  if (p.fam != FAM_STREAM) return PTA_ERR_UNSUPPORTED;   // fused into the stream kernel only
  if (d->num_seqs == 0) return PTA_OK;
  st = check_attn_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                       tree_mask, out);
  if (st != PTA_OK) return st;
  if (!k_new || !v_new) return PTA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % 16 != 0)
    return PTA_ERR_BAD_DIMS;                              // rows are moved in 16-byte chunks
  AttnArgs a = make_args(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                         tree_mask, scale, out, lse);
  a.part_tokens = 0;
  a.num_parts = 1;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_f32 = new_dtype == PTA_F32;
  return run_attn(d, a, p, (hipStream_t)stream);
}

size_t taco_paged_tree_attn_splitk_workspace_size(const pta_dims* d, int32_t partition_tokens) {
  if (check_dims(d) != PTA_OK) return 0;
  SplitLayout L;
  if (!split_layout(d, partition_tokens, &L)) return 0;
  return L.total;
}

pta_status taco_paged_tree_attn_splitk(const pta_dims* d, const void* q, const void* k_cache,
                                       const void* v_cache, const float* k_scale,
                                       const float* v_scale, const int32_t* block_tables,
                                       const int32_t* ctx_lens, const int32_t* q_lens,
                                       const uint8_t* tree_mask, float scale, void* out,
                                       float* lse, int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (!isfinite(scale)) return PTA_ERR_BAD_DIMS;
  SplitLayout L;
  if (!split_layout(d, partition_tokens, &L)) return PTA_ERR_BAD_DIMS;
  if (L.parts > 65535) return PTA_ERR_UNSUPPORTED;
  Plan p;
  st = plan_for(d, &p);
  if (st != PTA_OK) return st;
  if (d->num_seqs == 0) return PTA_OK;
  st = check_attn_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                       tree_mask, out);
  if (st != PTA_OK) return st;
  if (workspace == nullptr) return PTA_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PTA_ERR_BAD_DIMS;
  if (workspace_bytes < L.total) return PTA_ERR_WORKSPACE_TOO_SMALL;
  AttnArgs a = make_args(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                         tree_mask, scale, out, lse);
  char* ws = reinterpret_cast<char*>(workspace);
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.part_o = reinterpret_cast<float*>(ws + L.o_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.lse_off);
  a.part_tokens = partition_tokens;
  a.num_parts = (int32_t)L.parts;
  return run_attn(d, a, p, (hipStream_t)stream);
}

pta_status taco_paged_tree_attn_shared_prefix(const pta_dims* d, const void* q, const void* k_cache,
                                              const void* v_cache, const float* k_scale,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* ctx_lens, const int32_t* q_lens,
                                              const uint8_t* tree_mask, const int32_t* prefix_leader,
                                              int32_t max_group, int32_t shared_tokens, float scale,
                                              void* out, float* lse, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (!isfinite(scale)) return PTA_ERR_BAD_DIMS;
  if (max_group < 1) return PTA_ERR_BAD_DIMS;
  SplitLayout L;
  if (!split_layout(d, shared_tokens, &L)) return PTA_ERR_BAD_DIMS;
  if (L.parts > 65535) return PTA_ERR_UNSUPPORTED;
  Plan p;
  st = plan_for(d, &p);
  if (st != PTA_OK) return st;
  // the group's rows share one matrix-core stream unit of up to 32 rows
  const int G = d->num_q_heads / d->num_kv_heads;
  if (p.fam != FAM_STREAM || (int64_t)max_group * G * d->max_q_len > kStreamMaxRows) return PTA_ERR_UNSUPPORTED;
  p.rb = 2;
  if (d->num_seqs == 0) return PTA_OK;
  st = check_attn_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                       tree_mask, out);
  if (st != PTA_OK) return st;
  if (prefix_leader == nullptr || workspace == nullptr) return PTA_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PTA_ERR_BAD_DIMS;
  if (workspace_bytes < L.total) return PTA_ERR_WORKSPACE_TOO_SMALL;
  AttnArgs a = make_args(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens,
                         tree_mask, scale, out, lse);
  char* ws = reinterpret_cast<char*>(workspace);
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.part_o = reinterpret_cast<float*>(ws + L.o_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.lse_off);
  a.part_tokens = shared_tokens;
  a.num_parts = (int32_t)L.parts;
  a.prefix_leader = prefix_leader;
  a.max_group = max_group;
  return run_attn(d, a, p, (hipStream_t)stream);
}

size_t taco_paged_tree_attn_balanced_workspace_size(const pta_dims* d) {
  if (check_dims(d) != PTA_OK) return 0;
  Plan p;
  if (plan_for(d, &p) != PTA_OK) return 0;
  BalancedLayout L;
  if (balanced_layout(d, p, &L) != PTA_OK) return 0;
  return L.total;
}

pta_status taco_paged_tree_attn_balanced(const pta_dims* d, const void* q, const void* k_cache,
                                         const void* v_cache, const float* k_scale,
                                         const float* v_scale, const int32_t* block_tables,
                                         const int32_t* ctx_lens, const int32_t* q_lens,
                                         const uint8_t* tree_mask, float scale, void* out, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return balanced_call(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens, tree_mask, scale,
                       out, lse, workspace, workspace_bytes, false, (hipStream_t)stream);
}

pta_status taco_paged_tree_attn_balanced_append(const pta_dims* d, const void* q, const void* k_new,
                                                const void* v_new, int32_t new_dtype, void* k_cache, void* v_cache,
                                                const int32_t* block_tables, const int32_t* ctx_lens,
                                                const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  if (d == nullptr) return PTA_ERR_NULL_PTR;
  if (new_dtype != PTA_BF16) return PTA_ERR_BAD_DTYPE;   // rows in the cache's dtype (bf16 caches only)
  if (!k_new || !v_new) return PTA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % 16 != 0)
    return PTA_ERR_BAD_DIMS;                              // rows are moved in 16-byte chunks
  return balanced_call(d, q, k_cache, v_cache, nullptr, nullptr, block_tables, ctx_lens, q_lens, tree_mask, scale,
                       out, lse, workspace, workspace_bytes, false, (hipStream_t)stream, k_new, v_new);
}

pta_status taco_paged_tree_attn_balanced_noalloc(const pta_dims* d, const void* q, const void* k_cache,
                                                 const void* v_cache, const float* k_scale,
                                                 const float* v_scale, const int32_t* block_tables,
                                                 const int32_t* ctx_lens, const int32_t* q_lens,
                                                 const uint8_t* tree_mask, float scale, void* out, float* lse,
                                                 void* stream) {
  return balanced_call(d, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, q_lens, tree_mask, scale,
                       out, lse, nullptr, PTA_NOALLOC_SCRATCH_BYTES, true, (hipStream_t)stream);
}

pta_status taco_kv_append(const pta_dims* d, const void* k_new, const void* v_new,
                          int32_t new_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                          void* k_cache, void* v_cache, const float* k_scale,
                          const float* v_scale, void* stream) {
  if (d == nullptr) return PTA_ERR_NULL_PTR;
  if (d->num_kv_heads < 1 || d->num_kv_heads > 65535 || (d->head_dim != 64 && d->head_dim != 128) || d->page_size != kPage ||
      d->num_blocks < 1 || num_tokens < 0 || num_tokens > 65535 * 64)
    return PTA_ERR_BAD_DIMS;
  const int kv = d->kv_dtype;
  const bool ok = (kv == PTA_F32 && new_dtype == PTA_F32) || (kv == PTA_BF16 && new_dtype == PTA_BF16) ||
                  (kv == PTA_FP8_E4M3FN && (new_dtype == PTA_F32 || new_dtype == PTA_BF16));
  if (!ok) return PTA_ERR_BAD_DTYPE;
  if (num_tokens == 0) return PTA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PTA_ERR_NULL_PTR;
  if (kv == PTA_FP8_E4M3FN && (!k_scale || !v_scale)) return PTA_ERR_NULL_PTR;
  AppendArgs p{};
  p.k_new = k_new; p.v_new = v_new; p.slots = slot_mapping;
  p.k_cache = k_cache; p.v_cache = v_cache; p.k_scale = k_scale; p.v_scale = v_scale;
  p.N = num_tokens; p.Hkv = d->num_kv_heads; p.D = d->head_dim;
  p.num_slots = d->num_blocks * kPage;
  return launch_append(p, new_dtype, kv, (hipStream_t)stream) == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

pta_status taco_accept_commit(const pta_dims* d, const int32_t* cand_tokens, const int32_t* target_tokens,
                              const int32_t* target_prev, const int32_t* ctx_lens, const int32_t* q_lens,
                              const uint8_t* tree_mask, const int32_t* block_tables, void* k_cache,
                              void* v_cache, const float* k_scale, const float* v_scale, int32_t* n_accepted,
                              int32_t* accepted_path, int32_t* bonus_tokens, int32_t* new_ctx_lens,
                              void* stream) {
  pta_status st = check_dims(d);
  if (st != PTA_OK) return st;
  if (d->kv_dtype != PTA_F32 && d->kv_dtype != PTA_BF16 && d->kv_dtype != PTA_FP8_E4M3FN) return PTA_ERR_BAD_DTYPE;
  if (d->num_seqs == 0) return PTA_OK;
  if (!cand_tokens || !target_tokens || !target_prev || !ctx_lens || !q_lens || !block_tables || !k_cache ||
      !v_cache || !n_accepted || !accepted_path || !bonus_tokens || !new_ctx_lens)
    return PTA_ERR_NULL_PTR;
  if (d->max_q_len > 1 && !tree_mask) return PTA_ERR_NULL_PTR;
  if (d->kv_dtype == PTA_FP8_E4M3FN && (!k_scale || !v_scale)) return PTA_ERR_NULL_PTR;
  AcceptArgs p{};
  p.ctx = ctx_lens;
  p.qlen = q_lens;
  p.mask = d->max_q_len > 1 ? tree_mask : nullptr;
  p.cand = cand_tokens;
  p.target = target_tokens;
  p.target_prev = target_prev;
  p.tables = block_tables;
  p.k = k_cache;
  p.v = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.n_acc = n_accepted;
  p.path = accepted_path;
  p.bonus = bonus_tokens;
  p.new_ctx = new_ctx_lens;
  p.B = d->num_seqs;
  p.Hkv = d->num_kv_heads;
  p.D = d->head_dim;
  p.Qmax = d->max_q_len;
  p.MBS = d->max_blocks_per_seq;
  return launch_accept(p, d->kv_dtype, (hipStream_t)stream) == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

pta_status taco_pta_validate(const pta_dims* d, const int32_t* block_tables, const int32_t* ctx_lens,
                             const int32_t* q_lens, int32_t* d_flags, void* stream) {
  if (d == nullptr) return PTA_ERR_NULL_PTR;
  if (d->num_seqs < 0 || d->max_q_len < 1 || d->max_blocks_per_seq < 1 || d->page_size != kPage ||
      d->num_blocks < 1)
    return PTA_ERR_BAD_DIMS;
  if (!d_flags) return PTA_ERR_NULL_PTR;
  if (d->num_seqs > 0 && (!block_tables || !ctx_lens || !q_lens)) return PTA_ERR_NULL_PTR;
  ValidateArgs v{};
  v.tables = block_tables; v.ctx = ctx_lens; v.qlen = q_lens; v.flags = d_flags;
  v.B = d->num_seqs; v.Qmax = d->max_q_len; v.MBS = d->max_blocks_per_seq;
  v.max_ctx = d->max_ctx_len; v.page = d->page_size; v.num_blocks = d->num_blocks;
  return launch_validate(v, (hipStream_t)stream) == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

const char* taco_pta_status_string(pta_status s) {
  switch (s) {
    case PTA_OK: return "ok";
    case PTA_ERR_NULL_PTR: return "a required pointer is NULL";
    case PTA_ERR_BAD_DIMS: return "invalid or inconsistent dimensions";
    case PTA_ERR_BAD_DTYPE: return "unsupported dtype or dtype combination";
    case PTA_ERR_UNSUPPORTED: return "request not supported by the built kernels";
    case PTA_ERR_WORKSPACE_TOO_SMALL: return "split-K workspace too small";
    case PTA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t taco_pta_version(void) { return 100; }

}  // extern "C"
