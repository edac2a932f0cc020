// Matrix-core paged tree attention for many rows per KV head (33 to 256: the
// GQA group's q-heads times a candidate tree of up to 64 nodes).  Lookahead
// verification turns each sequence's decode GEMV into a real GEMM (TACO-LLM
// design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践", TurboAttention
// bullets of "整体方案分为两大部分": tensor-core use once vector-matrix work
// becomes matrix-matrix work).
//
// gfx950 design:
//   * Work unit = (sequence, KV head, token partition).  The workgroup has one
//     wave per 32 query rows (two 16-row MFMA blocks); every wave needs every
//     KV tile, so tiles are loaded once per workgroup into LDS and shared.
//   * A stage is two 16-token pages.  The stage's K and V page tiles are cut
//     into 1 KiB chunks, each read by one load instruction of one wave
//     (lane l: bytes 16 l + 1024 j, contiguous), with the block-table entries
//     read as wave-uniform scalars.  fp8 chunks are decoded to bf16 on the way
//     into LDS (exact; per-page scales folded into the scores and into P).
//   * Two stages ahead are issued into registers while the current stage is
//     computed from LDS; the next stage is written to the other LDS buffer
//     afterwards: one barrier per stage, a full stage of loads always in
//     flight.
//   * Per stage each wave runs the shared two-page flash update
//     (pair_compute, pta_flash.h): S^T = K Q^T with v_mfma_f32_16x16x32_bf16
//     (K read from LDS with ds_read_b128), masked online softmax with lazy
//     rescaling, then one 32-token O^T += V^T P^T step, again with the
//     full-rate v_mfma_f32_16x16x32_bf16 and ds_read_b64_tr_b16 for V^T.
//   * Rows are split across waves, not tokens, so the epilogue needs no
//     cross-wave merge; split-K partials merge in the last unit to arrive.
#include "pta_device.h"
#include "pta_flash.h"
#include "pta_launch.h"

namespace pta {

template <typename KT, int D>
struct TileStage {
  static constexpr int TILE_BYTES = kPage * D * KT::bytes;   // one page tile in HBM
  static constexpr int CPT = TILE_BYTES / 1024;              // 1 KiB chunks per page tile
  static constexpr int CHUNKS = 4 * CPT;                     // K page 0, K page 1, V page 0, V page 1
  static constexpr int TILE_LDS = StreamTile<KT, D>::TILE_LDS;
  static constexpr int STAGE_LDS = 4 * TILE_LDS;
};

template <typename KT, int D, int NWR>
__global__ __launch_bounds__(NWR * 64) void tile_attn_kernel(AttnArgs a) {
  constexpr int RB = 2;                                      // 32 rows per wave
  using T = TileStage<KT, D>;
  constexpr int CPW = (T::CHUNKS + NWR - 1) / NWR;           // chunks per wave per stage
  __shared__ __attribute__((aligned(16))) char lds[2][T::STAGE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  const int L = C - qb;
  const int M = a.G * qb;
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;           // partition past this sequence's context
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly

  StreamRows<D, RB> rows;
  load_rows(rows, a, b, hkv, qb, M, g, m, wave * 32);
  StreamState<D, RB> st;
  st.init();
  const bool wave_rows = wave * 32 < M;

  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int pgA = t0 / kPage;
  const int npg = (t1 + kPage - 1) / kPage - pgA;
  const int nst = (npg + 1) / 2;

  // stage s holds pages pgA + 2 s and, if it exists, pgA + 2 s + 1; wave w
  // moves chunks c = (w + i * NWR) mod CHUNKS (tile c / CPT, chunk c % CPT).
  // No branch guards the loads (a guarded load would make the compiler wait
  // for every outstanding load at the join); when NWR does not divide the
  // chunk count, surplus waves move a duplicate chunk, writing identical data.
  auto chunk_of = [&](int i) -> int {
    const int c = wave + i * NWR;
    if constexpr (T::CHUNKS % NWR == 0) return c;
    else return c % T::CHUNKS;
  };
  struct Scales { float k0, v0, k1, v1; };
  struct StageRegs {
    uint4 c[CPW];
    Scales sc;
  };
  auto issue = [&](StageRegs& R, int s) {
    const int p0 = pgA + 2 * s;
    const bool has1 = 2 * s + 1 < npg;
    const int64_t ph0 = table[p0];
    const int64_t ph1 = has1 ? (int64_t)table[p0 + 1] : ph0;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = chunk_of(i);
      const int tile = c / T::CPT, j = c % T::CPT;
      const int64_t ph = (tile & 1) ? ph1 : ph0;
      const char* base = (tile < 2 ? kbase : vbase) + (ph * a.Hkv + hkv) * T::TILE_BYTES;
      R.c[i] = *reinterpret_cast<const uint4*>(base + 1024 * j + 16 * lane);
    }
    if constexpr (KT::bytes == 1) {
      R.sc.k0 = a.k_scale[ph0 * a.Hkv + hkv];
      R.sc.v0 = a.v_scale[ph0 * a.Hkv + hkv];
      R.sc.k1 = a.k_scale[ph1 * a.Hkv + hkv];
      R.sc.v1 = a.v_scale[ph1 * a.Hkv + hkv];
    } else {
      R.sc = Scales{1.f, 1.f, 1.f, 1.f};
    }
  };
  auto write = [&](const StageRegs& R, int s, int buf) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = chunk_of(i);
      const int tile = c / T::CPT, j = c % T::CPT;
      const int pbase = (pgA + 2 * s + (tile & 1)) * kPage;
      // V rows past t1 are zeroed; K rows past t1 are masked out of the scores
      const bool partial = tile >= 2 && pbase + kPage > t1;
      stage_chunk<KT, D>(lds[buf] + tile * T::TILE_LDS, R.c[i], j, lane, partial, t1 - pbase);
    }
  };
  auto compute = [&](int s, int buf, const Scales& sc) {
    if (!wave_rows) return;
    const char* kl = lds[buf];
    const float cs = a.scale_log2;
    // a missing second page has its V tile zeroed and its tokens past t1
    pair_compute<D, RB>(rows, st, kl, kl + T::TILE_LDS, kl + 2 * T::TILE_LDS, kl + 3 * T::TILE_LDS,
                        (pgA + 2 * s) * kPage, L, t1, cs * sc.k0, cs * sc.k1, sc.v0, sc.v1, lane);
  };

  // Pipeline: LDS buffer s & 1 holds stage s while stage s + 1 sits in
  // registers and stage s + 2 is being loaded (register set s & 1), so a full
  // stage of loads is always in flight.  Prefetches are unconditional (past
  // the end they re-read the final stage, still in cache), which keeps the
  // compiler's load counters exact.  One barrier per stage.
  if (nst > 0) {
    StageRegs r0, r1;
    issue(r0, 0);
    issue(r1, min(1, nst - 1));
    write(r0, 0, 0);
    Scales sc_cur = r0.sc;
    __syncthreads();
    for (int s = 0;; s += 2) {
      issue(r0, min(s + 2, nst - 1));
      compute(s, 0, sc_cur);
      if (s + 1 >= nst) break;
      write(r1, s + 1, 1);
      sc_cur = r1.sc;
      __syncthreads();
      issue(r1, min(s + 3, nst - 1));
      compute(s + 1, 1, sc_cur);
      if (s + 2 >= nst) break;
      write(r0, s + 2, 0);
      sc_cur = r0.sc;
      __syncthreads();
    }
  }

  // ---- epilogue: each wave owns its rows outright
  reduce_row_sums(st);
  if (split_out) {
    auto addr = [&](int rb, float*& o, float*& l) {
      const int64_t prow = (((int64_t)b * a.Hq + rows.h[rb]) * a.Qmax + rows.i[rb]) * a.num_parts + part;
      o = a.part_o + prow * D;
      l = a.part_lse + prow;
    };
    store_partial_rows(rows, st, g, addr);
    splitk_finish<BF16, D>(a, b, hkv, C, qb);
  } else {
    store_final_rows(a, rows, st, b, g);
  }
}

// ============================================================ bf16 cache: direct-to-LDS
// bf16 page tiles need no conversion, so they go from HBM straight into LDS
// with global_load_lds_dwordx4 (gfx950: 16 bytes per lane, the wave's 64
// lanes fill 1 KiB of LDS at M0 + 16 * lane): no register staging, no VGPR
// cost for bytes in flight.  Three LDS stage buffers give two stages of loads
// in flight while one is computed, with one barrier per stage.
//
// The copies are issued with inline asm so that the compiler, which would
// otherwise wait for every outstanding copy before any LDS read, leaves the
// waits to the kernel: before the barrier that opens stage s a wave waits
// until only its copies of stage s + 1 remain in flight (vector memory
// operations complete in issue order, so any compiler-issued load only makes
// these waits longer, never too short).
//
// Tiles are unpadded (a copy writes 1 KiB contiguous) and swizzled: lane l
// of chunk j fetches 16-byte unit (l % UPR) ^ (row & (UPR - 1)) of row
// RPC j + l / UPR, so that tile_off<D, true> finds every unit and the
// row-strided operand reads spread over the LDS banks.
__device__ __forceinline__ void lds_copy16(uint32_t lds_addr, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_addr), "v"(gptr)
               : "memory", "m0");
}

// Two block-table entries through the scalar cache. The copies above are
// opaque to the compiler, so a table read it schedules as a vector load would
// be followed by a wait for every copy in flight; a scalar read waits only
// for itself.
__device__ __forceinline__ void scalar_pair(const int32_t* p0, const int32_t* p1, int& x0, int& x1) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(x0), "=&s"(x1) : "s"(p0), "s"(p1));
}

template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D, int NWR>
__global__ __launch_bounds__(NWR * 64) void tile_dma_kernel(AttnArgs a) {
  constexpr int RB = 2;
  constexpr int TILE = kPage * D * 2;                        // bf16 page tile, HBM and LDS
  constexpr int CPT = TILE / 1024;                           // 1 KiB copies per tile
  constexpr int CHUNKS = 4 * CPT;                            // K page 0, K page 1, V page 0, V page 1
  constexpr int CPW = (CHUNKS + NWR - 1) / NWR;              // copies per wave per stage
  constexpr int STAGE = 4 * TILE;
  constexpr int NBUF = 3;
  constexpr int UPR = 2 * D / 16;                            // 16-byte units per row
  constexpr int RPC = 1024 / (2 * D);                        // rows per copy
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  const int L = C - qb;
  const int M = a.G * qb;
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;           // partition past this sequence's context
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly

  StreamState<D, RB> st;
  st.init();
  const bool wave_rows = wave * 32 < M;

  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int pgA = t0 / kPage;
  const int npg = (t1 + kPage - 1) / kPage - pgA;
  const int nst = (npg + 1) / 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0][0];

  // this lane's slot in a copy: row RPC j + l / UPR, unit l % UPR, fetched from
  // the swizzled unit of the global row
  const int crow = lane / UPR, cunit = lane % UPR;
  auto copy_stage = [&](int s) {
    const int p0 = pgA + 2 * s;
    const bool has1 = 2 * s + 1 < npg;
    const int i1 = __builtin_amdgcn_readfirstlane(has1 ? p0 + 1 : p0);
    int x0, x1;
    scalar_pair(table + __builtin_amdgcn_readfirstlane(p0), table + i1, x0, x1);
    const int64_t ph0 = x0, ph1 = x1;
    const uint32_t dst = lds0 + (uint32_t)((s % NBUF) * STAGE);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      int c = wave + i * NWR;
      if constexpr (CHUNKS % NWR != 0) c %= CHUNKS;        // surplus waves repeat a copy
      const int tile = c / CPT, j = c % CPT;
      const int64_t ph = (tile & 1) ? ph1 : ph0;
      const int r = RPC * j + crow;
      const char* src = (tile < 2 ? kbase : vbase) + (ph * a.Hkv + hkv) * TILE + r * 2 * D +
                        ((cunit ^ (r & (UPR - 1))) << 4);
      lds_copy16(dst + (uint32_t)(tile * TILE + 1024 * j), src);
    }
  };

  // The query rows load behind the first two stages and everything lands
  // before the loop, so no wait on the query registers sits inside it.
  if (nst > 0) copy_stage(0);
  if (nst > 1) copy_stage(1);
  StreamRows<D, RB> rows;
  load_rows(rows, a, b, hkv, qb, M, g, m, wave * 32);
  wait_vmem_at_most<0>();
  if (nst > 0) {
    for (int s = 0; s < nst; ++s) {
      if (s + 1 < nst) wait_vmem_at_most<CPW>();
      else wait_vmem_at_most<0>();
      __syncthreads();        // stage s in LDS for all waves; stage s - 1 fully consumed
      char* sb = lds[s % NBUF];
      if (s == nst - 1) {
        // zero V rows past t1 in the last stage (and the whole V tile of a missing
        // second page): their slots may hold anything, and 0 * NaN would leak
        for (int pg = 0; pg < 2; ++pg) {
          const int pbase = (pgA + 2 * s + pg) * kPage;
          const int valid = max(0, min(kPage, t1 - pbase));
          char* vt = sb + (2 + pg) * TILE;
          for (int idx = threadIdx.x; idx < (kPage - valid) * UPR; idx += NWR * 64)
            *reinterpret_cast<uint4*>(vt + (valid + idx / UPR) * 2 * D + (idx % UPR) * 16) =
                make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
      }
      if (s + 2 < nst) copy_stage(s + 2);
      if (wave_rows)
        pair_compute<D, RB, true>(rows, st, sb, sb + TILE, sb + 2 * TILE, sb + 3 * TILE,
                                  (pgA + 2 * s) * kPage, L, t1, a.scale_log2, a.scale_log2, 1.f, 1.f,
                                  lane);
    }
  }

  // ---- epilogue: each wave owns its rows outright
  reduce_row_sums(st);
  if (split_out) {
    auto addr = [&](int rb, float*& o, float*& l) {
      const int64_t prow = (((int64_t)b * a.Hq + rows.h[rb]) * a.Qmax + rows.i[rb]) * a.num_parts + part;
      o = a.part_o + prow * D;
      l = a.part_lse + prow;
    };
    store_partial_rows(rows, st, g, addr);
    splitk_finish<BF16, D>(a, b, hkv, C, qb);
  } else {
    store_final_rows(a, rows, st, b, g);
  }
}

// ---------------------------------------------------------------- launchers
template <typename KT, int D, int NWR>
static hipError_t launch_tile_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (KT::bytes == 2)
    hipLaunchKernelGGL((tile_dma_kernel<D, NWR>), grid, dim3(NWR * 64), 0, s, a);
  else
    hipLaunchKernelGGL((tile_attn_kernel<KT, D, NWR>), grid, dim3(NWR * 64), 0, s, a);
  return hipGetLastError();
}

template <typename KT, int D>
static hipError_t launch_tile_d(const AttnArgs& a, int nwr, dim3 grid, hipStream_t s) {
  switch (nwr) {
    case 2: return launch_tile_t<KT, D, 2>(a, grid, s);
    case 4: return launch_tile_t<KT, D, 4>(a, grid, s);
    case 8: return launch_tile_t<KT, D, 8>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tile(const AttnArgs& a, int kv_dtype, int D, int nwr, dim3 grid, hipStream_t s) {
  if (kv_dtype == 1) {
    if (D == 64) return launch_tile_d<BF16, 64>(a, nwr, grid, s);
    if (D == 128) return launch_tile_d<BF16, 128>(a, nwr, grid, s);
  } else if (kv_dtype == 2) {
    if (D == 64) return launch_tile_d<FP8, 64>(a, nwr, grid, s);
    if (D == 128) return launch_tile_d<FP8, 128>(a, nwr, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
