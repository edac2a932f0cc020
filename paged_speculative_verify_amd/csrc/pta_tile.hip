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
    // a missing second page has its V tile zeroed and its tokens past t1
    pair_compute<D, RB, false, KT::bytes == 1>(rows, st, kl, kl + T::TILE_LDS, kl + 2 * T::TILE_LDS,
                                               kl + 3 * T::TILE_LDS, (pgA + 2 * s) * kPage, L, t1,
                                               score_scale(a, sc.k0), score_scale(a, sc.k1), sc.v0, sc.v1,
                                               lane);
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
// cost for bytes in flight.  Of NBUF LDS stage buffers one is read while a
// page pair is computed and NBUF - 1 are in flight, with one barrier per
// pair; NBUF is chosen per workgroup size to fill about 128 KiB of LDS per
// compute unit, since HBM latency needs that much in flight.
//
// The copies are issued with inline asm so that the compiler, which would
// otherwise wait for every outstanding copy before any LDS read, leaves the
// waits to the kernel: before the barrier that opens stage s a wave waits
// until only its copies of later stages remain in flight (vector memory
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

// One dword per lane from HBM into LDS at M0 + 4 * lane.
__device__ __forceinline__ void lds_copy4(uint32_t lds_addr, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(lds_addr), "v"(gptr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most k stages of CPW copies each are in flight (k <= K).
template <int CPW, int K>
__device__ __forceinline__ void wait_stages(int k) {
  if constexpr (K == 0) {
    wait_vmem_at_most<0>();
  } else {
    if (k >= K) wait_vmem_at_most<K * CPW>();
    else wait_stages<CPW, K - 1>(k);
  }
}

template <int D, int NWR, int NBUF>
struct DmaGeom {
  static constexpr int TILE = kPage * D * 2;                 // bf16 page tile, HBM and LDS
  static constexpr int CPT = TILE / 1024;                    // 1 KiB copies per tile
  static constexpr int CHUNKS = 4 * CPT;                     // K page 0, K page 1, V page 0, V page 1
  static constexpr int CPW = (CHUNKS + NWR - 1) / NWR;       // copies per wave per stage
  static constexpr int STAGE = 4 * TILE;
  static constexpr int UPR = 2 * D / 16;                     // 16-byte units per row
  static constexpr int RPC = 1024 / (2 * D);                 // rows per copy
  static constexpr int LDS_BYTES = NBUF * STAGE;
  static_assert(NBUF >= 2 && (NBUF - 2) * CPW < 64, "stages in flight exceed the vmcnt range");
};

// The 32-row blocks of one (sequence b, KV head hkv) over tokens [t0, t1):
// wave w owns rows row0 + 32 w .. + 31 of the unit's M = G * q_b rows; every
// wave takes part in the copies whether or not it owns rows.  On return st
// holds the wave's flash state with its row sums reduced; the LDS buffers may
// still be read by other waves (the caller synchronises before reusing them).
//
// Software pipeline over page pairs, iteration s:
//   1. S of pair s + 1 (matrix core)     with  P of pair s (vector ALU)
//   2. P.V of pair s (matrix core)       with  masking and lane maxima of
//                                              pair s + 1 (vector ALU)
//   3. the rare move of a row's reference maximum for pair s + 1
// so most vector work of one pair has matrix-core work of another to hide
// behind.  The factor a reference-max move applies to O waits until the P.V
// of pair s has been added (l and m move at once).
//
// DMA stage j (j = -1 .. nst - 1) holds the K tiles of page pair j + 1 and
// the V tiles of pair j, in buffer (j + 1) % NBUF: iteration s reads one
// buffer (K for the scores of pair s + 1, V for the P.V of pair s) and the
// other NBUF - 1 buffers are all in flight.  Stage -1 carries K of pair 0
// (its V half repeats pair 0, unused) and stage nst - 1 repeats K of the
// last pair (its score products are masked out), so every stage moves the
// same number of chunks.  A missing second page of a pair repeats the first
// (its tokens are masked, its V rows zeroed).
template <int D, int NWR, int NBUF>
__device__ __forceinline__ void dma_range(const AttnArgs& a, char* lds, uint32_t lds0, const int* tring,
                                          uint32_t tring0, StreamRows<D, 2>& rows, StreamState<D, 2>& st,
                                          int b, int hkv, int qb, int row0, int t0, int t1, int wave,
                                          int lane, int prog0 = 0, int prog_len = 0) {
  using Gm = DmaGeom<D, NWR, NBUF>;
  constexpr int RB = 2;
  const int g = lane >> 4, m = lane & 15;
  const int C = a.ctx[b];
  const int L = C - qb;
  const int M = a.G * qb;
  const int wrow0 = row0 + wave * 32;
  const bool wave_rows = wrow0 < M;
  const float c = score_scale(a, 1.f);     // Q carries the sign of a negative scale

  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int pgA = t0 / kPage;
  const int npg = (t1 + kPage - 1) / kPage - pgA;
  const int nst = (npg + 1) / 2;

  // Block-table entries of the range are staged in an LDS ring of kRing
  // entries (relative page e at tring[e % kRing]), 64 entries per dword DMA
  // issued by wave 0: chunks 0..3 before the loop, chunk c in the iteration
  // where the copies have just left chunk c - 4 behind, about 90 iterations
  // before its first use.  Every stage copy reads its four entries from LDS,
  // so no copy waits on a table load.
  constexpr int kRing = 256;
  const int nch = (npg + 63) / 64;
  auto issue_chunk = [&](int ch) {
    const int e = min(64 * ch + lane, npg - 1);           // clamped: stays inside the range
    lds_copy4(tring0 + (uint32_t)((ch & 3) * 256), table + pgA + e);
  };
  const int crow = lane / Gm::UPR, cunit = lane % Gm::UPR;
  __builtin_assume(wave >= 0 && wave < NWR);     // lets the copies' tile selection fold
  auto copy_stage = [&](int j) {
    const int kr = 2 * min(j + 1, nst - 1), vr = 2 * max(j, 0);      // relative pages
    const bool k2 = kr + 1 < npg, v2 = vr + 1 < npg;
    const int2 kk = *reinterpret_cast<const int2*>(tring + (kr & (kRing - 1)));
    const int2 vv = *reinterpret_cast<const int2*>(tring + (vr & (kRing - 1)));
    const int xk0 = __builtin_amdgcn_readfirstlane(kk.x);
    const int xk1 = __builtin_amdgcn_readfirstlane(k2 ? kk.y : kk.x);
    const int xv0 = __builtin_amdgcn_readfirstlane(vv.x);
    const int xv1 = __builtin_amdgcn_readfirstlane(v2 ? vv.y : vv.x);
    const uint32_t dst = lds0 + (uint32_t)(((j + 1) % NBUF) * Gm::STAGE);
#pragma unroll
    for (int i = 0; i < Gm::CPW; ++i) {
      int cc = wave + i * NWR;
      if constexpr (Gm::CHUNKS % NWR != 0) cc %= Gm::CHUNKS;   // surplus waves repeat a copy
      const int tile = cc / Gm::CPT, jj = cc % Gm::CPT;
      const int64_t ph = tile == 0 ? xk0 : tile == 1 ? xk1 : tile == 2 ? xv0 : xv1;
      const int r = Gm::RPC * jj + crow;
      const char* src = (tile < 2 ? kbase : vbase) + (ph * a.Hkv + hkv) * Gm::TILE + r * 2 * D +
                        ((cunit ^ (r & (Gm::UPR - 1))) << 4);
      lds_copy16(dst + (uint32_t)(tile * Gm::TILE + 1024 * jj), src);
    }
  };
  auto buf = [&](int j) { return lds + ((j + 1) % NBUF) * Gm::STAGE; };
  auto pbase = [&](int s) { return (pgA + 2 * s) * kPage; };
  const int plain_end = min(L, t1);     // pairs ending here or before need no mask

  // The first table chunks and the query rows load together (one round trip,
  // and no wait on the query registers inside the loop); the first stages
  // then read their entries from the ring like every later stage, and only
  // stage -1 must land before the first score products.
  const int pro = min(NBUF, nst + 1);                // stages -1 .. pro - 2
  if (wave == 0)
    for (int ch = 0; ch < min(4, nch); ++ch) issue_chunk(ch);
  load_rows(rows, a, b, hkv, qb, M, g, m, wrow0);
  wait_vmem_at_most<0>();
  __syncthreads();
  for (int j = -1; j < pro - 1; ++j) copy_stage(j);
  wait_stages<Gm::CPW, NBUF - 1>(pro - 1);
  __syncthreads();

  // masked raw scores of the pair whose P comes next, in two register sets
  // that alternate between iterations (no copy from the score accumulators)
  float xa[RB][8], xb[RB][8];
  float alpha[RB] = {1.f, 1.f};      // O's factor owed before the next P.V
  bool pend = false;
  if (wave_rows) {
    PairScores<RB> sc;
    pair_scores<D, RB, true>(rows, sc, buf(-1), buf(-1) + Gm::TILE, lane);
    if (pbase(0) + 2 * kPage > plain_end) pair_mask<D, RB>(rows, sc, pbase(0), L, t1, lane);
    bool need;
    pair_max_prep<D, RB>(st, sc, xa, need, c);
    pair_max_finish<D, RB>(st, xa, need, alpha, c);  // O is still zero: its factor is moot
  }

  // One iteration of the pipeline: P of pair s from x, scores of pair s + 1 into xn.
  auto step = [&](int s, char* sb, float (&x)[RB][8], float (&xn)[RB][8]) {
    if (pend) {                       // the factor owed since pair s's maximum moved
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < D / 16; ++db) st.o[rb][db] *= alpha[rb];
    }
    // 1. S of pair s + 1 with P of pair s
    PairScores<RB> sn;
    pair_scores<D, RB, true>(rows, sn, sb, sb + Gm::TILE, lane);
    bf16x8 p[RB];
    pair_p<D, RB>(st, x, p, c);
    // 2. P.V of pair s with the masked scores of pair s + 1
    pair_pv_mma<D, RB, true, false>(st, p, p, sb + 2 * Gm::TILE, sb + 3 * Gm::TILE, lane);
    if (pbase(s + 1) + 2 * kPage > plain_end) pair_mask<D, RB>(rows, sn, pbase(s + 1), L, t1, lane);
    bool need;
    pair_max_prep<D, RB>(st, sn, xn, need, c);
    // 3. the rare reference-max move for pair s + 1
    pend = pair_max_finish<D, RB>(st, xn, need, alpha, c);
  };

  // One stage: wait, the tail's V zeroing, the next copies, the step.
  auto stage = [&](int s, float (&x)[RB][8], float (&xn)[RB][8]) {
    wait_stages<Gm::CPW, NBUF - 2>(min(NBUF - 2, nst - 1 - s));
    __syncthreads();        // stage s in LDS for all waves; stage s - 1 fully consumed
    char* sb = buf(s);
    if (s == nst - 1) {
      // zero V rows past t1 in the last pair (and the whole V tile of a missing
      // second page): their slots may hold anything, and 0 * NaN would leak
      for (int pg = 0; pg < 2; ++pg) {
        const int pb = pbase(s) + pg * kPage;
        const int valid = max(0, min(kPage, t1 - pb));
        char* vt = sb + (2 + pg) * Gm::TILE;
        for (int idx = threadIdx.x; idx < (kPage - valid) * Gm::UPR; idx += NWR * 64)
          *reinterpret_cast<uint4*>(vt + (valid + idx / Gm::UPR) * 2 * D + (idx % Gm::UPR) * 16) =
              make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }
    if ((s + NBUF - 1) % 32 == 0 && wave == 0) {
      const int ch = (s + NBUF - 1) / 32 + 3;
      if (ch < nch) issue_chunk(ch);
    }
    if ((s & 3) == 0) pace(prog0 + 2 * s, prog_len);     // every 4th pair: the level moves 3 times
    if (s + NBUF - 1 < nst) copy_stage(s + NBUF - 1);     // into the buffer stage s - 1 used
    if (wave_rows) step(s, sb, x, xn);
  };
  for (int s = 0; s < nst; s += 2) {
    stage(s, xa, xb);
    if (s + 1 < nst) stage(s + 1, xb, xa);
  }
  reduce_row_sums(st);
}

// Two waves per SIMD must fit: at most 256 VGPRs per wave.
template <int D, int NWR, int NBUF>
__global__ __launch_bounds__(NWR * 64) __attribute__((amdgpu_waves_per_eu(2))) void tile_dma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[DmaGeom<D, NWR, NBUF>::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) int tring[256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;           // partition past this sequence's context
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];
  const uint32_t tring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)&tring[0];

  StreamRows<D, 2> rows;
  StreamState<D, 2> st;
  st.init();
  dma_range<D, NWR, NBUF>(a, lds, lds0, tring, tring0, rows, st, b, hkv, qb, 0, t0, t1, wave, lane);

  // ---- epilogue: each wave owns its rows outright
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

// ------------------------------------------------------------ balanced tile grid
// Persistent grid for many rows per KV head.  Unit u = b * Hkv + hkv owns
// positions [S_u, S_u + P_b) of one page line (P_b = ceil(C_b / 16),
// S_u = Hkv * PS_b + hkv * P_b with PS the exclusive prefix of P over the
// sequences).  The line is cut into N equal slices; slice w is worked by RG
// workgroups, one per row group of NWR waves * 32 rows, so every row of a
// unit is covered.  The row groups of one slice are launched 8 workgroup ids
// apart: workgroups are handed to the 8 XCDs in turn, so they share an XCD
// and its L2, and the KV pages reach L2 from HBM once.  A slice that covers a
// whole unit writes its rows; otherwise it stores a normalised partial in
// slot w + u (unique: slices and units are both ordered along the line), and
// slice_merge_kernel, launched right after, merges them in slice order.
// (Merging inside this launch, by the unit's last slice, leaves a few
// workgroups reading many partials at the end of the launch while the rest of
// the device idles.)
template <int D, int NWR, int NBUF>
__global__ __launch_bounds__(NWR * 64) __attribute__((amdgpu_waves_per_eu(2))) void tile_balanced_kernel(AttnArgs a) {
  using Gm = DmaGeom<D, NWR, NBUF>;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) int tring[256];
  __shared__ int wave_tot[NWR];
  extern __shared__ int ps[];       // [B + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int B = a.B;
  const int Rmax = a.G * a.Qmax;
  const int RG = (Rmax + NWR * 32 - 1) / (NWR * 32);
  const int blk = blockIdx.x;
  const int rg = (blk >> 3) % RG;
  const int64_t w = (int64_t)((blk >> 3) / RG) * 8 + (blk & 7);
  const int64_t NS = gridDim.x / RG;

  // ---- exclusive prefix of pages per sequence (every workgroup computes it)
  page_prefix<NWR * 64>(a, ps, wave_tot, tid);
  const int64_t W = (int64_t)a.Hkv * __builtin_amdgcn_readfirstlane(ps[B]);
  const int64_t N = min(NS, max((int64_t)1, W / kMinSlicePages));
  if (w >= N) return;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];
  const uint32_t tring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)&tring[0];
  const int row0 = rg * NWR * 32;

  const int64_t x0 = w * W / N;
  const int64_t xe = (w + 1) * W / N;
  int64_t x = x0;
  while (x < xe) {
    // the unit holding position x: largest b with PS_b <= x / Hkv
    const int key = (int)(x / a.Hkv);
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(ps[mid]) <= key) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo;
    const int psb = __builtin_amdgcn_readfirstlane(ps[b]);
    const int Pb = __builtin_amdgcn_readfirstlane(ps[b + 1]) - psb;
    const int64_t off = x - (int64_t)a.Hkv * psb;
    const int hkv = (int)(off / Pb);
    const int k0 = (int)(off % Pb);
    const int k1 = (int)min((int64_t)Pb, k0 + (xe - x));
    const int u = b * a.Hkv + hkv;
    const int C = a.ctx[b];
    const int qb = a.qlen[b];
    const int M = a.G * qb;

    __syncthreads();          // LDS stage buffers free from the previous unit
    StreamRows<D, 2> rows;
    StreamState<D, 2> st;
    st.init();
    if (row0 < M) {
      dma_range<D, NWR, NBUF>(a, lds, lds0, tring, tring0, rows, st, b, hkv, qb, row0, k0 * kPage,
                              min(C, k1 * kPage), wave, lane, (int)(x - x0), (int)(xe - x0));
      if (k0 == 0 && k1 == Pb) {
        store_final_rows(a, rows, st, b, g);        // the whole unit in this slice
      } else {
        auto addr = [&](int rb, float*& o, float*& l) {
          const int64_t r = (w + u) * Rmax + row0 + wave * 32 + rb * 16 + m;
          o = a.part_o + r * D;
          l = a.part_lse + r;
        };
        store_partial_rows(rows, st, g, addr);
      }
    }
    x += k1 - k0;
  }
}

// ---------------------------------------------------------------- slice merge
// Second launch of both balanced grids: one workgroup per (unit, 32-row
// block) merges the partials of a unit cut into several slices, all slices
// read at once with plain 16-byte loads (the attention launch has completed)
// and combined by log-sum-exp in slice order.  Slice bounds are recomputed
// from the same page line as the attention launch (NS slices at most, at
// least kMinSlicePages pages each); slice w's partial of unit u is slot w + u.
template <typename QT, int D>
__global__ __launch_bounds__(256) void slice_merge_kernel(AttnArgs a, int NS) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int TPR = 8;                  // threads per row
  constexpr int IPT = D / 4 / TPR;        // 16-byte items per thread
  constexpr int PB = 4;                   // slices per batch (all workgroups resident at once)
  __shared__ int red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Rmax = a.G * a.Qmax;
  const int nblk = (Rmax + 31) / 32;
  const int u = blockIdx.x / nblk, rblk = blockIdx.x % nblk;
  const int b = u / a.Hkv, hkv = u % a.Hkv;
  const int qb = a.qlen[b];
  const int M = a.G * qb;
  if (rblk * 32 >= M) return;

  int before = 0, total = 0;              // pages of sequences < b, of all sequences
  for (int j = tid; j < a.B; j += 256) {
    const int p = (a.ctx[j] + kPage - 1) / kPage + a.slice_pad;   // the unit's length on the line
    total += p;
    before += j < b ? p : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    before += __shfl_xor(before, o, 64);
    total += __shfl_xor(total, o, 64);
  }
  if (lane == 0) {
    red[0][wv] = before;
    red[1][wv] = total;
  }
  __syncthreads();
  before = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  total = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const int Pb = (a.ctx[b] + kPage - 1) / kPage;
  const int Pl = Pb + a.slice_pad;
  const int64_t W = (int64_t)a.Hkv * total;
  const int64_t N = min((int64_t)NS, max((int64_t)1, W / kMinSlicePages));
  // the unit's pages sit at line positions S + slice_pad .. S + Pl - 1
  const int64_t S = (int64_t)a.Hkv * before + (int64_t)hkv * Pl + a.slice_pad;
  auto wg_of = [&](int64_t x) -> int64_t { return ((x + 1) * N - 1) / W; };
  const int64_t wfirst = wg_of(S);
  const int np = (int)(wg_of(S + Pb - 1) - wfirst + 1);
  if (np == 1) return;                    // the attention launch wrote this unit's rows
  const int r = rblk * 32 + tid / TPR;
  if (r >= M) return;
  const int d0 = (tid % TPR) * IPT * 4;

  float mrun = NEG_INF, wsum = 0.f;
  f32x4 acc[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) acc[k] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np; p0 += PB) {
    float lp[PB];
    f32x4 op[PB][IPT];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const bool ok = p0 + j < np;
      const int64_t rr = (wfirst + (ok ? p0 + j : 0) + u) * Rmax + r;
      lp[j] = ok ? a.part_lse[rr] : NEG_INF;
#pragma unroll
      for (int k = 0; k < IPT; ++k)
        op[j][k] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + rr * D + d0 + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mx = mrun;
#pragma unroll
    for (int j = 0; j < PB; ++j) mx = fmaxf(mx, lp[j]);
    const float muse = mx == NEG_INF ? 0.f : mx;
    const float alpha = __expf(mrun - muse);
    wsum *= alpha;
#pragma unroll
    for (int k = 0; k < IPT; ++k) acc[k] *= alpha;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const float w = __expf(lp[j] - muse);
      wsum += w;
#pragma unroll
      for (int k = 0; k < IPT; ++k) acc[k] += w * op[j][k];
    }
    mrun = mx;
  }
  const float muse = mrun == NEG_INF ? 0.f : mrun;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int h = hkv * a.G + r / qb, i = r % qb;
  const int64_t o = (((int64_t)b * a.Qmax + i) * a.Hq + h) * D + d0;
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const f32x4 res = acc[k] * inv;
    if constexpr (QT::bytes == 4) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o + 4 * k) = res;
    } else {
      uint2 w;
      w.x = pack_bf16x2(res[0], res[1]);
      w.y = pack_bf16x2(res[2], res[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o + 4 * k) = w;
    }
  }
  if (d0 == 0 && a.lse != nullptr)
    a.lse[((int64_t)b * a.Hq + h) * a.Qmax + i] = wsum > 0.f ? muse + __logf(wsum) : NEG_INF;
}

// ---------------------------------------------------------------- launchers
// Stage buffers per workgroup size: about 128 KiB of LDS per compute unit at
// D = 128 (one 8-wave or two 4-wave workgroups).
template <int NWR>
constexpr int dma_bufs() { return NWR == 8 ? 8 : 4; }

template <typename KT, int D, int NWR>
static hipError_t launch_tile_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (KT::bytes == 2)
    hipLaunchKernelGGL((tile_dma_kernel<D, NWR, dma_bufs<NWR>()>), grid, dim3(NWR * 64), 0, s, a);
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

// Balanced tile grid.  With a == nullptr: report the workgroups that fit the
// current device at once (compute units times occupancy).  Otherwise launch
// *nwg workgroups.
template <int D, int NWR>
static hipError_t tile_balanced_t(const AttnArgs* a, int B, int* nwg, hipStream_t s) {
  constexpr int NBUF = dma_bufs<NWR>();
  const size_t dyn = (size_t)(B + 1) * sizeof(int);
  if (a == nullptr) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, tile_balanced_kernel<D, NWR, NBUF>, NWR * 64, dyn);
    if (e != hipSuccess) return e;
    *nwg = cus * (per > 0 ? per : 1);
    return hipSuccess;
  }
  hipLaunchKernelGGL((tile_balanced_kernel<D, NWR, NBUF>), dim3((unsigned)*nwg), dim3(NWR * 64), dyn, s, *a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int RG = (a->G * a->Qmax + NWR * 32 - 1) / (NWR * 32);
  return launch_slice_merge(*a, D, *nwg / RG, s);
}

hipError_t launch_slice_merge(const AttnArgs& a, int D, int NS, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.Hkv * ((a.G * a.Qmax + 31) / 32);
  if (D == 64) hipLaunchKernelGGL((slice_merge_kernel<BF16, 64>), dim3((unsigned)blocks), dim3(256), 0, s, a, NS);
  else if (D == 128) hipLaunchKernelGGL((slice_merge_kernel<BF16, 128>), dim3((unsigned)blocks), dim3(256), 0, s, a, NS);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t tile_balanced(const AttnArgs* a, int D, int nwr, int B, int* nwg, hipStream_t s) {
  if (D == 64) {
    if (nwr == 2) return tile_balanced_t<64, 2>(a, B, nwg, s);
    if (nwr == 4) return tile_balanced_t<64, 4>(a, B, nwg, s);
  } else if (D == 128) {
    if (nwr == 2) return tile_balanced_t<128, 2>(a, B, nwg, s);
    if (nwr == 4) return tile_balanced_t<128, 4>(a, B, nwg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
