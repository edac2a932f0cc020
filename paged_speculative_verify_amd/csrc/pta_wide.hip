// Wide-tree paged tree attention on gfx950: many query rows per KV head (33 to
// 256, the GQA group's q-heads times a candidate tree), bf16 KV.  Lookahead
// verification turns each sequence's decode GEMV into a real GEMM (TACO-LLM
// design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践", TurboAttention
// bullets of "整体方案分为两大部分": matrix units once vector-matrix work
// becomes matrix-matrix work; "优化策略总结" item 2: on-chip use independent
// of the sequence length).
//
// With this many rows per KV tile the 16x16x32-product kernel of pta_tile.hip
// issues about 260 instructions per wave and page pair for 32 matrix-core
// products; this one is written to issue as few as it can (about 190):
//   * v_mfma_f32_32x32x16_bf16 for S^T = K Q^T and O^T += V^T P^T: a wave's 32
//     rows are the N dimension, so per 32-token page pair a wave issues 8 + 8
//     products (half the count of the 16x16x32 form, and fewer matrix-core
//     cycles per flop on this GPU).  Lane (h, n) = (lane / 32, lane % 32) owns
//     row n and tokens 8 j + 4 h + i (j, i < 4) of the pair; those 16 scores,
//     in that order, are exactly the lane's two bf16x8 B operands of P^T for
//     the two 16-token steps of P.V, so P needs no data movement.
//   * V^T operands come from ds_read_b64_tr_b16 (16-lane transposed reads of
//     4 tokens x 16 dims), K operands from ds_read_b128; every LDS address is
//     a per-lane register computed once plus an immediate (the stage loop is
//     unrolled over the LDS buffers, so each buffer's offset is a constant).
//   * Page tiles go HBM -> LDS with buffer_load_dwordx4 ... lds: each wave
//     moves whole page tiles (one m0 setup, the chunks addressed by the
//     instruction's offset field, the page by a scalar offset), so a copy
//     costs no vector address arithmetic.  The buffer resource's size bounds
//     the in-tile offsets; the page base rides in the scalar offset, outside
//     the range check, so page ids must name pool pages (the call's contract).
//     Page ids arrive by scalar loads one stage ahead.
//   * Row sums take the bf16 P values already packed for the matrix core
//     (v_dot2c_f32_bf16 against (1, 1)), so l is the sum of exactly the
//     weights P.V used.
//   * Tiles are swizzled so that both operand reads touch every LDS bank once
//     per pass (wide_unit): no bank conflicts (the 16x16x32 kernel's layout
//     costs its reads about a quarter of the compute unit's cycles here).
//   * One schedule per stage (scheduling groups): K reads three products ahead,
//     the vector work of pair s's P between pair s + 1's score products, a
//     page's V^T reads ahead of its P.V products.
// Measured on the widest tree (256 rows per KV head, 32K-128K tokens), the
// call is 4-5% faster than the 16x16x32 kernel's, measured back to back; with
// the copies and the per-stage barrier taken out (a timing-only build) the
// same arithmetic takes about 22% less time than the whole kernel.
// Pipeline, stages and masks follow the shared-tile kernel of pta_tile.hip:
// DMA stage j holds K of page pair j + 1 and V of pair j; iteration s computes
// S of pair s + 1 and P, P.V of pair s; reference maxima move lazily.
// The verify step's KV append can ride in the same grid (the fused-append
// entry): each unit piece writes the candidate rows on its own pages first.
#include "pta_device.h"
#include "pta_flash.h"
#include "pta_launch.h"

#include <type_traits>

namespace pta {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// LDS: a K region and a V region of NBUF stage buffers each (stage buffer b
// holds two page tiles in each region), so every buffer's offset inside its
// region is a 16-bit immediate of the LDS reads.
template <int D, int NWR, int NBUF>
struct WideGeom {
  static constexpr int TILE = kPage * D * 2;                 // bf16 page tile, HBM and LDS
  static constexpr int CPT = TILE / 1024;                    // 1 KiB chunks per tile
  static constexpr int PAIR = 2 * TILE;                      // one pair's K (or V) tiles
  static constexpr int VREG = NBUF * PAIR;                   // start of the V region
  static constexpr int UPR = 2 * D / 16;                     // 16-byte units per row
  static constexpr int KS = D / 16;                          // 32x32x16 k-steps over the head dim
  static constexpr int DB = D / 32;                          // 32-dim blocks of O^T
  static constexpr int CPW = 4 * CPT / NWR;                  // copies per wave per stage
  static constexpr int LOADS = CPW;
  static constexpr int NTW = CPW >= CPT ? CPW / CPT : 1;     // tiles a wave touches per stage
  static constexpr int CPTW = CPW >= CPT ? CPT : CPW;        // copies per touched tile
  static constexpr int LDS_BYTES = 2 * VREG;
  static_assert(NWR == 2 || NWR == 4, "2 or 4 waves of 32 rows");
  static_assert(CPW >= 1 && (4 * CPT) % NWR == 0, "whole copies per wave");
  static_assert(NBUF >= 2 && NBUF % 2 == 0 && (NBUF - 2) * LOADS < 64, "stage count");
  static_assert(VREG <= 65536, "LDS offsets must fit the 16-bit immediate");
  // LDS byte offset of tile t (0, 1: K of the stage's later pair; 2, 3: V of
  // its earlier pair) of stage buffer b
  static constexpr int tile_lds(int b, int t) { return (t < 2 ? 0 : VREG) + b * PAIR + (t & 1) * TILE; }
};

// Buffer resource over `bytes` bytes at `base` (raw, stride 0).  The copies
// put a page tile's base in the scalar offset, which the range check does not
// cover, so every page id must name a page of the pool (the call's contract);
// the check covers the in-tile vector and instruction offsets.
__device__ __forceinline__ i32x4 wide_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = (int32_t)(uint32_t)p;
  r[1] = (int32_t)(uint32_t)(p >> 32);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

// N consecutive 1 KiB chunks of one page tile from rsrc + soff into LDS at
// m0val: chunk c reads rsrc + soff + voff[c] + 1024 c and writes m0val +
// 1024 c + 16 lane (the instruction offset moves both addresses alike).  The
// s_nop covers the wait state an M0 write needs before an LDS-DMA load.
// NTH: the nontemporal (streaming) hint, for page tiles no other workgroup reads.
#define PTA_WIDE_COPIES(H)                                                                              \
  if constexpr (CPT == 1) {                                                                             \
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"                                                    \
                 "buffer_load_dwordx4 %1, %2, %3 offen" H " lds"                                        \
                 :                                                                                      \
                 : "s"(m0val), "v"(voff[0]), "s"(rsrc), "s"(soff)                                       \
                 : "memory", "m0");                                                                     \
  } else if constexpr (CPT == 4) {                                                                      \
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"                                                    \
                 "buffer_load_dwordx4 %1, %5, %6 offen" H " lds\n\t"                                   \
                 "buffer_load_dwordx4 %2, %5, %6 offen offset:1024" H " lds\n\t"                       \
                 "buffer_load_dwordx4 %3, %5, %6 offen offset:2048" H " lds\n\t"                       \
                 "buffer_load_dwordx4 %4, %5, %6 offen offset:3072" H " lds"                            \
                 :                                                                                      \
                 : "s"(m0val), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rsrc),       \
                   "s"(soff)                                                                            \
                 : "memory", "m0");                                                                     \
  } else {                                                                                              \
    static_assert(CPT == 2, "1, 2 or 4 chunks");                                                        \
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"                                                    \
                 "buffer_load_dwordx4 %1, %3, %4 offen" H " lds\n\t"                                   \
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:1024" H " lds"                            \
                 :                                                                                      \
                 : "s"(m0val), "v"(voff[0]), "v"(voff[1]), "s"(rsrc), "s"(soff)                         \
                 : "memory", "m0");                                                                     \
  }

template <int CPT, bool NTH>
__device__ __forceinline__ void wide_copy_tile(uint32_t m0val, const i32x4& rsrc, uint32_t soff,
                                               const uint32_t (&voff)[CPT]) {
  if constexpr (NTH) {
    PTA_WIDE_COPIES(" nt")
  } else {
    PTA_WIDE_COPIES("")
  }
}
#undef PTA_WIDE_COPIES

// A wave-uniform table entry through the scalar cache (s_load): a vector load
// would join the vmcnt queue behind the page copies, and waiting for it would
// wait for every copy in flight.  The table is read-only during the launch.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}

template <int I, int N, typename F>
__device__ __forceinline__ void wide_static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    wide_static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void wide_static_for(F&& f) {
  wide_static_for_impl<0, N>(f);
}

template <int N>
__device__ __forceinline__ void wide_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most k later stages of L copies each are in flight (k <= K).
template <int L, int K>
__device__ __forceinline__ void wide_wait_stages(int k) {
  if constexpr (K == 0) {
    wide_wait_vm<0>();
  } else {
    if (k >= K) wide_wait_vm<K * L>();
    else wide_wait_stages<L, K - 1>(k);
  }
}

// The lane's row of the unit (row = row0 + lane % 32): Q^T operands, candidate
// mask bits and output coordinates.
template <int D>
struct WideRows {
  bf16x8 qop[D / 16];   // B operand of k-step ks: dims 16 ks + 8 h + (0..7) of the row
  uint64_t mbits;
  bool ok;
  int hq, i;
};

// Flash state of the lane's row: O^T (o[db][4 j + r] = dim 32 db + 8 j + 4 h + r),
// the reference maximum (log2 units) and the sum of the lane's own tokens.
template <int D>
struct WideState {
  f32x16 o[D / 32];
  float m, l;
};

template <int D>
__device__ __forceinline__ void wide_load_rows(WideRows<D>& R, const AttnArgs& a, int b, int hkv, int qb, int M,
                                               int lane, int row0) {
  const int n = lane & 31, h = lane >> 5;
  const int row = row0 + n;
  R.ok = row < M;
  R.hq = hkv * a.G + (R.ok ? row / qb : 0);
  R.i = R.ok ? row % qb : 0;
  const uint16_t* qp =
      reinterpret_cast<const uint16_t*>(a.q) + (((int64_t)b * a.Qmax + R.i) * a.Hq + R.hq) * D + 8 * h;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 w = R.ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
    R.qop[ks] = __builtin_bit_cast(bf16x8, w);
  }
  R.mbits = R.ok ? load_mask_row(a.mask, b, R.i, qb, a.Qmax) : 0ull;
  // a negative scale moves into Q's sign (after the mask loads are issued, so the
  // row's loads share one round trip)
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 w = __builtin_bit_cast(uint4, R.qop[ks]);
      w.x ^= 0x80008000u;
      w.y ^= 0x80008000u;
      w.z ^= 0x80008000u;
      w.w ^= 0x80008000u;
      R.qop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// Physical 16-byte unit holding logical unit u of tile row r (an involution,
// so it also names the logical unit a physical slot holds).  D = 128: the
// unit's high bits are XORed with the row's low bits and its low bits with the
// row's high bits, so both operand reads touch every bank once per pass: the K
// reads (one unit of 16 rows) and the transposed V reads (4 units of 4 rows).
// D = 64: the unit is XORed with the row.
template <int D>
__device__ __forceinline__ int wide_unit(int r, int u) {
  if constexpr (D == 128) return (((u >> 2) ^ (r & 3)) << 2) | ((u & 3) ^ ((r >> 2) & 3));
  else return u ^ (r & (2 * D / 16 - 1));
}

// Per-lane LDS offsets inside a stage buffer (the buffer's offset is added as
// an immediate): K operand of k-step ks, and the two transposed V reads of
// dim block db (tokens 4 h + 0..3 and 8 + 4 h + 0..3 of a page).
template <int D>
struct WideOffsets {
  uint32_t k[D / 16];
  uint32_t v[D / 32][2];
};

template <int D>
__device__ __forceinline__ void wide_offsets(WideOffsets<D>& W, int lane, uint32_t vreg) {
  constexpr int TILE = kPage * D * 2;
  constexpr int UPR = 2 * D / 16;
  const int n = lane & 31, h = lane >> 5;
  const int pg = n >> 4, r = n & 15;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    W.k[ks] = (uint32_t)(pg * TILE + r * 2 * D + (wide_unit<D>(r, 2 * ks + h) << 4));
  const int q = lane >> 4, i = lane & 15, dh = q & 1;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int rr = 4 * h + (i >> 2) + 8 * rd;
      const int u = 4 * db + 2 * dh + ((i & 3) >> 1);
      W.v[db][rd] = vreg + (uint32_t)(rr * 2 * D + (wide_unit<D>(rr, u) << 4) + 8 * (i & 1));
    }
}

// S^T of one page pair from the K tiles at byte offset KB of the LDS array.
template <int D, int KB>
__device__ __forceinline__ f32x16 wide_scores(const WideRows<D>& R, const WideOffsets<D>& W, const char* lds) {
  f32x16 s = {};
  bf16x8 k[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) k[ks] = *reinterpret_cast<const bf16x8*>(lds + W.k[ks] + KB);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[ks], R.qop[ks], s, 0, 0, 0);
  return s;
}

// Masked scores: tokens past t1, and candidates the row's tree does not show,
// become -inf.  Lane token e = 4 j + i is pbase + 8 j + 4 h + i.
__device__ __forceinline__ void wide_mask(f32x16& s, uint64_t mbits, int pbase, int L, int t1, int lane) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int h = lane >> 5;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int t = pbase + 8 * (e >> 2) + 4 * h + (e & 3);
    const int sh = t - L;
    const bool cand = (unsigned)sh < 64u && ((mbits >> (sh & 63)) & 1ull);
    s[e] = (t < t1 && (t < L || cand)) ? s[e] : NEG_INF;
  }
}

// Lane maximum of a pair's raw scores and whether the scaled maximum passes
// the row's reference by more than the lazy headroom.
__device__ __forceinline__ bool wide_max_prep(const f32x16& s, float m, float c, float& pm) {
  auto mx = [](float u, float v) { return __builtin_elementwise_maximum(u, v); };
  const float a0 = mx(mx(s[0], s[1]), s[2]), a1 = mx(mx(s[3], s[4]), s[5]);
  const float a2 = mx(mx(s[6], s[7]), s[8]), a3 = mx(mx(s[9], s[10]), s[11]);
  const float a4 = mx(mx(s[12], s[13]), s[14]);
  pm = mx(mx(mx(a0, a1), a2), mx(mx(a3, a4), s[15]));
  return c * pm > m + kLazyTau;
}

// The rare move of the reference maximum (wave-uniform decision): the row's
// two lanes (h = 0, 1) agree on the new maximum; l is rescaled here and O's
// factor is returned for the caller to apply before the next P.V.
template <int D>
__device__ __forceinline__ bool wide_max_finish(WideState<D>& st, float pm, bool need, float c, float& alpha) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  if (__builtin_amdgcn_ballot_w64(need) == 0) return false;
  pm = fmaxf(pm, shfl_xor(pm, 32));
  const float mnew = fmaxf(st.m, c * pm);
  alpha = fast_exp2(st.m - (mnew == NEG_INF ? 0.f : mnew));
  st.m = mnew;
  st.l *= alpha;
  return true;
}

// P of a pair in bf16 (p[t] = B operand of 16-token step t) and its row sum.
template <int D>
__device__ __forceinline__ void wide_p(WideState<D>& st, const f32x16& x, float c, bf16x8 (&p)[2]) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  const float nm = st.m == NEG_INF ? 0.f : -st.m;
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = fast_exp2(fmaf(x[8 * t + 2 * k], c, nm));
      const float p1 = fast_exp2(fmaf(x[8 * t + 2 * k + 1], c, nm));
      w[k] = pack_bf16x2(p0, p1);
      st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[k]), one, st.l, false);
    }
    p[t] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// O^T += V^T P^T for one pair from the V tiles at byte offset VB of the V
// region (whose start W.v already holds).
template <int D, int VB>
__device__ __forceinline__ void wide_pv(WideState<D>& st, const WideOffsets<D>& W, const bf16x8 (&p)[2],
                                        const char* lds) {
  constexpr int TILE = kPage * D * 2, DB = D / 32;
  auto rd = [&](uint32_t off) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off)); };
  auto cat = [](s16x4 va, s16x4 vb) {
    return __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint2, va).x, __builtin_bit_cast(uint2, va).y,
                                                 __builtin_bit_cast(uint2, vb).x, __builtin_bit_cast(uint2, vb).y));
  };
  // the first page's operands are all read before its products, and each
  // product of the first page is followed by the read of the matching operand
  // of the second page, so every product finds its operand in registers
  s16x4 va[DB], vb[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    va[db] = rd(W.v[db][0] + VB);
    vb[db] = rd(W.v[db][1] + VB);
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat(va[db], vb[db]), p[0], st.o[db], 0, 0, 0);
    va[db] = rd(W.v[db][0] + VB + TILE);
    vb[db] = rd(W.v[db][1] + VB + TILE);
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat(va[db], vb[db]), p[1], st.o[db], 0, 0, 0);
}

// The unit's rows row0 + 32 wave .. over tokens [t0, t1) of sequence b, KV
// head hkv.  Every wave takes part in the copies whether or not it owns rows.
// On return st holds the wave's flash state with l summed over the row's two
// lanes; the LDS buffers may still be read by other waves.
template <int D, int NWR, int NBUF>
__device__ __forceinline__ void wide_range(const AttnArgs& a, char* lds, uint32_t lds0, const i32x4& krs,
                                           const i32x4& vrs, WideRows<D>& R, WideState<D>& st, int b, int hkv,
                                           int qb, int row0, int t0, int t1, int wave, int lane, int prog0,
                                           int prog_len) {
  using Gm = WideGeom<D, NWR, NBUF>;
  const int C = a.ctx[b];
  const int L = C - qb;
  const int M = a.G * qb;
  const int wrow0 = row0 + wave * 32;
  const bool wave_rows = wrow0 < M;
  const float c = score_scale(a, 1.f);

  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const int pgA = t0 / kPage;
  const int npg = (t1 + kPage - 1) / kPage - pgA;
  const int nst = (npg + 1) / 2;
  const uint32_t hk_off = (uint32_t)hkv * (uint32_t)Gm::TILE;
  // the streaming hint when this workgroup alone reads the unit's tiles: a single row
  // group and no page shared between block tables (row groups of one slice share
  // each tile through L2)
  const bool nt_pages = a.stream_pages != 0 && a.G * a.Qmax <= NWR * 32;
  const uint32_t ph_stride = (uint32_t)a.Hkv * (uint32_t)Gm::TILE;

  // This wave's copies: chunks wave * CPW .. + CPW - 1 of the stage's 4 * CPT
  // (tile = chunk / CPT).  Copy lane l of chunk c of a tile fills physical slot
  // l % UPR of row c * rows-per-chunk + l / UPR, so it reads the logical unit
  // that slot holds; the offset of the wave's first chunk in its tile (jj0 KiB)
  // is folded in here and into m0.
  const int jj0 = (wave * Gm::CPW) % Gm::CPT;
  uint32_t voff[Gm::CPTW];
#pragma unroll
  for (int cc = 0; cc < Gm::CPTW; ++cc) {
    const int rpc = 1024 / (2 * D);
    const int rr = rpc * (jj0 + cc) + lane / Gm::UPR;
    voff[cc] = (uint32_t)(1024 * jj0 + (lane / Gm::UPR) * 2 * D + (wide_unit<D>(rr, lane % Gm::UPR) << 4));
  }
  WideOffsets<D> W;
  wide_offsets<D>(W, lane, (uint32_t)Gm::VREG);

  // relative page of tile `tile` in DMA stage j (K tiles: pair j + 1, V tiles:
  // pair j; the last pair's K repeats past the end, a missing second page of a
  // pair repeats its first)
  auto rel_page = [&](int j, int tile) -> int {
    const int pr = tile < 2 ? min(j + 1, nst - 1) : max(j, 0);
    const int p = 2 * pr + (tile & 1);
    return p < npg ? p : 2 * pr;
  };
  const int tile0 = (wave * Gm::CPW) / Gm::CPT;        // first tile this wave copies into
  // the page ids of this wave's tiles of stage j (wave-uniform scalar loads)
  auto page_ids = [&](int j, int (&ph)[Gm::NTW]) {
#pragma unroll
    for (int k = 0; k < Gm::NTW; ++k) ph[k] = scalar_load(table + pgA + rel_page(j, tile0 + k));
  };
  auto copy_stage = [&](int j, const int (&ph)[Gm::NTW], int buf) {
#pragma unroll
    for (int k = 0; k < Gm::NTW; ++k) {
      const int tile = tile0 + k;
      const uint32_t soff = (uint32_t)ph[k] * ph_stride + hk_off;
      const uint32_t dst = lds0 + (uint32_t)((tile < 2 ? 0 : Gm::VREG) + buf * Gm::PAIR + (tile & 1) * Gm::TILE +
                                             1024 * jj0);
      if (nt_pages) wide_copy_tile<Gm::CPTW, true>(dst, tile < 2 ? krs : vrs, soff, voff);
      else wide_copy_tile<Gm::CPTW, false>(dst, tile < 2 ? krs : vrs, soff, voff);
    }
  };

  // prologue: rows and the first stages (-1 .. pro - 2)
  wide_load_rows<D>(R, a, b, hkv, qb, M, lane, wrow0);
  st.m = -__builtin_huge_valf();
  st.l = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = {};
  const int pro = min(NBUF, nst + 1);
  int ph[Gm::NTW];
  page_ids(-1, ph);
  for (int j = -1; j < pro - 1; ++j) {
    copy_stage(j, ph, (j + 1) % NBUF);
    page_ids(j + 1, ph);
  }
  // ph now holds stage pro - 1's pages: the first copy issued inside the loop
  wide_wait_stages<Gm::LOADS, NBUF - 1>(pro - 1);
  __syncthreads();

  f32x16 xa, xb;                           // raw scores of the pair whose P comes next
  float alpha = 1.f;
  bool pend = false;
  if (wave_rows) {
    xa = wide_scores<D, 0>(R, W, lds);
    if (pgA * kPage + 2 * kPage > min(L, t1)) wide_mask(xa, R.mbits, pgA * kPage, L, t1, lane);
    float pm;
    const bool need = wide_max_prep(xa, st.m, c, pm);
    wide_max_finish<D>(st, pm, need, c, alpha);      // O is still zero: its factor is moot
  }
  const int plain_end = min(L, t1);

  // iteration s with LDS buffer BUF = (s + 1) % NBUF; x holds pair s's scores
  auto stage = [&](auto bufc, int s, f32x16& x, f32x16& xn) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int PREV = (BUF + NBUF - 1) % NBUF;    // stage s - 1's buffer, refilled here
    wide_wait_stages<Gm::LOADS, NBUF - 2>(min(NBUF - 2, nst - 1 - s));
    __syncthreads();                       // stage s in LDS for all waves; stage s - 1 consumed
    if (s == nst - 1) {
      // V rows past t1 in the last pair (and all of a missing second page) are
      // zeroed: their slots may hold anything, and 0 * NaN would leak
      const int pb = (pgA + 2 * s) * kPage;
      for (int pg = 0; pg < 2; ++pg) {
        const int valid = max(0, min(kPage, t1 - pb - pg * kPage));
        char* vt = lds + Gm::tile_lds(BUF, 2 + pg);
        for (int idx = threadIdx.x; idx < (kPage - valid) * Gm::UPR; idx += NWR * 64)
          *reinterpret_cast<uint4*>(vt + (valid + idx / Gm::UPR) * 2 * D + (idx % Gm::UPR) * 16) =
              make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }
    if ((s & 3) == 0) pace(prog0 + 2 * s, prog_len);
    if (s + NBUF - 1 < nst) {
      copy_stage(s + NBUF - 1, ph, PREV);
      if (s + NBUF < nst) page_ids(s + NBUF, ph);
    }
    if (wave_rows) {
      if (pend) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
      }
      xn = wide_scores<D, Gm::tile_lds(BUF, 0)>(R, W, lds);            // S of pair s + 1
      bf16x8 p[2];
      wide_p<D>(st, x, c, p);                                          // P of pair s
      wide_pv<D, BUF * Gm::PAIR>(st, W, p, lds);                       // P.V of pair s
      // K reads three ahead; each score product of pair s + 1 followed by six vector
      // instructions of pair s's P; the V^T reads of the first page, then each P.V
      // product of the first page followed by the matching reads of the second
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 5) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x080, 8, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x080, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      const int pbn = (pgA + 2 * (s + 1)) * kPage;
      if (pbn + 2 * kPage > plain_end) wide_mask(xn, R.mbits, pbn, L, t1, lane);
      float pm;
      const bool need = wide_max_prep(xn, st.m, c, pm);
      pend = wide_max_finish<D>(st, pm, need, c, alpha);
    }
  };
  // NBUF iterations per round, so every buffer offset is a constant; NBUF is
  // even, so the two score register sets alternate the same way every round
  for (int s = 0; s < nst; s += NBUF) {
    bool more = true;
    wide_static_for<NBUF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (!more) return;
      if (s + i >= nst) {
        more = false;
        return;
      }
      if constexpr (i % 2 == 0) stage(std::integral_constant<int, (i + 1) % NBUF>{}, s + i, xa, xb);
      else stage(std::integral_constant<int, (i + 1) % NBUF>{}, s + i, xb, xa);
    });
  }
  st.l += shfl_xor(st.l, 32);
}

// Final rows of a lane: out = O / l (bf16), lse = ln l + max (lanes h = 0).
template <int D>
__device__ __forceinline__ void wide_store_final(const AttnArgs& a, const WideRows<D>& R, const WideState<D>& st,
                                                 int b, int lane) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  if (!R.ok) return;
  const int h = lane >> 5;
  const float lt = st.l;
  const float muse = st.m == NEG_INF ? 0.f : st.m;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (((int64_t)b * a.Qmax + R.i) * a.Hq + R.hq) * D + 4 * h;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 w;
      w.x = pack_bf16x2(st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv);
      w.y = pack_bf16x2(st.o[db][4 * j + 2] * inv, st.o[db][4 * j + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * db + 8 * j) = w;
    }
  if (h == 0 && a.lse != nullptr)
    a.lse[((int64_t)b * a.Hq + R.hq) * a.Qmax + R.i] = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
}

// Partial row of a lane (normalised O and natural-log LSE) into o (D floats)
// and *l, with plain stores (read by a later launch) or device-coherent ones
// (read by the last arriving unit of the same launch).
template <int D, bool COHERENT>
__device__ __forceinline__ void wide_store_partial(const WideRows<D>& R, const WideState<D>& st, float* o, float* l,
                                                   int lane) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  if (!R.ok) return;
  const int h = lane >> 5;
  const float lt = st.l;
  const float muse = st.m == NEG_INF ? 0.f : st.m;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = {st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv, st.o[db][4 * j + 2] * inv,
                       st.o[db][4 * j + 3] * inv};
      float* dst = o + 32 * db + 8 * j + 4 * h;
      if constexpr (COHERENT) store_coherent4(dst, v);
      else *reinterpret_cast<f32x4*>(dst) = v;
    }
  if (h == 0) {
    if constexpr (COHERENT) store_coherent(l, lse);
    else *l = lse;
  }
}

// The fused KV append of one unit piece: the candidate rows r of (b, hkv) whose
// positions L + r fall in [lo, hi) (the piece's tokens) are copied from k_new /
// v_new ([B][Qmax][Hkv][D] bf16) into their paged slots, 16 bytes per thread
// and step, every load issued before the first store; the caller's barrier
// follows the wait here, so the piece's page copies see the rows.  Each row
// group of a unit writes the rows of the pieces it works (identical bytes), and
// only the piece that holds a page reads it, so no other workgroup waits.
template <int D, int NT>
__device__ __forceinline__ void wide_append_rows(const AttnArgs& a, int b, int hkv, int L, int qb, int lo, int hi,
                                                 int tid) {
  constexpr int CPR = D / 8;                                    // 16-byte chunks per row
  const int r0 = max(0, lo - L), r1 = min(qb, hi - L);
  if (r1 <= r0) return;
  const int n = 2 * (r1 - r0) * CPR;
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  for (int e0 = 0; e0 < n; e0 += 4 * NT) {
    uint4 val[4];
    int64_t dst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + tid + i * NT;
      if (e >= n) continue;
      const int which = e / ((r1 - r0) * CPR), r = r0 + (e / CPR) % (r1 - r0), c = e % CPR;
      const int t = L + r;
      const int64_t page = table[t / kPage];
      dst[i] = ((((page * a.Hkv + hkv) * kPage + t % kPage) * D + c * 8) << 1) | which;
      const int64_t src = (((int64_t)b * a.Qmax + r) * a.Hkv + hkv) * D + c * 8;
      val[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(which ? a.v_new : a.k_new) + src);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + tid + i * NT >= n) continue;
      void* cache = const_cast<void*>((dst[i] & 1) ? a.v : a.k);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(cache) + (dst[i] >> 1)) = val[i];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);    // this thread's stores have completed
}

// ------------------------------------------------------------ balanced grid
// Same page line, slices, row groups and partial slots as tile_balanced_kernel
// (pta_tile.hip); slice_merge_kernel merges the partials in a second launch.
template <int D, int NWR, int NBUF>
__global__ __launch_bounds__(NWR * 64) __attribute__((amdgpu_waves_per_eu(2))) void wide_balanced_kernel(AttnArgs a) {
  using Gm = WideGeom<D, NWR, NBUF>;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  __shared__ int wave_tot[NWR];
  extern __shared__ int ps[];       // [B + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.B;
  const int Rmax = a.G * a.Qmax;
  const int RG = (Rmax + NWR * 32 - 1) / (NWR * 32);
  const int blk = blockIdx.x;
  const int rg = (blk >> 3) % RG;
  const int64_t w = (int64_t)((blk >> 3) / RG) * 8 + (blk & 7);
  const int64_t NS = gridDim.x / RG;

  page_prefix<NWR * 64>(a, ps, wave_tot, tid);
  const int64_t Wl = (int64_t)a.Hkv * __builtin_amdgcn_readfirstlane(ps[B]);
  const int64_t N = min(NS, max((int64_t)1, Wl / kMinSlicePages));
  if (w >= N) return;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];
  const uint32_t pool = (uint32_t)((uint64_t)a.num_blocks * (uint64_t)a.Hkv * (uint64_t)Gm::TILE);
  const i32x4 krs = wide_rsrc(a.k, pool), vrs = wide_rsrc(a.v, pool);
  const int row0 = rg * NWR * 32;

  const int64_t x0 = w * Wl / N;
  const int64_t xe = (w + 1) * Wl / N;
  int64_t x = x0;
  while (x < xe) {
    const int key = (int)(x / a.Hkv);
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(ps[mid]) <= key) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo;
    const int psb = __builtin_amdgcn_readfirstlane(ps[b]);
    const int Pl = __builtin_amdgcn_readfirstlane(ps[b + 1]) - psb;   // unit length on the line
    const int64_t off = x - (int64_t)a.Hkv * psb;
    const int hkv = (int)(off / Pl);
    const int k0l = (int)(off % Pl);
    const int k1l = (int)min((int64_t)Pl, k0l + (xe - x));
    const int prog0 = (int)(x - x0) + max(0, a.slice_pad - k0l);   // slice progress at the first page
    x += k1l - k0l;
    // the unit's pages follow slice_pad positions of padding on the line
    const int Pb = Pl - a.slice_pad;
    const int k0 = max(0, k0l - a.slice_pad), k1 = max(0, k1l - a.slice_pad);
    if (k1 <= k0) continue;                  // only padding of this unit in the slice
    const int u = b * a.Hkv + hkv;
    const int C = a.ctx[b];
    const int qb = a.qlen[b];
    const int M = a.G * qb;

    // the step's KV append, for the candidates on this piece's pages (k_new set by the
    // fused entry); the barrier below orders it before the piece's page copies
    if (a.k_new != nullptr && row0 < M)
      wide_append_rows<D, NWR * 64>(a, b, hkv, C - qb, qb, k0 * kPage, min(C, k1 * kPage), tid);
    __syncthreads();          // LDS stage buffers free from the previous unit
    if (row0 < M) {
      WideRows<D> R;
      WideState<D> st;
      wide_range<D, NWR, NBUF>(a, lds, lds0, krs, vrs, R, st, b, hkv, qb, row0, k0 * kPage, min(C, k1 * kPage),
                               wave, lane, prog0, (int)(xe - x0));
      if (k0 == 0 && k1 == Pb) {
        wide_store_final<D>(a, R, st, b, lane);
      } else {
        const int64_t r = (w + u) * Rmax + row0 + wave * 32 + (lane & 31);
        wide_store_partial<D, false>(R, st, a.part_o + r * D, a.part_lse + r, lane);
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
// Occupancy query (a == nullptr) or launch of *nwg workgroups plus the slice
// merge, as tile_balanced.  Four stage buffers (three stages in flight) fit
// two workgroups per compute unit.
template <int D, int NWR>
static hipError_t wide_balanced_t(const AttnArgs* a, int B, int* nwg, hipStream_t s) {
  constexpr int NBUF = 4;
  const size_t dyn = (size_t)(B + 1) * sizeof(int);
  if (a == nullptr) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, wide_balanced_kernel<D, NWR, NBUF>, NWR * 64, dyn);
    if (e != hipSuccess) return e;
    *nwg = cus * (per > 0 ? per : 1);
    return hipSuccess;
  }
  hipLaunchKernelGGL((wide_balanced_kernel<D, NWR, NBUF>), dim3((unsigned)*nwg), dim3(NWR * 64), dyn, s, *a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int RG = (a->G * a->Qmax + NWR * 32 - 1) / (NWR * 32);
  return launch_slice_merge(*a, D, *nwg / RG, s);
}

hipError_t wide_balanced(const AttnArgs* a, int D, int nwr, int B, int* nwg, hipStream_t s) {
  if (D == 64) {
    if (nwr == 2) return wide_balanced_t<64, 2>(a, B, nwg, s);
    if (nwr == 4) return wide_balanced_t<64, 4>(a, B, nwg, s);
  } else if (D == 128) {
    if (nwr == 2) return wide_balanced_t<128, 2>(a, B, nwg, s);
    if (nwr == 4) return wide_balanced_t<128, 4>(a, B, nwg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
