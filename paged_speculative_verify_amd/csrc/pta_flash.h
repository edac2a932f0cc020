// Flash-attention building blocks shared by the matrix-core kernels (gfx950):
// page tiles staged in LDS as bf16 rows, the rows a lane owns, its online
// softmax state, the two-page update with v_mfma_f32_16x16x32_bf16 for both
// S^T = K Q^T and O^T += V^T P^T (V^T read with ds_read_b64_tr_b16), and the
// stores of final or partial rows.
//
// Lane (g, m) = (lane / 16, lane % 16) owns rows 16 rb + m of the unit and, in
// every 16-token page, tokens 4 g + r (r < 4) of the S^T accumulator; its O^T
// accumulators hold dims 16 db + 4 g + r of the same rows.
#pragma once

#include "pta_device.h"

namespace pta {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLazyTau = 8.0f;   // log2 headroom before a row's reference max moves
constexpr int kMinSlicePages = 8;  // balanced mode: fewest pages per wave slice

// Issue priority of the calling wave, 0 (lowest) .. 3.
__device__ __forceinline__ void set_priority(int level) {
  switch (level) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// Priority that falls as a wave gets through its share of a balanced grid's
// work (3 in the first quarter .. 0 in the last), so work-groups sharing a
// compute unit progress at the same pace instead of the oldest first.
__device__ __forceinline__ void pace(int done, int total) {
  if (total > 0) set_priority(3 - min(3, (int)((uint32_t)(4 * done) / (uint32_t)total)));
}

template <typename KT, int D>
struct StreamTile {
  static constexpr int KK = D / 32;                           // 16x16x32 k-steps over the head dim
  static constexpr int DB = D / 16;                           // 16-dim blocks of O^T
  static constexpr int LOADS = (kPage * D * KT::bytes) / 1024;     // 16-byte loads per lane per tile
  static constexpr int STR = 2 * D + 32;                      // bytes per bf16 row in LDS (bank skew)
  static constexpr int TILE_LDS = kPage * STR;                // one bf16 tile in LDS
  static constexpr int WAVE_LDS = 4 * TILE_LDS;               // per-wave K and V tiles of a page pair
};

// Write 1 KiB load chunk j of a page tile (lane l holds bytes 16 l + 1024 j)
// into a bf16 LDS tile (fp8 codes decoded exactly); rows at or past `valid`
// are zeroed when `partial`.
template <typename KT, int D>
__device__ __forceinline__ void stage_chunk(char* dst, uint4 w, int j, int lane, bool partial, int valid) {
  constexpr int STR = StreamTile<KT, D>::STR;
  const int byte = 1024 * j + 16 * lane;
  if constexpr (KT::bytes == 2) {
    const int t = byte / (2 * D), col = byte % (2 * D);
    if (partial) {
      if (t >= valid) w = make_uint4(0, 0, 0, 0);
    }
    *reinterpret_cast<uint4*>(dst + t * STR + col) = w;
  } else {
    const int t = byte / D, d0 = byte % D;
    uint4 lo, hi;
    lo.x = fp8x2_to_bf16x2<false>(w.x); lo.y = fp8x2_to_bf16x2<true>(w.x);
    lo.z = fp8x2_to_bf16x2<false>(w.y); lo.w = fp8x2_to_bf16x2<true>(w.y);
    hi.x = fp8x2_to_bf16x2<false>(w.z); hi.y = fp8x2_to_bf16x2<true>(w.z);
    hi.z = fp8x2_to_bf16x2<false>(w.w); hi.w = fp8x2_to_bf16x2<true>(w.w);
    if (partial) {
      if (t >= valid) { lo = make_uint4(0, 0, 0, 0); hi = lo; }
    }
    *reinterpret_cast<uint4*>(dst + t * STR + 2 * d0) = lo;
    *reinterpret_cast<uint4*>(dst + t * STR + 2 * d0 + 16) = hi;
  }
}

// All chunks of one page tile.
template <typename KT, int D>
__device__ __forceinline__ void stage_tile(char* dst, const uint4 (&c)[StreamTile<KT, D>::LOADS], int lane,
                                           bool partial, int valid) {
#pragma unroll
  for (int j = 0; j < StreamTile<KT, D>::LOADS; ++j) stage_chunk<KT, D>(dst, c[j], j, lane, partial, valid);
}

// The rows a lane owns (row = row0 + 16 rb + m of the unit): Q^T operands,
// candidate mask bits and output coordinates.
template <int D, int RB>
struct StreamRows {
  bf16x8 qop[RB][D / 32];
  uint64_t mbits[RB];
  bool ok[RB];
  int h[RB], i[RB];
};

template <int D, int RB>
__device__ __forceinline__ void load_rows(StreamRows<D, RB>& R, const AttnArgs& a, int b, int hkv, int qb,
                                          int M, int g, int m, int row0 = 0) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 16 + m;
    R.ok[rb] = row < M;
    R.h[rb] = hkv * a.G + (R.ok[rb] ? row / qb : 0);
    R.i[rb] = R.ok[rb] ? row % qb : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         (((int64_t)b * a.Qmax + R.i[rb]) * a.Hq + R.h[rb]) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const uint4 w = R.ok[rb] ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
      R.qop[rb][kk] = __builtin_bit_cast(bf16x8, w);
    }
    R.mbits[rb] = R.ok[rb] ? load_mask_row(a.mask, b, R.i[rb], qb, a.Qmax) : 0ull;
  }
  // A negative scale moves into the sign of Q (exact: every score just changes
  // sign), so the score scale c = |scale| log2(e) used below is positive.
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        uint4 w = __builtin_bit_cast(uint4, R.qop[rb][kk]);
        w.x ^= 0x80008000u;
        w.y ^= 0x80008000u;
        w.z ^= 0x80008000u;
        w.w ^= 0x80008000u;
        R.qop[rb][kk] = __builtin_bit_cast(bf16x8, w);
      }
  }
}

// Positive score scale (log2 units) of a page: |scale| log2(e) times the
// page's K scale, at least the smallest normal float (a zero scale then gives
// every visible token p = 1, as it should, and -inf scores stay -inf).
__device__ __forceinline__ float score_scale(const AttnArgs& a, float kscale) {
  return fmaxf(fabsf(a.scale_log2) * kscale, 1.17549435e-38f);
}

// Flash state of a lane's rows: O^T accumulators (dims 16 db + 4 g + r), the
// reference maximum (log2 units) and the partial row sum of this lane's tokens.
template <int D, int RB>
struct StreamState {
  f32x4 o[RB][D / 16];
  float m[RB], l[RB];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m[rb] = -__builtin_huge_valf();
      l[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[rb][db] = {};
    }
  }
};

// Byte offset of 16-byte unit `u` of row `r` in a bf16 LDS tile of D dims.
// Padded tiles put rows STR = 2 D + 32 bytes apart; swizzled tiles keep rows
// 2 D bytes apart (so a tile is contiguous, as direct global-to-LDS loads
// write it) and XOR the unit with the row, which spreads row-strided operand
// reads over the banks.
template <int D, bool SWZ>
__device__ __forceinline__ int tile_off(int r, int u) {
  if constexpr (SWZ) {
    constexpr int UPR = 2 * D / 16;           // 16-byte units per row
    return r * 2 * D + ((u ^ (r & (UPR - 1))) << 4);
  } else {
    return r * (2 * D + 32) + (u << 4);
  }
}

// Two consecutive pages of the flash update at once (tiles kl0/vl0 and
// kl1/vl1, first token at pbase): S^T = K Q^T per page, one lazy max check
// over both, and a single 32-token O^T += V^T P^T step with
// v_mfma_f32_16x16x32_bf16 (full rate on gfx950, where the 16-token
// instruction runs at half rate).  The k index of that step runs over tokens
// {4 g + e, 16 + 4 g + e} for lane group g: the B operand is the lane's two
// S^T accumulators (P in bf16, alone or as a hi/lo pair) and the A operand is two
// ds_read_b64_tr_b16 reads, one from each V tile.  A missing second page must
// be presented with its V tile zeroed and its tokens at or past t1 (masked).
template <int RB>
struct PairScores {
  f32x4 s[2][RB];     // [page][row block]: lane holds tokens 4 g + r of the page, row m
};

template <int D, int RB, bool SWZ>
__device__ __forceinline__ void pair_scores(const StreamRows<D, RB>& rows, PairScores<RB>& S,
                                            const char* kl0, const char* kl1, int lane) {
  constexpr int KK = D / 32;
  const int g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int pg = 0; pg < 2; ++pg)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) S.s[pg][rb] = {};
  // 2 * RB independent accumulation chains, interleaved
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kl0 + tile_off<D, SWZ>(m, 4 * kk + g));
    const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kl1 + tile_off<D, SWZ>(m, 4 * kk + g));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      S.s[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, rows.qop[rb][kk], S.s[0][rb], 0, 0, 0);
      S.s[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, rows.qop[rb][kk], S.s[1][rb], 0, 0, 0);
    }
  }
}

// ---- the same update split for a software pipeline (tile kernels).  Scores
// stay raw (q . k) until P is formed: the scale c > 0 (log2 units; a caller
// folds a negative scale into the sign of Q) enters the exponent,
// p = 2^(c s - m) in one fused multiply-add, and the reference maximum m is c
// times the raw maximum (rounding is monotonic, so that is the maximum of the
// scaled scores).  pair_mask sets the scores of invisible tokens to -inf and
// is only needed for pairs that reach the candidates or the end of the range;
// pair_max_prep takes lane maxima (straight-line, to share issue slots with
// matrix-core work); pair_max_finish moves m and l at once when needed and
// returns O's factor for later; pair_p forms P in bf16; and pair_pv_mma adds
// the P.V products.  The pipelined wide-tree kernels take P as one bf16 value
// per element (the usual precision of bf16 flash kernels): the row sum l stays
// in fp32, and the rounding moves an output by at most 2^-8 of the largest
// |V| of the row's context, by far less for spread attention; dropping the low
// half saves a third of their matrix-core work.
template <int D, int RB>
__device__ __forceinline__ void pair_mask(const StreamRows<D, RB>& rows, PairScores<RB>& S, int pbase, int L,
                                          int t1, int lane) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int g = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pg = e >> 2, r = e & 3;
      const int t = pbase + 16 * pg + 4 * g + r;
      const int sh = t - L;
      const bool cand = (unsigned)sh < 64u && ((rows.mbits[rb] >> (sh & 63)) & 1ull);
      S.s[pg][rb][r] = (t < t1 && (t < L || cand)) ? S.s[pg][rb][r] : NEG_INF;
    }
}

template <int D, int RB>
__device__ __forceinline__ void pair_max_prep(const StreamState<D, RB>& st, const PairScores<RB>& S,
                                              float (&x)[RB][8], bool& need, float c) {
  need = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[rb][e] = S.s[e >> 2][rb][e & 3];
    // NaN-propagating maximum (v_maximum3_f32): no quieting of the matrix-core
    // results first; masked scores are already -inf, visible ones finite
    auto mx = [](float u, float v) { return __builtin_elementwise_maximum(u, v); };
    const float pm = mx(mx(mx(x[rb][0], x[rb][1]), x[rb][2]), mx(mx(x[rb][3], x[rb][4]), x[rb][5]));
    const float pm2 = mx(pm, mx(x[rb][6], x[rb][7]));
    need |= c * pm2 > st.m[rb] + kLazyTau;
  }
}

// Returns true (wave-uniform) when some row's reference maximum moved; then
// alpha holds the factor O must be multiplied by before the products of this
// pair are added (l is rescaled here).
template <int D, int RB>
__device__ __forceinline__ bool pair_max_finish(StreamState<D, RB>& st, const float (&x)[RB][8], bool need,
                                                float (&alpha)[RB], float c) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  if (__builtin_amdgcn_ballot_w64(need) == 0) return false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float pm = x[rb][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) pm = fmaxf(pm, x[rb][e]);
    pm = fmaxf(pm, shfl_xor(pm, 16));
    pm = fmaxf(pm, shfl_xor(pm, 32));
    const float mnew = fmaxf(st.m[rb], c * pm);
    alpha[rb] = fast_exp2(st.m[rb] - (mnew == NEG_INF ? 0.f : mnew));
    st.m[rb] = mnew;
    st.l[rb] *= alpha[rb];
  }
  return true;
}

template <int D, int RB>
__device__ __forceinline__ void pair_p(StreamState<D, RB>& st, const float (&x)[RB][8], bf16x8 (&p)[RB],
                                       float c) {
  constexpr float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float nm = st.m[rb] == NEG_INF ? 0.f : -st.m[rb];
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = fast_exp2(fmaf(x[rb][2 * k], c, nm)), p1 = fast_exp2(fmaf(x[rb][2 * k + 1], c, nm));
      st.l[rb] += p0 + p1;
      h[k] = pack_bf16x2(p0, p1);
    }
    p[rb] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  }
}

template <int D, int RB, bool SWZ, bool LO = true>
__device__ __forceinline__ void pair_pv_mma(StreamState<D, RB>& st, const bf16x8 (&phi)[RB],
                                            const bf16x8 (&plo)[RB], const char* vl0, const char* vl1,
                                            int lane) {
  constexpr int DB = D / 16;
  const int g = lane >> 4, m = lane & 15;
  const int vrow = 4 * g + (m >> 2);
#pragma unroll
  for (int db = 0; db < DB; db += 2) {
    bf16x8 vt[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int voff = tile_off<D, SWZ>(vrow, 2 * (db + e) + ((m & 3) >> 1)) + 8 * (m & 1);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl0 + voff));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl1 + voff));
      vt[e] = __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint2, va).x,
                                                   __builtin_bit_cast(uint2, va).y,
                                                   __builtin_bit_cast(uint2, vb).x,
                                                   __builtin_bit_cast(uint2, vb).y));
    }
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        st.o[rb][db + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[e], phi[rb], st.o[rb][db + e], 0, 0, 0);
    if constexpr (LO) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          st.o[rb][db + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[e], plo[rb], st.o[rb][db + e], 0, 0, 0);
    }
  }
}

// The whole update of one pair for kernels that do not pipeline it: page
// score scales c0, c1 > 0 (score_scale), V scales vs0, vs1 folded into P when
// VS (fp8 pages).  Raw maxima are taken per page and scaled once.  fp8 pages
// take P as bf16 alone (no low half): the extra rounding moves the output by
// at most 2^-9 of the page's largest |V|, far below the error fp8 storage of
// V itself carries, and it saves a third of the matrix-core work.
template <int D, int RB, bool SWZ, bool VS>
__device__ __forceinline__ void pair_compute(const StreamRows<D, RB>& rows, StreamState<D, RB>& st,
                                             const char* kl0, const char* kl1, const char* vl0,
                                             const char* vl1, int pbase, int L, int t1, float c0,
                                             float c1, float vs0, float vs1, int lane) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int DB = D / 16;
  PairScores<RB> S;
  pair_scores<D, RB, SWZ>(rows, S, kl0, kl1, lane);
  if (pbase + 2 * kPage > min(L, t1)) pair_mask<D, RB>(rows, S, pbase, L, t1, lane);
  auto mx = [](float u, float v) { return __builtin_elementwise_maximum(u, v); };
  float xm[RB];
  bool need = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float pm0 = mx(mx(S.s[0][rb][0], S.s[0][rb][1]), mx(S.s[0][rb][2], S.s[0][rb][3]));
    const float pm1 = mx(mx(S.s[1][rb][0], S.s[1][rb][1]), mx(S.s[1][rb][2], S.s[1][rb][3]));
    xm[rb] = fmaxf(c0 * pm0, c1 * pm1);
    need |= xm[rb] > st.m[rb] + kLazyTau;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float pm = xm[rb];
      pm = fmaxf(pm, shfl_xor(pm, 16));
      pm = fmaxf(pm, shfl_xor(pm, 32));
      const float mnew = fmaxf(st.m[rb], pm);
      const float alpha = fast_exp2(st.m[rb] - (mnew == NEG_INF ? 0.f : mnew));
      st.m[rb] = mnew;
      st.l[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) st.o[rb][db] *= alpha;
    }
  }
  bf16x8 phi[RB], plo[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float nm = st.m[rb] == NEG_INF ? 0.f : -st.m[rb];
    uint32_t h[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pg = k >> 1;
      const float c = pg ? c1 : c0;
      float p0 = fast_exp2(fmaf(S.s[pg][rb][(2 * k) & 3], c, nm));
      float p1 = fast_exp2(fmaf(S.s[pg][rb][(2 * k + 1) & 3], c, nm));
      st.l[rb] += p0 + p1;
      if constexpr (VS) {
        const float v = pg ? vs1 : vs0;
        p0 *= v;
        p1 *= v;
      }
      h[k] = pack_bf16x2(p0, p1);
      if constexpr (!VS) lo[k] = pack_bf16x2(p0 - bf16_lo(h[k]), p1 - bf16_hi(h[k]));
      else lo[k] = 0u;
    }
    phi[rb] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    plo[rb] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
  }
  pair_pv_mma<D, RB, SWZ, !VS>(st, phi, plo, vl0, vl1, lane);
}

// Row sums over the lane's four 16-lane groups (every group holds 4 of each
// page's 16 tokens).
template <int D, int RB>
__device__ __forceinline__ void reduce_row_sums(StreamState<D, RB>& st) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st.l[rb] += shfl_xor(st.l[rb], 16);
    st.l[rb] += shfl_xor(st.l[rb], 32);
  }
}

// Final rows of a lane: out = O / l (bf16), lse = ln l + max.
template <int D, int RB>
__device__ __forceinline__ void store_final_rows(const AttnArgs& a, const StreamRows<D, RB>& rows,
                                                 const StreamState<D, RB>& st, int b, int g) {
  constexpr float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rows.ok[rb]) continue;
    const float lt = st.l[rb];
    const float muse = st.m[rb] == NEG_INF ? 0.f : st.m[rb];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
    const int h = rows.h[rb], i = rows.i[rb];
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (((int64_t)b * a.Qmax + i) * a.Hq + h) * D + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      uint2 w;
      w.x = pack_bf16x2(st.o[rb][db][0] * inv, st.o[rb][db][1] * inv);
      w.y = pack_bf16x2(st.o[rb][db][2] * inv, st.o[rb][db][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * db) = w;
    }
    if (g == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.Hq + h) * a.Qmax + i] = lse;
  }
}

// Partial rows of a lane (normalised O and natural-log LSE), stored with
// device-coherent word stores.  row_addr(rb, o, l) gives the row's O words and
// LSE word.
template <int D, int RB, typename AddrFn>
__device__ __forceinline__ void store_partial_rows(const StreamRows<D, RB>& rows,
                                                   const StreamState<D, RB>& st, int g, AddrFn row_addr) {
  constexpr float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rows.ok[rb]) continue;
    const float lt = st.l[rb];
    const float muse = st.m[rb] == NEG_INF ? 0.f : st.m[rb];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
    float* o;
    float* l;
    row_addr(rb, o, l);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) store_coherent4(o + 16 * db + 4 * g, st.o[rb][db] * inv);
    if (g == 0) store_coherent(l, lse);
  }
}

}  // namespace pta
