// Matrix-core paged tree attention for few rows per KV head (M = G * q_len
// <= 32: GQA decode and short candidate chains).  The verify step turns each
// sequence's decode GEMV into a small GEMM (TACO-LLM design talk
// "大模型倍速推理引擎 TACO-LLM 的设计与实践", TurboAttention bullets of
// "整体方案分为两大部分"); with so few rows the work is a pure HBM stream, and
// the kernel is written so that almost nothing but the page loads costs time:
//
//   * Work unit = (sequence, KV head, token partition).  Every query row of the
//     unit (the GQA group's q-heads times the candidates) is handled by every
//     wave, so each KV page tile crosses HBM once per group.  The NW waves of
//     the workgroup take the unit's pages round-robin, each wave with its own
//     flash-style softmax state (on-chip state independent of the context
//     length, "优化策略总结" item 2); the waves are merged in LDS at the end.
//   * No barrier in the main loop.  K is loaded from HBM straight into the
//     A-operand layout of v_mfma_f32_16x16x32_bf16 (lane (g, m) holds 8
//     consecutive dims of token m), so S^T = K Q^T needs no LDS.  V is copied
//     into a per-wave LDS tile and read back with ds_read_b64_tr_b16, whose
//     16-lane transpose yields exactly the A operand of O^T += V^T P^T
//     (v_mfma_f32_16x16x16_bf16); P^T is the S^T accumulator itself.
//   * The next page's loads are issued before the current page is computed
//     (two register sets, ping-pong), keeping one page per wave in flight.
//   * Softmax rescaling is lazy: a row's reference maximum only moves when a
//     score exceeds it by more than 2^8, so the accumulator rescale (and the
//     cross-lane max) is skipped on almost every page.  The result is the same
//     exact softmax; terms are bounded by 2^8 so nothing overflows.
//   * fp8 e4m3fn pages are decoded to bf16 exactly on the way in (the pages'
//     fast dequantisation inside attention, 618zxw.cn article section
//     "LLM量子化技術による推論コストの削減"); the per-(page, KV head) scales
//     are folded into the score multiplier and into P.
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLazyTau = 8.0f;   // log2 headroom before a row's reference max moves

template <typename KT, int D>
struct StreamTile {
  static constexpr int KK = D / 32;                           // 16x16x32 k-steps over the head dim
  static constexpr int DB = D / 16;                           // 16-dim blocks of O^T
  static constexpr int K_LOADS = KK;                          // per lane per page
  static constexpr int V_LOADS = (kPage * D * KT::bytes) / 1024;   // 16-byte loads per lane per page
  static constexpr int VSTR = 2 * D + 32;                     // bytes per bf16 V row in LDS (bank skew)
  static constexpr int V_BYTES = kPage * VSTR;                // per-wave V tile
};

template <typename KT>
struct KChunk;
template <>
struct KChunk<BF16> {
  using raw = uint4;
  static __device__ __forceinline__ raw load(const char* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ bf16x8 op(const raw& r) { return __builtin_bit_cast(bf16x8, r); }
};
template <>
struct KChunk<FP8> {
  using raw = uint2;
  static __device__ __forceinline__ raw load(const char* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ bf16x8 op(const raw& r) {
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(r.x);
    o.y = fp8x2_to_bf16x2<true>(r.x);
    o.z = fp8x2_to_bf16x2<false>(r.y);
    o.w = fp8x2_to_bf16x2<true>(r.y);
    return __builtin_bit_cast(bf16x8, o);
  }
};

// One page's operands in flight.
template <typename KT, int D>
struct PageRegs {
  typename KChunk<KT>::raw k[StreamTile<KT, D>::K_LOADS];
  uint4 v[StreamTile<KT, D>::V_LOADS];
  float ks, vs;
};

template <typename KT, int D, int RB, int NW>
__global__ __launch_bounds__(NW * 64) void stream_attn_kernel(AttnArgs a) {
  using T = StreamTile<KT, D>;
  using KC = KChunk<KT>;
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int ROWS = 16 * RB;

  __shared__ __attribute__((aligned(16))) char vlds[NW][T::V_BYTES];
  __shared__ float red_m[NW][ROWS];
  __shared__ float red_l[NW][ROWS];
  static_assert(NW == 1 || RB * T::DB * 64 * 16 <= NW * T::V_BYTES, "merge buffer must fit the V tiles");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4;          // 16-lane group
  const int m = lane & 15;          // lane within the group
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

  // ---- rows of this lane (row = 16 rb + m) and their Q^T operands
  bf16x8 qop[RB][T::KK];
  uint64_t mbits[RB];
  bool row_ok[RB];
  int row_h[RB], row_i[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rb * 16 + m;
    row_ok[rb] = row < M;
    row_h[rb] = hkv * a.G + (row_ok[rb] ? row / qb : 0);
    row_i[rb] = row_ok[rb] ? row % qb : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         (((int64_t)b * a.Qmax + row_i[rb]) * a.Hq + row_h[rb]) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const uint4 w = row_ok[rb] ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
      qop[rb][kk] = __builtin_bit_cast(bf16x8, w);
    }
    mbits[rb] = row_ok[rb] ? load_mask_row(a.mask, b, row_i[rb], qb, a.Qmax) : 0ull;
  }

  // ---- this wave's pages: pg = pgA + wave + k * NW, k < nk
  const int pgA = t0 / kPage;
  const int npg = (t1 + kPage - 1) / kPage - pgA;
  const int nk = npg > wave ? (npg - wave + NW - 1) / NW : 0;
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  constexpr int64_t TILE_BYTES = (int64_t)kPage * D * KT::bytes;
  constexpr int ROW_BYTES = D * KT::bytes;

  // physical block of this wave's page k (wave-uniform: a scalar load)
  auto phys_of = [&](int k) -> int { return table[pgA + wave + k * NW]; };

  auto issue = [&](PageRegs<KT, D>& R, int phys32) {
    const int64_t phys = phys32;
    const int64_t tile = (phys * a.Hkv + hkv) * TILE_BYTES;
    const char* kp = kbase + tile + m * ROW_BYTES + 8 * g * KT::bytes;
#pragma unroll
    for (int kk = 0; kk < T::K_LOADS; ++kk) R.k[kk] = KC::load(kp + 32 * kk * KT::bytes);
    const char* vp = vbase + tile + 16 * lane;
#pragma unroll
    for (int j = 0; j < T::V_LOADS; ++j) R.v[j] = *reinterpret_cast<const uint4*>(vp + 1024 * j);
    if constexpr (KT::bytes == 1) {
      R.ks = a.k_scale[phys * a.Hkv + hkv];
      R.vs = a.v_scale[phys * a.Hkv + hkv];
    } else {
      R.ks = 1.f;
      R.vs = 1.f;
    }
  };

  f32x4 oacc[RB][T::DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = NEG_INF;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) oacc[rb][db] = {};
  }
  char* vl = vlds[wave];

  auto consume = [&](const PageRegs<KT, D>& R, int k) {
    const int pg = pgA + wave + k * NW;
    const int pbase = pg * kPage;
    const bool partial = pbase + kPage > t1;

    // 1. V tile -> LDS as bf16 rows (tail slots past the context are zeroed)
    if constexpr (KT::bytes == 2) {
#pragma unroll
      for (int j = 0; j < T::V_LOADS; ++j) {
        const int byte = 1024 * j + 16 * lane;
        const int t = byte / (2 * D), col = byte % (2 * D);
        uint4 w = R.v[j];
        if (partial) {
          if (pbase + t >= t1) w = make_uint4(0, 0, 0, 0);
        }
        *reinterpret_cast<uint4*>(vl + t * T::VSTR + col) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::V_LOADS; ++j) {
        const int byte = 1024 * j + 16 * lane;
        const int t = byte / D, d0 = byte % D;
        const uint4 c = R.v[j];
        uint4 lo, hi;
        lo.x = fp8x2_to_bf16x2<false>(c.x); lo.y = fp8x2_to_bf16x2<true>(c.x);
        lo.z = fp8x2_to_bf16x2<false>(c.y); lo.w = fp8x2_to_bf16x2<true>(c.y);
        hi.x = fp8x2_to_bf16x2<false>(c.z); hi.y = fp8x2_to_bf16x2<true>(c.z);
        hi.z = fp8x2_to_bf16x2<false>(c.w); hi.w = fp8x2_to_bf16x2<true>(c.w);
        if (partial) {
          if (pbase + t >= t1) { lo = make_uint4(0, 0, 0, 0); hi = lo; }
        }
        *reinterpret_cast<uint4*>(vl + t * T::VSTR + 2 * d0) = lo;
        *reinterpret_cast<uint4*>(vl + t * T::VSTR + 2 * d0 + 16) = hi;
      }
    }

    // 2. S^T[16 tokens][16 rows] = K Q^T per row block
    f32x4 sacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = {};
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const bf16x8 kop = KC::op(R.k[kk]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[rb][kk], sacc[rb], 0, 0, 0);
    }

    // 3. scores in log2 units, mask by select; lazy reference-max update
    const float c = a.scale_log2 * R.ks;
    const bool plain = pbase + kPage <= min(L, t1);
    float x[RB][4];
    bool need = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float pm = NEG_INF;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sacc[rb][r] * c;
        if (!plain) {
          const int t = pbase + 4 * g + r;
          const int sh = t - L;
          const bool cand = (unsigned)sh < 64u && ((mbits[rb] >> (sh & 63)) & 1ull);
          v = (t < t1 && (t < L || cand)) ? v : NEG_INF;
        }
        v = row_ok[rb] ? v : NEG_INF;
        x[rb][r] = v;
        pm = fmaxf(pm, v);
      }
      need |= pm > m_run[rb] + kLazyTau;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float pm = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
        pm = fmaxf(pm, shfl_xor(pm, 16));
        pm = fmaxf(pm, shfl_xor(pm, 32));
        const float mnew = fmaxf(m_run[rb], pm);
        const float alpha = fast_exp2(m_run[rb] - (mnew == NEG_INF ? 0.f : mnew));
        m_run[rb] = mnew;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) oacc[rb][db] *= alpha;
      }
    }

    // 4. P^T (bf16) straight from the S^T registers; O^T += V^T P^T
    s16x4 pop[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float muse = m_run[rb] == NEG_INF ? 0.f : m_run[rb];
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(x[rb][r] - muse);
        l_run[rb] += p[r];
      }
      const uint32_t w0 = pack_bf16x2(p[0] * R.vs, p[1] * R.vs);
      const uint32_t w1 = pack_bf16x2(p[2] * R.vs, p[3] * R.vs);
      pop[rb] = __builtin_bit_cast(s16x4, make_uint2(w0, w1));
    }
    const char* vrd = vl + (4 * g + (m >> 2)) * T::VSTR + 8 * (m & 3);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrd + 32 * db));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pop[rb], oacc[rb][db], 0, 0, 0);
    }
  };

  // ---- main loop: two register sets, the next page always in flight.  The
  // prefetch is issued unconditionally (the last one re-reads the final page,
  // which is still in cache) so the compiler's load counters stay exact and
  // the wait before each page covers only that page's own loads.
  PageRegs<KT, D> r0, r1;
  if (nk > 0) {
    // block-table entries are read two pages ahead of their use
    int ph_a = phys_of(0), ph_b = phys_of(min(1, nk - 1));
    issue(r0, ph_a);
    for (int k = 0;; k += 2) {
      ph_a = phys_of(min(k + 2, nk - 1));
      issue(r1, ph_b);
      consume(r0, k);
      if (k + 1 >= nk) break;
      ph_b = phys_of(min(k + 3, nk - 1));
      issue(r0, ph_a);
      consume(r1, k + 1);
      if (k + 2 >= nk) break;
    }
  }

  // ---- merge the waves: row max, row sum, then O^T accumulated in LDS in wave order
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += shfl_xor(l_run[rb], 16);
    l_run[rb] += shfl_xor(l_run[rb], 32);
  }
  float Ltot[RB], Muse[RB];
  if constexpr (NW > 1) {
    if (g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        red_m[wave][rb * 16 + m] = m_run[rb];
        red_l[wave][rb * 16 + m] = l_run[rb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = NEG_INF;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_m[w][rb * 16 + m]);
      Muse[rb] = mx == NEG_INF ? 0.f : mx;
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) lt += red_l[w][rb * 16 + m] * fast_exp2(red_m[w][rb * 16 + m] - Muse[rb]);
      Ltot[rb] = lt;
      const float f = fast_exp2(m_run[rb] - Muse[rb]);
#pragma unroll
      for (int db = 0; db < T::DB; ++db) oacc[rb][db] *= f;
    }
    f32x4* ob = reinterpret_cast<f32x4*>(&vlds[0][0]);   // V tiles are dead after the barrier
    for (int w = 0; w < NW; ++w) {
      if (wave == w) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < T::DB; ++db) {
            f32x4& slot = ob[(rb * T::DB + db) * 64 + lane];
            if (w > 0) oacc[rb][db] += slot;
            if (w < NW - 1) slot = oacc[rb][db];
          }
      }
      if (w < NW - 1) __syncthreads();
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      Muse[rb] = m_run[rb] == NEG_INF ? 0.f : m_run[rb];
      Ltot[rb] = l_run[rb];
    }
  }

  // ---- epilogue (last wave): row 16 rb + m, dims 16 db + 4 g + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (wave != NW - 1 || !row_ok[rb]) continue;
    const float lt = Ltot[rb];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (Muse[rb] + fast_log2(lt)) * kLn2 : NEG_INF;
    const int h = row_h[rb], i = row_i[rb];
    if (split_out) {
      const int64_t prow = (((int64_t)b * a.Hq + h) * a.Qmax + i) * a.num_parts + part;
      float* op = a.part_o + prow * D + 4 * g;
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_coherent(op + 16 * db + e, oacc[rb][db][e] * inv);
      if (g == 0) store_coherent(a.part_lse + prow, lse);
    } else {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (((int64_t)b * a.Qmax + i) * a.Hq + h) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        uint2 w;
        w.x = pack_bf16x2(oacc[rb][db][0] * inv, oacc[rb][db][1] * inv);
        w.y = pack_bf16x2(oacc[rb][db][2] * inv, oacc[rb][db][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * db) = w;
      }
      if (g == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.Hq + h) * a.Qmax + i] = lse;
    }
  }
  if (split_out) splitk_finish<BF16, D>(a, b, hkv, C, qb);
}

// ---------------------------------------------------------------- launchers
template <typename KT, int D, int RB, int NW>
static hipError_t launch_stream_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((stream_attn_kernel<KT, D, RB, NW>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename KT, int D>
static hipError_t launch_stream_d(const AttnArgs& a, int rb, int nw, dim3 grid, hipStream_t s) {
  if (rb == 1 && nw == 4) return launch_stream_t<KT, D, 1, 4>(a, grid, s);
  if (rb == 2 && nw == 4) return launch_stream_t<KT, D, 2, 4>(a, grid, s);
  if (rb == 1 && nw == 8) return launch_stream_t<KT, D, 1, 8>(a, grid, s);
  if (rb == 2 && nw == 8) return launch_stream_t<KT, D, 2, 8>(a, grid, s);
  if (rb == 1 && nw == 1) return launch_stream_t<KT, D, 1, 1>(a, grid, s);
  if (rb == 2 && nw == 1) return launch_stream_t<KT, D, 2, 1>(a, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const AttnArgs& a, int kv_dtype, int D, int rb, int nw, dim3 grid,
                         hipStream_t s) {
  if (kv_dtype == 1) {
    if (D == 64) return launch_stream_d<BF16, 64>(a, rb, nw, grid, s);
    if (D == 128) return launch_stream_d<BF16, 128>(a, rb, nw, grid, s);
  } else if (kv_dtype == 2) {
    if (D == 64) return launch_stream_d<FP8, 64>(a, rb, nw, grid, s);
    if (D == 128) return launch_stream_d<FP8, 128>(a, rb, nw, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
