// Vector-ALU paged tree attention for small row counts per KV head
// (M = G * q_len <= 8, e.g. GQA decode).  With so few rows the contraction is
// too thin for matrix cores; the kernel is an HBM stream and is written to
// keep many 16-byte page loads in flight.
//
// Work unit = (sequence b, KV head, token partition): every q-head of the GQA
// group and every candidate of the sequence is processed by the same
// workgroup, so each KV page tile is read from HBM once per group.  Waves of
// the workgroup take the unit's pages round-robin, each with its own
// online-softmax state (FlashAttention-style streaming: on-chip state does not
// grow with the context), and are merged through LDS at the end.
//
// Page tile (16 tokens x D) is read with 16-byte loads; one load instruction
// of a wave covers 1 KiB of the tile contiguously.  Lane layout: LPT lanes
// share one token (each owning EPL consecutive dims), TPL = 64 / LPT tokens per
// load, NL = 16 / TPL loads per page.  Partial dot products are reduced across
// the LPT lanes with butterfly shuffles.
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

template <typename KT>
struct KvLane {
  static constexpr int EPL = 16 / KT::bytes;     // elements per 16-byte load
};

// decode one 16-byte chunk (EPL elements) into floats
template <typename KT>
__device__ __forceinline__ void decode_chunk(const uint4& c, float* f);

template <>
__device__ __forceinline__ void decode_chunk<F32>(const uint4& c, float* f) {
  f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
}
template <>
__device__ __forceinline__ void decode_chunk<BF16>(const uint4& c, float* f) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) { f[2 * k] = bf16_lo(w[k]); f[2 * k + 1] = bf16_hi(w[k]); }
}
template <>
__device__ __forceinline__ void decode_chunk<FP8>(const uint4& c, float* f) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f32x2 lo = fp8x2_to_f32<false>(w[k]);
    f32x2 hi = fp8x2_to_f32<true>(w[k]);
    f[4 * k] = lo[0]; f[4 * k + 1] = lo[1]; f[4 * k + 2] = hi[0]; f[4 * k + 3] = hi[1];
  }
}

template <typename QT>
__device__ __forceinline__ float load_q(const void* q, int64_t idx);
template <>
__device__ __forceinline__ float load_q<F32>(const void* q, int64_t idx) {
  return reinterpret_cast<const float*>(q)[idx];
}
template <>
__device__ __forceinline__ float load_q<BF16>(const void* q, int64_t idx) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(q)[idx] << 16);
}

template <typename QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<F32>(void* out, int64_t idx, float v) {
  reinterpret_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<BF16>(void* out, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}

template <typename QT, typename KT, int D, int MR, int NW>
__global__ __launch_bounds__(NW * 64) void valu_attn_kernel(AttnArgs a) {
  constexpr int EPL = KvLane<KT>::EPL;
  constexpr int LPT = D / EPL;          // lanes per token
  constexpr int TPL = 64 / LPT;         // tokens per load instruction
  constexpr int NL = kPage / TPL;       // load instructions per page tile
  static_assert(LPT >= 1 && LPT <= 64 && NL >= 1, "bad lane layout");
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ float sm_m[NW][MR];
  __shared__ float sm_l[NW][MR];
  __shared__ float sm_acc[NW][MR][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int dsl = lane % LPT;           // dim slice owned by this lane
  const int tl = lane / LPT;            // token within a load
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  const int L = C - qb;
  const int M = a.G * qb;               // rows of this unit
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;               // partition past this sequence's context
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly

  // rows: r = g * qb + i  ->  q-head hkv * G + g, candidate i
  float qv[MR][EPL];
  uint64_t mbits[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const bool ok = r < M;
    const int g = ok ? r / qb : 0, i = ok ? r % qb : 0;
    const int64_t base = (((int64_t)b * a.Qmax + i) * a.Hq + hkv * a.G + g) * D + dsl * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[r][e] = ok ? load_q<QT>(a.q, base + e) : 0.f;
    mbits[r] = ok ? load_mask_row(a.mask, b, i, qb, a.Qmax) : 0ull;
  }

  float m[MR], l[MR], acc[MR][EPL];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    m[r] = NEG_INF;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
  }

  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const int pg0 = t0 / kPage, pg1 = (t1 + kPage - 1) / kPage;

  for (int pg = pg0 + wave; pg < pg1; pg += NW) {
    const int64_t phys = table[pg];
    const int64_t tile = (phys * a.Hkv + hkv) * (int64_t)(kPage * D * KT::bytes);
    uint4 kr[NL], vr[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kr[j] = *reinterpret_cast<const uint4*>(kbase + tile + j * 1024 + lane * 16);
      vr[j] = *reinterpret_cast<const uint4*>(vbase + tile + j * 1024 + lane * 16);
    }
    float kscale = 1.f, vscale = 1.f;
    if constexpr (KT::bytes == 1) {
      kscale = a.k_scale[phys * a.Hkv + hkv];
      vscale = a.v_scale[phys * a.Hkv + hkv];
    }

    // scores (partial over this lane's dims, then reduced over the LPT lanes)
    float s[NL][MR];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float kf[EPL];
      decode_chunk<KT>(kr[j], kf);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qv[r][e], kf[e], d);
        s[j][r] = d;
      }
    }
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int r = 0; r < MR; ++r) s[j][r] = wave_sum_range<1, LPT>(s[j][r]);

    // scale, mask (select, never arithmetic on masked values), page max
    const float sl = a.scale_log2 * kscale;
    const bool plain = (pg + 1) * kPage <= min(L, t1);   // whole page committed and in range
    float pmax[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) pmax[r] = NEG_INF;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int t = pg * kPage + j * TPL + tl;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        float x = s[j][r] * sl;
        if (!plain) {
          const int sh = t - L;
          const bool cand = (unsigned)sh < 64u && ((mbits[r] >> (sh & 63)) & 1ull);
          x = (t < t1 && (t < L || cand)) ? x : NEG_INF;
        }
        s[j][r] = x;
        pmax[r] = fmaxf(pmax[r], x);
      }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      pmax[r] = wave_max_range<LPT, 64>(pmax[r]);
      const float mnew = fmaxf(m[r], pmax[r]);
      const float muse = mnew == NEG_INF ? 0.f : mnew;
      const float alpha = fast_exp2(m[r] - muse);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        s[j][r] = fast_exp2(s[j][r] - muse);
        psum += s[j][r];
      }
      l[r] = l[r] * alpha + psum;
      m[r] = mnew;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] *= alpha;
    }

    // acc += p * V   (slots past the context may hold anything, so their V is zeroed)
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float vf[EPL];
      decode_chunk<KT>(vr[j], vf);
      if (!plain && pg * kPage + j * TPL + tl >= t1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float p = s[j][r] * vscale;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = fmaf(p, vf[e], acc[r][e]);
      }
    }
  }

  // combine the token groups of the wave (lanes with equal dsl)
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    l[r] = wave_sum_range<LPT, 64>(l[r]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[r][e] = wave_sum_range<LPT, 64>(acc[r][e]);
  }
  if (tl == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][dsl * EPL + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r) { sm_m[wave][r] = m[r]; sm_l[wave][r] = l[r]; }
  }
  __syncthreads();

  // merge the waves and write this unit's rows
  for (int idx = threadIdx.x; idx < MR * D; idx += NW * 64) {
    const int r = idx / D, d = idx % D;
    if (r >= M) continue;
    float mx = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w][r]);
    const float muse = mx == NEG_INF ? 0.f : mx;
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w][r] - muse);
      lt += f * sm_l[w][r];
      ot += f * sm_acc[w][r][d];
    }
    const float o = lt > 0.f ? ot / lt : 0.f;
    const float lse = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
    const int g = r / qb, i = r % qb, h = hkv * a.G + g;
    if (split_out) {
      const int64_t row = (((int64_t)b * a.Hq + h) * a.Qmax + i) * a.num_parts + part;
      store_coherent(a.part_o + row * D + d, o);
      if (d == 0) store_coherent(a.part_lse + row, lse);
    } else {
      store_out<QT>(a.out, (((int64_t)b * a.Qmax + i) * a.Hq + h) * D + d, o);
      if (d == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.Hq + h) * a.Qmax + i] = lse;
    }
  }
  if (split_out) splitk_finish<QT, D>(a, b, hkv, C, qb);
}

// ---------------------------------------------------------------- launchers
template <typename QT, typename KT, int D, int MR>
static hipError_t launch_valu_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NW = 4;
  hipLaunchKernelGGL((valu_attn_kernel<QT, KT, D, MR, NW>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename QT, typename KT, int D>
static hipError_t launch_valu_d(const AttnArgs& a, int mr, dim3 grid, hipStream_t s) {
  switch (mr) {
    case 1: return launch_valu_t<QT, KT, D, 1>(a, grid, s);
    case 2: return launch_valu_t<QT, KT, D, 2>(a, grid, s);
    case 4: return launch_valu_t<QT, KT, D, 4>(a, grid, s);
    case 8: return launch_valu_t<QT, KT, D, 8>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

template <typename QT, typename KT>
static hipError_t launch_valu_k(const AttnArgs& a, int D, int mr, dim3 grid, hipStream_t s) {
  if (D == 64) return launch_valu_d<QT, KT, 64>(a, mr, grid, s);
  if (D == 128) return launch_valu_d<QT, KT, 128>(a, mr, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_valu(const AttnArgs& a, int q_dtype, int kv_dtype, int D, int mr, dim3 grid,
                       hipStream_t s) {
  if (q_dtype == 0 && kv_dtype == 0) return launch_valu_k<F32, F32>(a, D, mr, grid, s);
  if (q_dtype == 1 && kv_dtype == 1) return launch_valu_k<BF16, BF16>(a, D, mr, grid, s);
  if (q_dtype == 1 && kv_dtype == 2) return launch_valu_k<BF16, FP8>(a, D, mr, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pta
