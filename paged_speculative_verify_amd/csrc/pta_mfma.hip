// Matrix-core paged tree attention for row counts per KV head that make a
// real contraction (M = G * q_len of several tens to hundreds).  Lookahead
// turns each sequence's decode GEMV into a small GEMM whose rows are the GQA
// group's q-heads times the candidates (TACO-LLM design talk
// "大模型倍速推理引擎 TACO-LLM 的设计与实践", TurboAttention bullets of
// "整体方案分为两大部分").
//
// gfx950 design:
//   * Work unit = (sequence, KV head, token partition).  The workgroup has one
//     wave per 32 rows; row r is (group member r / q_b, candidate r % q_b).
//   * A stage is 32 tokens (two 16-token pages).  The workgroup copies the
//     stage's K tile [32][D] and V tile into LDS, V stored transposed
//     (V^T[D][32]) so the PV operand reads are 8-byte vectors; fp8 codes are
//     decoded to bf16 on the way in (exact) and their per-page scale is
//     applied to the score / probability columns.  The next stage's global
//     loads are issued before the current stage is computed (register
//     prefetch + two LDS buffers, one barrier per stage).
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K
//     from LDS, B = Q^T held in registers for the whole unit), so every lane
//     owns one row (column of S^T) and 16 of the 32 tokens: the row max needs
//     one cross-lane step.  Online softmax in the log2 domain with the scale
//     folded into one multiply; masking by select.  Then O^T += V^T P^T with
//     the same instruction (A = V^T from LDS, B = P^T straight from the S^T
//     accumulator registers rounded to bf16).
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

template <int D>
struct MfmaTile {
  static constexpr int KROW = D + 8;        // bf16 elements per K row in LDS (bank skew)
  static constexpr int VROW = 32 + 4;       // bf16 elements per V^T row in LDS
  static constexpr int K_ELEMS = 32 * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = D / 8;      // 8-element chunks per token row
  static constexpr int ITEMS = 16 * CHUNKS; // (token pair, chunk) items per stage
};

// 8 consecutive KV elements of one token as 8 bf16 (4 x uint32)
template <typename KT>
struct Chunk8;
template <>
struct Chunk8<BF16> {
  using raw = uint4;
  static __device__ __forceinline__ raw load(const char* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ uint4 to_bf16(const raw& r) { return r; }
};
template <>
struct Chunk8<FP8> {
  using raw = uint2;
  static __device__ __forceinline__ raw load(const char* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ uint4 to_bf16(const raw& r) {
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(r.x);
    o.y = fp8x2_to_bf16x2<true>(r.x);
    o.z = fp8x2_to_bf16x2<false>(r.y);
    o.w = fp8x2_to_bf16x2<true>(r.y);
    return o;
  }
};

template <typename KT, int D, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) void mfma_attn_kernel(AttnArgs a) {
  using T = MfmaTile<D>;
  using CK = Chunk8<KT>;
  constexpr int NT = NWAVE * 64;
  constexpr int IPT = (T::ITEMS + NT - 1) / NT;     // items per thread per stage
  constexpr int KSTEPS = D / 16;
  constexpr int MBLK = D / 32;
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::BUF_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;         // row of this lane within the wave's 32-row block
  const int half = lane >> 5;        // which 4-token group of each 8 the lane holds
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  const int L = C - qb;
  const int M = a.G * qb;
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly
  const int nst = (t1 - t0 + 31) / 32;

  // ---- this lane's row and its Q^T operand (B of S^T = K Q^T)
  const int row = wave * 32 + col;
  const bool row_ok = row < M;
  const bool wave_active = wave * 32 < M;
  const int g = row_ok ? row / qb : 0, ci = row_ok ? row % qb : 0;
  const int h = hkv * a.G + g;
  bf16x8 qop[KSTEPS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         (((int64_t)b * a.Qmax + ci) * a.Hq + h) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint4 w = row_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const uint64_t mbits = row_ok ? load_mask_row(a.mask, b, ci, qb, a.Qmax) : 0ull;

  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  constexpr int64_t TILE_BYTES = (int64_t)kPage * D * KT::bytes;
  constexpr int ROW_BYTES = D * KT::bytes;

  // ---- stage loader: item = (token pair tp, 8-dim chunk c)
  typename CK::raw rk[IPT][2], rv[IPT][2];
  auto issue_loads = [&](int st) {
    const int sbase = t0 + st * 32;
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int tp = item / T::CHUNKS, c = item % T::CHUNKS;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = sbase + 2 * tp + e;
        if (item < T::ITEMS && t < t1) {
          const int64_t phys = table[t / kPage];
          const int64_t off = (phys * a.Hkv + hkv) * TILE_BYTES + (t % kPage) * ROW_BYTES +
                              c * 8 * KT::bytes;
          rk[it][e] = CK::load(kbase + off);
          rv[it][e] = CK::load(vbase + off);
        } else {
          rk[it][e] = {};
          rv[it][e] = {};
        }
      }
    }
  };
  auto write_lds = [&](int buf) {
    uint16_t* kl = lds + buf * T::BUF_ELEMS;
    uint16_t* vl = kl + T::K_ELEMS;
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      if (item >= T::ITEMS) continue;
      const int tp = item / T::CHUNKS, c = item % T::CHUNKS;
      const uint4 k0 = CK::to_bf16(rk[it][0]), k1 = CK::to_bf16(rk[it][1]);
      *reinterpret_cast<uint4*>(kl + (2 * tp) * T::KROW + c * 8) = k0;
      *reinterpret_cast<uint4*>(kl + (2 * tp + 1) * T::KROW + c * 8) = k1;
      // V^T: for each of the 8 dims, the (token 2tp, token 2tp+1) pair as one word
      const uint4 v0 = CK::to_bf16(rv[it][0]), v1 = CK::to_bf16(rv[it][1]);
      const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);  // dim 2w
        const uint32_t hi = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);  // dim 2w+1
        *reinterpret_cast<uint32_t*>(vl + (c * 8 + 2 * w) * T::VROW + 2 * tp) = lo;
        *reinterpret_cast<uint32_t*>(vl + (c * 8 + 2 * w + 1) * T::VROW + 2 * tp) = hi;
      }
    }
  };

  f32x16 oacc[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) oacc[mb] = {};
  float m = NEG_INF, lpart = 0.f;

  issue_loads(0);
  write_lds(0);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) issue_loads(st + 1);

    if (wave_active) {
      const uint16_t* kl = lds + buf * T::BUF_ELEMS;
      const uint16_t* vl = kl + T::K_ELEMS;
      const int sbase = t0 + st * 32;

      // S^T[32 tokens][32 rows] = K Q^T
      f32x16 sacc = {};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kl + col * T::KROW + kk * 16 + half * 8);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], sacc, 0, 0, 0);
      }

      // per-page scales (fp8): registers 0..7 hold page 0 tokens, 8..15 page 1
      float sl0 = a.scale_log2, sl1 = a.scale_log2, vs0 = 1.f, vs1 = 1.f;
      if constexpr (KT::bytes == 1) {
        const int p0 = sbase / kPage;
        const int64_t ph0 = table[p0];
        sl0 *= a.k_scale[ph0 * a.Hkv + hkv];
        vs0 = a.v_scale[ph0 * a.Hkv + hkv];
        if (sbase + 16 < t1) {
          const int64_t ph1 = table[p0 + 1];
          sl1 *= a.k_scale[ph1 * a.Hkv + hkv];
          vs1 = a.v_scale[ph1 * a.Hkv + hkv];
        }
      }

      // scale + mask, row max (this lane's 16 tokens, then the other half-wave)
      const bool plain = sbase + 32 <= min(L, t1);
      float x[16];
      float mx = NEG_INF;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = sacc[r] * (r < 8 ? sl0 : sl1);
        if (!plain) {
          const int t = sbase + 8 * (r >> 2) + 4 * half + (r & 3);
          const int sh = t - L;
          const bool cand = (unsigned)sh < 64u && ((mbits >> (sh & 63)) & 1ull);
          v = (t < t1 && (t < L || cand)) ? v : NEG_INF;
        }
        x[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx);
      const float muse = mnew == NEG_INF ? 0.f : mnew;
      const float alpha = fast_exp2(m - muse);
      m = mnew;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = fast_exp2(x[r] - muse);
        psum += x[r];
      }
      lpart = lpart * alpha + psum;
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) oacc[mb] *= alpha;

      // P^T operands (bf16), fp8: times the page's V scale
      bf16x8 pop[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float vsc = ks == 0 ? vs0 : vs1;
#pragma unroll
        for (int j = 0; j < 8; ++j) pop[ks][j] = (__bf16)(x[8 * ks + j] * vsc);
      }
      // O^T[D][32 rows] += V^T P^T
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) {
        const uint16_t* vrow = vl + (mb * 32 + col) * T::VROW + 4 * half;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 16 * ks);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 * ks + 8);
          const uint4 w = make_uint4(lo.x, lo.y, hi.x, hi.y);
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pop[ks],
                                                             oacc[mb], 0, 0, 0);
        }
      }
    }

    if (st + 1 < nst) write_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: this lane's row, dims 32mb + 8(r/4) + 4*half + (r%4)
  const float lt = lpart + shfl_xor(lpart, 32);   // the two halves of the row's 32 tokens
  if (row_ok) {
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float muse = m == NEG_INF ? 0.f : m;
  const float lse = lt > 0.f ? (muse + fast_log2(lt)) * kLn2 : NEG_INF;
  if (split_out) {
    const int64_t prow = (((int64_t)b * a.Hq + h) * a.Qmax + ci) * a.num_parts + part;
    float* op = a.part_o + prow * D;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + 8 * q4 + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) store_coherent(op + d + e, oacc[mb][4 * q4 + e] * inv);
      }
    if (half == 0) store_coherent(a.part_lse + prow, lse);
  } else {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (((int64_t)b * a.Qmax + ci) * a.Hq + h) * D;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + 8 * q4 + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(oacc[mb][4 * q4] * inv, oacc[mb][4 * q4 + 1] * inv);
        w.y = pack_bf16x2(oacc[mb][4 * q4 + 2] * inv, oacc[mb][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d) = w;
      }
    if (half == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.Hq + h) * a.Qmax + ci] = lse;
  }
  }
  if (split_out) splitk_finish<BF16, D>(a, b, hkv, C, qb);
}

// ---------------------------------------------------------------- launchers
template <typename KT, int D, int NWAVE>
static hipError_t launch_mfma_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((mfma_attn_kernel<KT, D, NWAVE>), grid, dim3(NWAVE * 64), 0, s, a);
  return hipGetLastError();
}

template <typename KT, int D>
static hipError_t launch_mfma_d(const AttnArgs& a, int nwave, dim3 grid, hipStream_t s) {
  switch (nwave) {
    case 1: return launch_mfma_t<KT, D, 1>(a, grid, s);
    case 2: return launch_mfma_t<KT, D, 2>(a, grid, s);
    case 4: return launch_mfma_t<KT, D, 4>(a, grid, s);
    case 8: return launch_mfma_t<KT, D, 8>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(const AttnArgs& a, int kv_dtype, int D, int nwave, dim3 grid, hipStream_t s) {
  if (kv_dtype == 1) {
    if (D == 64) return launch_mfma_d<BF16, 64>(a, nwave, grid, s);
    if (D == 128) return launch_mfma_d<BF16, 128>(a, nwave, grid, s);
  } else if (kv_dtype == 2) {
    if (D == 64) return launch_mfma_d<FP8, 64>(a, nwave, grid, s);
    if (D == 128) return launch_mfma_d<FP8, 128>(a, nwave, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
