// Internal device-side definitions for libpta (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pta {

// ---------------------------------------------------------------- element tags
struct F32 { using storage = float; static constexpr int bytes = 4; };
struct BF16 { using storage = uint16_t; static constexpr int bytes = 2; };
struct FP8 { using storage = uint8_t; static constexpr int bytes = 1; };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything one attention launch needs.  Passed by value.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* qlen;
  const uint8_t* mask;     // may be null when Qmax == 1
  void* out;
  float* lse;              // may be null
  float* part_o;           // split-K partial outputs [B][Hq][Qmax][P][D], or null (unsplit)
  float* part_lse;         // split-K partial LSE     [B][Hq][Qmax][P]
  int32_t* counters;       // split-K arrival counters [B][Hkv] (zero between calls)
  int32_t total_waves;     // balanced mode: waves in the persistent grid
  float scale_log2;        // softmax scale * log2(e)
  int32_t B, Hq, Hkv, G, Qmax, MBS;
  int32_t part_tokens;     // partition length in tokens (split) or 0
  int32_t num_parts;       // partitions per sequence (grid.x)
  int32_t seq_order;       // whole-context stream grid: 0 grid order, 1 long/short pairs, 2 longest first
  // shared-prefix entry: leader (first sequence) of each sequence's group of consecutive
  // sequences sharing partition 0 (null otherwise), and the largest group size
  const int32_t* prefix_leader;
  int32_t max_group;
  // fused KV append (whole-context stream grid): the candidates' new K/V rows
  // [B][Qmax][Hkv][D] (cache dtype, or bf16/f32 when new_f32 says so for fp8
  // caches), written into their paged slots before the unit reads its pages;
  // null otherwise
  const void* k_new;
  const void* v_new;
  int32_t new_f32;
  int64_t num_blocks;
  // no page is named by two sequences' block tables: page tiles that one
  // workgroup alone reads take the nontemporal (streaming) load hint
  int32_t stream_pages;
  // balanced grids: pages of padding in front of every unit on the page line
  // (the slices then even out pages plus a fixed cost per unit piece); 0 = none
  int32_t slice_pad;
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// two e4m3fn codes (bytes sel*2, sel*2+1 of w) -> two floats, exact (hardware convert)
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// two e4m3fn codes -> two bf16 (packed), exact: every finite e4m3fn value is a bf16 value
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round a float32 to an OCP e4m3fn code: nearest, ties to even, saturating at
// +-448; NaN -> 0x7F.  Written from the format's definition (1 sign bit,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormal step 2^-9).
__device__ __forceinline__ uint32_t f32_to_e4m3fn_sat(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t s = (bits >> 24) & 0x80u;
  uint32_t mag = bits & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7fu;                 // NaN
  float a = __uint_as_float(mag);
  if (a >= 448.0f) return s | 0x7eu;                    // saturate (also +-inf)
  if (a < 0.015625f) {                                  // below 2^-6: multiples of 2^-9
    int m = __float2int_rn(a * 512.0f);                 // exact scaling, ties to even
    return s | (uint32_t)m;                             // m == 8 is code 0x08 = 2^-6
  }
  int e = (int)(mag >> 23) - 127;                       // -6..8
  uint32_t mant = mag & 0x7fffffu;
  uint32_t keep = mant >> 20, rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1u;
  uint32_t code = ((uint32_t)(e + 7) << 3) + keep;      // a carry out of keep bumps the exponent
  if (code > 0x7eu) code = 0x7eu;
  return s | code;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <int LO, int HI>   // reduce max over lanes differing in bits [log2 LO, log2 HI)
__device__ __forceinline__ float wave_max_range(float v) {
#pragma unroll
  for (int o = LO; o < HI; o <<= 1) v = fmaxf(v, shfl_xor(v, o));
  return v;
}
template <int LO, int HI>
__device__ __forceinline__ float wave_sum_range(float v) {
#pragma unroll
  for (int o = LO; o < HI; o <<= 1) v += shfl_xor(v, o);
  return v;
}

// Candidate-mask row i of sequence b as a 64-bit set (bit j = mask[b][i][j], j < qb).
__device__ __forceinline__ uint64_t load_mask_row(const uint8_t* mask, int b, int i, int qb,
                                                  int Qmax) {
  if (mask == nullptr) return 1ull;          // Qmax == 1: the candidate sees itself
  const uint8_t* row = mask + ((int64_t)b * Qmax + i) * Qmax;
  uint64_t bits = 0;
  if (((reinterpret_cast<uintptr_t>(mask) | (uintptr_t)Qmax) & 3) == 0) {
    // rows 4-byte aligned: one dword per 4 candidates (inside the row, since qb <= Qmax and
    // Qmax is a multiple of 4), all loads issued before the first use: one round trip
    const uint32_t* r4 = reinterpret_cast<const uint32_t*>(row);
    const int nw = (qb + 3) >> 2;
    uint32_t w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = e < nw ? r4[e] : 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      // the top bit of each nonzero byte, then those four bits gathered into bits 24..27
      const uint32_t t = (((w[e] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[e]) & 0x80808080u;
      bits |= (uint64_t)((((t >> 7) * 0x01020408u) >> 24) & 0xFu) << (4 * e);
    }
    return qb >= 64 ? bits : bits & ((1ull << qb) - 1ull);
  }
  // 16 independent byte loads per group (indices clamped into the row), so a
  // row costs one memory round trip per 16 candidates rather than one each
  for (int j0 = 0; j0 < qb; j0 += 16) {
    uint8_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = row[min(j0 + e, qb - 1)];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (j0 + e < qb && v[e] != 0) bits |= 1ull << (j0 + e);
  }
  return bits;
}

// ---------------------------------------------------------------- split-K finish
// Partials travel between work units through device-coherent single-word
// accesses (agent-scope atomic stores / loads: write-through and re-read at the
// device coherence point, so no unit needs a whole-cache write-back or
// invalidate).  A unit's partial stores complete (s_waitcnt) before its
// arrival is counted.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four consecutive words (16-byte aligned) with one device-coherent store: the
// same write-through as store_coherent, but a whole 16-byte piece per lane,
// so the memory side sees full sectors instead of one partial write per word.
// A store of more than 8 bytes reads its data registers after issue, so a
// vector ALU write to them needs a wait state first; the compiler inserts none
// after inline asm, hence the s_nop.
__device__ __forceinline__ void store_coherent4(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True when this work unit's results go to workspace partials (split-K and the
// sequence spans more than one partition); a sequence that fits in one
// partition is written straight to out/lse with no partial and no merge.
__device__ __forceinline__ bool unit_writes_partials(const AttnArgs& a, int C) {
  return a.part_o != nullptr && C > a.part_tokens;
}

// Merge np partial results of rows r0 .. M - 1 of work unit (b, hkv) by
// log-sum-exp and store the final rows (out in the q dtype, lse):
//   LSE = ln sum_p exp(LSE_p),   out = sum_p exp(LSE_p - LSE) O_p
// (the long-sequence design of the 618zxw.cn article, section
// "長シーケンス推論最適化におけるTurboAttention": the sequence is processed in
// parts that are combined).  slot(r, p) gives the partial output row (D
// floats) and its log-sum-exp word for row r, part p; parts are read in index
// order, so the result does not depend on which worker merges.  Executed by
// nthr threads; each takes IT (row, 4 dims) items at a time, with the loads of
// PB parts of all of them in flight at once and an online rescale across
// batches of parts.
template <typename QT, int D, typename SlotFn>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int b, int hkv, int qb, int M, int np,
                                           SlotFn slot, int tid, int nthr, int r0 = 0) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int Q4 = D / 4;
  constexpr int PB = 4;      // parts per batch
  constexpr int IT = 2;      // items per thread per round: IT * PB partials in flight
  const int items = (M - r0) * Q4;
  for (int base = tid; base < items; base += nthr * IT) {
    float mrun[IT], wsum[IT];
    f32x4 acc[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      mrun[k] = NEG_INF;
      wsum[k] = 0.f;
      acc[k] = {0.f, 0.f, 0.f, 0.f};
    }
    for (int p0 = 0; p0 < np; p0 += PB) {
      float lp[IT][PB];
      f32x4 op[IT][PB];
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        const int idx = base + k * nthr;
        const bool iok = idx < items;
        const int r = r0 + (iok ? idx : 0) / Q4, d = ((iok ? idx : 0) % Q4) * 4;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const bool ok = iok && p0 + j < np;
          const auto sl = slot(r, ok ? p0 + j : 0);
          lp[k][j] = ok ? load_coherent(sl.lse) : NEG_INF;
#pragma unroll
          for (int e = 0; e < 4; ++e) op[k][j][e] = ok ? load_coherent(sl.o + d + e) : 0.f;
        }
      }
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        float mx = mrun[k];
#pragma unroll
        for (int j = 0; j < PB; ++j) mx = fmaxf(mx, lp[k][j]);
        const float muse = mx == NEG_INF ? 0.f : mx;
        const float alpha = __expf(mrun[k] - muse);          // 0 while nothing has been seen
        wsum[k] *= alpha;
        acc[k] *= alpha;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const float w = __expf(lp[k][j] - muse);           // exp(-inf) = 0: no visible key there
          wsum[k] += w;
          acc[k] += w * op[k][j];
        }
        mrun[k] = mx;
      }
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int idx = base + k * nthr;
      if (idx >= items) continue;
      const int r = r0 + idx / Q4, d = (idx % Q4) * 4;
      const float muse = mrun[k] == NEG_INF ? 0.f : mrun[k];
      const float inv = wsum[k] > 0.f ? 1.f / wsum[k] : 0.f;
      const f32x4 res = acc[k] * inv;
      const int h = hkv * a.G + r / qb, i = r % qb;
      const int64_t o = (((int64_t)b * a.Qmax + i) * a.Hq + h) * D + d;
      if constexpr (QT::bytes == 4) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = res;
      } else {
        uint2 w;
        w.x = pack_bf16x2(res[0], res[1]);
        w.y = pack_bf16x2(res[2], res[3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o) = w;
      }
      if (d == 0 && a.lse != nullptr)
        a.lse[((int64_t)b * a.Hq + h) * a.Qmax + i] = wsum[k] > 0.f ? muse + __logf(wsum[k]) : NEG_INF;
    }
  }
}

// Exclusive prefix of KV pages over the sequences, into ps[0..B] (ps[B] =
// all pages), by the NT threads of a workgroup: each thread sums a contiguous
// chunk of sequences, a wave scans its threads with shuffles, and the wave
// totals (wave_tot, NT / 64 words of LDS) are added in front.  Each sequence
// counts a.slice_pad pages more than it holds (each of its units is that much
// longer on the page line).
template <int NT>
__device__ __forceinline__ void page_prefix(const AttnArgs& a, int* ps, int* wave_tot, int tid) {
  const int B = a.B;
  const int chunk = (B + NT - 1) / NT;
  const int lo = min(B, tid * chunk), hi = min(B, lo + chunk);
  int s = 0;
  for (int bb = lo; bb < hi; ++bb) s += (a.ctx[bb] + kPage - 1) / kPage + a.slice_pad;
  const int lane = tid & 63, wv = tid >> 6;
  int inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wave_tot[wv] = inc;
  __syncthreads();
  int before = 0;
  for (int j = 0; j < wv; ++j) before += wave_tot[j];
  int base = before + inc - s;
  if (tid == NT - 1) ps[B] = before + inc;
  for (int bb = lo; bb < hi; ++bb) {
    ps[bb] = base;
    base += (a.ctx[bb] + kPage - 1) / kPage + a.slice_pad;
  }
  __syncthreads();
}

struct PartSlot {
  const float* o;     // D floats
  const float* lse;   // one word
};

// Called by every thread of a split-K work unit (sequence b, KV head hkv) once
// its normalised partial output and log-sum-exp are stored with
// store_coherent.  The last unit of (b, hkv) to arrive merges the partitions
// of all its rows and resets the arrival counter to zero for the next call.
// Ordering through the memory model, with one agent-scope release per arrival
// and one acquire per unit: every wave's partial stores complete (vmcnt) and
// precede the workgroup barrier; the barrier precedes thread 0's release
// arrival at agent scope (release is cumulative over what happens before it);
// the last arriver's thread 0 follows its arrival with an agent-scope acquire
// fence, and the second barrier orders that fence before every thread's
// partial loads.  (A release and an acquire in every wave of every arrival
// write back and invalidate the L2 several times per unit: on the
// shared-prefix decode entry that measured 3.5x slower.)
template <typename QT, int D>
__device__ __forceinline__ void splitk_finish(const AttnArgs& a, int b, int hkv, int C, int qb) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's partial stores are complete
  __syncthreads();
  const int np = (C + a.part_tokens - 1) / a.part_tokens;
  int32_t* cnt = a.counters + (int64_t)b * a.Hkv + hkv;
  if (threadIdx.x == 0) {
    const bool last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  auto slot = [&](int r, int p) {
    const int h = hkv * a.G + r / qb, i = r % qb;
    const int64_t prow = (((int64_t)b * a.Hq + h) * a.Qmax + i) * a.num_parts + p;
    return PartSlot{a.part_o + prow * D, a.part_lse + prow};
  };
  merge_rows<QT, D>(a, b, hkv, qb, a.G * qb, np, slot, threadIdx.x, blockDim.x);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace pta
