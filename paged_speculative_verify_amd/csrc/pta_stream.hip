// Matrix-core paged tree attention for few rows per KV head (M = G * q_len
// <= 32: GQA decode and short candidate chains).  The verify step turns each
// sequence's decode GEMV into a small GEMM (TACO-LLM design talk
// "大模型倍速推理引擎 TACO-LLM 的设计与实践", TurboAttention bullets of
// "整体方案分为两大部分"); with so few rows the work is a pure HBM stream, and
// the kernels are written so that almost nothing but the page loads costs time:
//
//   * Every query row of a (sequence, KV head) unit -- the GQA group's q-heads
//     times the candidates -- is handled by the same wave, so each KV page
//     tile crosses HBM once per group.  Each wave keeps its own flash-style
//     softmax state (on-chip state independent of the context length,
//     "优化策略总结" item 2).
//   * No barrier while streaming.  Every page load instruction reads 1 KiB
//     contiguous (lane l: bytes 16 l + 1024 j of the page tile): loading K
//     straight into the MFMA operand layout would make each instruction touch
//     16 rows x 64 B, which measures ~20% below contiguous tiles on MI355X.
//     Pages go in pairs: the K and V tiles of two pages into per-wave LDS
//     tiles (fp8 decoded to bf16 on the way); K comes back with ds_read_b128
//     as the A operand of v_mfma_f32_16x16x32_bf16 (lane (g, m): 8 consecutive
//     dims of token m) for S^T = K Q^T, and V with two ds_read_b64_tr_b16,
//     whose 16-lane transpose yields the A operand of one 32-token
//     O^T += V^T P^T step, again v_mfma_f32_16x16x32_bf16 (the 16-token
//     bf16 instruction runs at half rate on gfx950); P^T is the pair of S^T
//     accumulators, as a bf16 hi/lo pair.
//   * The next pair's loads are issued right after the current pair is
//     written to LDS and before it is computed, so they are in flight while
//     the wave computes.
//   * Softmax rescaling is lazy: a row's reference maximum only moves when a
//     score exceeds it by more than 2^8, so the accumulator rescale (and the
//     cross-lane max) is skipped on almost every page.  The result is the same
//     exact softmax; terms are bounded by 2^8 so nothing overflows.
//   * fp8 e4m3fn pages are decoded to bf16 exactly on the way in (the pages'
//     fast dequantisation inside attention, 618zxw.cn article section
//     "LLM量子化技術による推論コストの削減"); the per-(page, KV head) scales
//     are folded into the score multiplier and into P.
//
// Two kernels share this core:
//   stream_attn_kernel      one workgroup per (unit, token partition); its
//                           waves take the page pairs round-robin and are
//                           merged in LDS (whole-context and split-K entry
//                           points).
//   stream_balanced_kernel  persistent grid; the pages of all units are laid
//                           end to end and every wave takes an equal
//                           contiguous slice, so ragged context lengths cost
//                           no load imbalance.  A slice that ends inside a
//                           unit leaves a partial in the workspace, and a
//                           second launch on the same stream
//                           (slice_merge_kernel) merges each unit's partials
//                           in slice order; no counters.
#include "pta_device.h"
#include "pta_flash.h"
#include "pta_launch.h"

namespace pta {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// 16 bytes of a page tile; nontemporal (streaming) when no other workgroup reads the
// page (a template choice: a runtime one lets the compiler merge both loads into one
// without the hint)
template <bool NT>
__device__ __forceinline__ uint4 tile_load(const char* p) {
  if constexpr (NT) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p)));
  else return *reinterpret_cast<const uint4*>(p);
}

// Page pairs j = j0, j0 + js, ... of the range [pA, pB): pair j is pages
// pA + 2j and, if it is in the range, pA + 2j + 1 (else the first page again,
// its tokens masked and its V rows zeroed).  One pair's K and V chunks are in
// registers at a time: they are written to the wave's four LDS tiles, the next
// pair's loads are issued (unconditionally, the last one repeats the final
// pair, so the compiler's load counters stay exact), and the pair is computed
// with one 32-token P.V step per output block (pair_compute).
template <typename KT, int D>
struct PairRegs {
  uint4 k[2][StreamTile<KT, D>::LOADS];
  uint4 v[2][StreamTile<KT, D>::LOADS];
  float ks[2], vs[2];
};

// prog_len > 0: the wave owns a slice of prog_len pages of which prog0 come
// before this range, and paces itself by its progress through the slice.
template <typename KT, int D, int RB, bool NT>
__device__ __forceinline__ void stream_pairs(const AttnArgs& a, const StreamRows<D, RB>& rows,
                                             StreamState<D, RB>& st, int b, int hkv, int L, int t_end,
                                             int pA, int pB, int j0, int js, char* wl, int lane,
                                             int prog0 = 0, int prog_len = 0) {
  using T = StreamTile<KT, D>;
  constexpr int64_t TILE_BYTES = (int64_t)kPage * D * KT::bytes;
  const int npair = (pB - pA + 1) / 2;
  const int n = j0 < npair ? (npair - 1 - j0) / js + 1 : 0;
  if (n <= 0) return;
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);

  PairRegs<KT, D> R;
  // Block-table entries are read one pair ahead of the tile loads that need
  // them, so no tile load waits on a table round trip.
  int32_t phn[2];
  auto read_table = [&](int idx) {
    const int p0 = pA + 2 * (j0 + idx * js);
    const int p1 = p0 + 1 < pB ? p0 + 1 : p0;           // index stays inside the range
    phn[0] = table[p0];
    phn[1] = table[p1];
  };
  auto issue = [&]() {
    const int64_t ph[2] = {__builtin_amdgcn_readfirstlane(phn[0]), __builtin_amdgcn_readfirstlane(phn[1])};
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int64_t tile = (ph[pg] * a.Hkv + hkv) * TILE_BYTES + 16 * lane;
#pragma unroll
      for (int j = 0; j < T::LOADS; ++j) R.k[pg][j] = tile_load<NT>(kbase + tile + 1024 * j);
#pragma unroll
      for (int j = 0; j < T::LOADS; ++j) R.v[pg][j] = tile_load<NT>(vbase + tile + 1024 * j);
      if constexpr (KT::bytes == 1) {
        R.ks[pg] = a.k_scale[ph[pg] * a.Hkv + hkv];
        R.vs[pg] = a.v_scale[ph[pg] * a.Hkv + hkv];
      } else {
        R.ks[pg] = 1.f;
        R.vs[pg] = 1.f;
      }
    }
  };
  char* k0l = wl;
  char* k1l = wl + T::TILE_LDS;
  char* v0l = wl + 2 * T::TILE_LDS;
  char* v1l = wl + 3 * T::TILE_LDS;
  read_table(0);
  issue();
  read_table(min(1, n - 1));
  for (int idx = 0; idx < n; ++idx) {
    const int pb0 = (pA + 2 * (j0 + idx * js)) * kPage;
    const float c0 = score_scale(a, R.ks[0]), c1 = score_scale(a, R.ks[1]);
    const float vs0 = R.vs[0], vs1 = R.vs[1];
    stage_tile<KT, D>(k0l, R.k[0], lane, false, kPage);
    stage_tile<KT, D>(k1l, R.k[1], lane, false, kPage);
    stage_tile<KT, D>(v0l, R.v[0], lane, pb0 + kPage > t_end, t_end - pb0);
    stage_tile<KT, D>(v1l, R.v[1], lane, pb0 + 2 * kPage > t_end, t_end - pb0 - kPage);
    pace(prog0 + 2 * idx, prog_len);
    issue();                          // pair idx + 1 (the last pair again at the end)
    read_table(min(idx + 2, n - 1));
    pair_compute<D, RB, false, KT::bytes == 1>(rows, st, k0l, k1l, v0l, v1l, pb0, L, t_end, c0, c1, vs0, vs1,
                                               lane);
  }
}

// ============================================================ per-unit kernel
// Sequence worked by grid index z of the whole-context entry, by context
// length (ties by index; the order is recomputed in LDS by every workgroup,
// `scratch` holds 2 B ints and is free again when this returns).
//   a.seq_order == 1, the whole grid resident at once (two workgroups per
//     compute unit): a CU's time is the sum of the two contexts it holds, so
//     indices z and z + ceil(B / 2) take the i-th longest and the i-th
//     shortest sequence; with workgroups handed out in index order the two
//     that share a CU carry a long and a short context.
//   a.seq_order == 2, a grid larger than what is resident: longest first, so
//     the short contexts fill the slots that free up at the end.
// B > 256 keeps z.
template <int NT>
__device__ __forceinline__ int ordered_sequence(const AttnArgs& a, int z, int* scratch, int tid) {
  const int B = a.B;
  if (B > 256) return z;
  int* len = scratch;
  int* order = scratch + B;
  for (int i = tid; i < B; i += NT) len[i] = a.ctx[i];
  __syncthreads();
  for (int i = tid; i < B; i += NT) {
    const int ci = len[i];
    int r = 0;
    for (int j = 0; j < B; ++j) {
      const int cj = len[j];
      r += (cj > ci) || (cj == ci && j < i);
    }
    order[r] = i;
  }
  __syncthreads();
  const int h = (B + 1) / 2;
  const int seq = order[a.seq_order == 1 && z >= h ? B - 1 - (z - h) : z];
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(seq);
}

// Rows of a shared-prefix group (sequences lead .. lead + n - 1, whose block
// tables alias the pages of partition 0): the G * q_j rows of member j follow
// those of member j - 1, row r of member j being q-head hkv * G + r / q_j,
// candidate r % q_j.  Every row sees every token of the shared prefix (it lies
// in each member's committed part), so no candidate mask bits are needed.
// bj[rb] receives the member sequence of the lane's row block rb.
template <int D, int RB>
__device__ __forceinline__ void load_group_rows(StreamRows<D, RB>& R, int (&bj)[RB], const AttnArgs& a, int lead,
                                                int n, int hkv, int g, int m) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rb * 16 + m;
    int base = 0, mem = -1, rl = 0, qj = 1;
    for (int t = 0; t < n; ++t) {
      const int qt = a.qlen[lead + t];
      if (mem < 0 && row < base + a.G * qt) {
        mem = t;
        rl = row - base;
        qj = qt;
      }
      base += a.G * qt;
    }
    R.ok[rb] = mem >= 0;
    bj[rb] = lead + (mem >= 0 ? mem : 0);
    R.h[rb] = hkv * a.G + (R.ok[rb] ? rl / qj : 0);
    R.i[rb] = R.ok[rb] ? rl % qj : 0;
    R.mbits[rb] = 0ull;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         (((int64_t)bj[rb] * a.Qmax + R.i[rb]) * a.Hq + R.h[rb]) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 w = R.ok[rb] ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
      if (a.scale_log2 < 0.f) {                // a negative scale moves into the sign of Q
        w.x ^= 0x80008000u;
        w.y ^= 0x80008000u;
        w.z ^= 0x80008000u;
        w.w ^= 0x80008000u;
      }
      R.qop[rb][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// The KV append of the verify step fused into the attention launch: the
// unit's q_b new K and V rows (candidates at logical positions L .. C - 1,
// KV head hkv) go to their paged slots, fp8 caches storing RNE-saturated codes
// of x / scale with the slot's (page, KV head) scale, and the workgroup waits
// for the stores before any page is read.  Only this workgroup reads this
// unit's (page, KV head) tiles in the launch, so nothing else can see a half
// written row.  Each thread moves whole 8-element chunks (q_b <= ROWS, so at
// most MAXC of them) and issues every load before its first store, so the
// append costs about one load and one store round trip.
template <typename KT, int D, int ROWS, int NT>
__device__ __forceinline__ void append_unit_rows(const AttnArgs& a, int b, int hkv, int L, int qb, int tid) {
  constexpr int CPR = D / 8;                                  // chunks per row
  constexpr int MAXC = (2 * ROWS * CPR + NT - 1) / NT;
  typedef uint32_t Chunk __attribute__((ext_vector_type(KT::bytes * 2)));   // 8 cache elements
  const int32_t* table = a.tables + (int64_t)b * a.MBS;
  const int n = 2 * qb * CPR;
  Chunk val[MAXC];
  int64_t dst[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int e = tid + i * NT;
    if (e >= n) continue;
    const int which = e / (qb * CPR), r = (e / CPR) % qb, c = e % CPR;
    const int t = L + r;
    const int64_t page = table[t / kPage];
    dst[i] = ((((page * a.Hkv + hkv) * kPage + t % kPage) * D + c * 8) << 1) | which;
    const int64_t src = (((int64_t)b * a.Qmax + r) * a.Hkv + hkv) * D + c * 8;
    const void* in = which ? a.v_new : a.k_new;
    if constexpr (KT::bytes == 2) {
      val[i] = *reinterpret_cast<const Chunk*>(reinterpret_cast<const uint16_t*>(in) + src);
    } else {
      float x[8];
      if (a.new_f32) {
        const float4 lo = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(in) + src);
        const float4 hi = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(in) + src + 4);
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(in) + src);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(u[k] << 16);
          x[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
      }
      const float scl = (which ? a.v_scale : a.k_scale)[page * a.Hkv + hkv];
      uint32_t code[2] = {0u, 0u};
#pragma unroll
      for (int k = 0; k < 8; ++k) code[k >> 2] |= f32_to_e4m3fn_sat(__fdiv_rn(x[k], scl)) << (8 * (k & 3));
      val[i] = Chunk{code[0], code[1]};
    }
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (tid + i * NT >= n) continue;
    void* cache = const_cast<void*>((dst[i] & 1) ? a.v : a.k);
    *reinterpret_cast<Chunk*>(reinterpret_cast<char*>(cache) + (dst[i] >> 1) * KT::bytes) = val[i];
  }
  __builtin_amdgcn_s_waitcnt(0);    // this thread's stores have completed
  __syncthreads();
}

template <typename KT, int D, int RB, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void stream_attn_kernel(AttnArgs a) {
  using T = StreamTile<KT, D>;
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int ROWS = 16 * RB;

  __shared__ __attribute__((aligned(16))) char vlds[NW][T::WAVE_LDS];
  __shared__ float red_m[NW][ROWS];
  __shared__ float red_l[NW][ROWS];
  static_assert(NW == 1 || RB * T::DB * 64 * 16 <= NW * T::WAVE_LDS, "merge buffer must fit the tiles");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4;          // 16-lane group
  const int m = lane & 15;          // lane within the group
  const int part = blockIdx.x, hkv = blockIdx.y;
  static_assert(sizeof(vlds) >= 2 * 256 * sizeof(int), "the pairing scratch must fit the tiles");
  const int b = a.part_tokens > 0 || a.seq_order == 0
                    ? (int)blockIdx.z
                    : ordered_sequence<NW * 64>(a, blockIdx.z, reinterpret_cast<int*>(&vlds[0][0]), threadIdx.x);

  const int C = a.ctx[b];
  const int qb = a.qlen[b];
  int L = C - qb;
  const int M = a.G * qb;
  int t0 = 0, t1 = C;
  if (a.part_tokens > 0) {
    t0 = part * a.part_tokens;
    t1 = min(C, t0 + a.part_tokens);
    if (t0 >= t1) return;           // partition past this sequence's context
  }
  const bool split_out = unit_writes_partials(a, C);   // else: final output written directly

  // Shared-prefix entry, partition 0: a group's leader works the shared pages
  // once for the rows of every member; the other members skip the partition.
  int grp = 0;
  int bj[RB];
  if (a.prefix_leader != nullptr && part == 0) {
    // a follower within reach of its leader (the leader counts exactly these) leaves the
    // partition to it; any other sequence works its own partition 0
    const int lead = a.prefix_leader[b];
    // (a leader that does not lead itself leaves its would-be followers to work their own
    // partition 0: a malformed leader array degrades to ordinary split-K, never to a lost row)
    if (lead >= 0 && lead < b && b - lead < a.max_group && a.prefix_leader[lead] == lead) {
      bool chain = true;                 // every sequence between the leader and b follows it too
      for (int t = lead + 1; t < b; ++t) chain = chain && a.prefix_leader[t] == lead;
      if (chain) return;
    }
    if (lead == b) {
      grp = 1;
      while (grp < a.max_group && b + grp < a.B && a.prefix_leader[b + grp] == b) ++grp;
      grp = __builtin_amdgcn_readfirstlane(grp);
    }
    if (grp == 1) grp = 0;          // a group of one: the ordinary partition
  }

  StreamRows<D, RB> rows;
  if (grp > 1) {
    load_group_rows(rows, bj, a, b, grp, hkv, g, m);
    L = t1;                         // every shared token is visible to every row
  } else {
    load_rows(rows, a, b, hkv, qb, M, g, m);
  }
  // the append's round trips overlap the row loads above
  if (a.k_new != nullptr && a.part_tokens == 0) append_unit_rows<KT, D, ROWS, NW * 64>(a, b, hkv, L, qb, threadIdx.x);
  StreamState<D, RB> st;
  st.init();

  // this wave's page pairs: wave, wave + NW, ... of the unit's range
  const int pgA = t0 / kPage;
  const int pgB = (t1 + kPage - 1) / kPage;
  // every (page, KV head) tile of a unit is read by this workgroup alone unless block
  // tables share pages (the shared-prefix entry's partition 0 is read once per group)
  if (a.stream_pages) stream_pairs<KT, D, RB, true>(a, rows, st, b, hkv, L, t1, pgA, pgB, wave, NW, vlds[wave], lane);
  else stream_pairs<KT, D, RB, false>(a, rows, st, b, hkv, L, t1, pgA, pgB, wave, NW, vlds[wave], lane);
  reduce_row_sums(st);

  // ---- merge the waves: row max, row sum, then O^T accumulated in LDS in wave order
  if constexpr (NW > 1) {
    if (g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        red_m[wave][rb * 16 + m] = st.m[rb];
        red_l[wave][rb * 16 + m] = st.l[rb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = NEG_INF;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_m[w][rb * 16 + m]);
      const float muse = mx == NEG_INF ? 0.f : mx;
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) lt += red_l[w][rb * 16 + m] * fast_exp2(red_m[w][rb * 16 + m] - muse);
      const float f = fast_exp2(st.m[rb] - muse);
#pragma unroll
      for (int db = 0; db < T::DB; ++db) st.o[rb][db] *= f;
      st.m[rb] = mx;
      st.l[rb] = lt;
    }
    f32x4* ob = reinterpret_cast<f32x4*>(&vlds[0][0]);   // page tiles are dead after the barrier
    for (int w = 0; w < NW; ++w) {
      if (wave == w) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < T::DB; ++db) {
            f32x4& slot = ob[(rb * T::DB + db) * 64 + lane];
            if (w > 0) st.o[rb][db] += slot;
            if (w < NW - 1) slot = st.o[rb][db];
          }
      }
      if (w < NW - 1) __syncthreads();
    }
  }

  // ---- epilogue (last wave holds the merged rows)
  if (grp > 1) {
    if (wave == NW - 1) {
      auto addr = [&](int rb, float*& o, float*& l) {
        const int64_t prow = (((int64_t)bj[rb] * a.Hq + rows.h[rb]) * a.Qmax + rows.i[rb]) * a.num_parts;
        o = a.part_o + prow * D;
        l = a.part_lse + prow;
      };
      store_partial_rows(rows, st, g, addr);
    }
    for (int t = 0; t < grp; ++t) {
      const int bt = b + t;
      splitk_finish<BF16, D>(a, bt, hkv, a.ctx[bt], a.qlen[bt]);
    }
    return;
  }
  if (wave == NW - 1) {
    if (split_out) {
      auto addr = [&](int rb, float*& o, float*& l) {
        const int64_t prow =
            (((int64_t)b * a.Hq + rows.h[rb]) * a.Qmax + rows.i[rb]) * a.num_parts + part;
        o = a.part_o + prow * D;
        l = a.part_lse + prow;
      };
      store_partial_rows(rows, st, g, addr);
    } else {
      store_final_rows(a, rows, st, b, g);
    }
  }
  if (split_out) splitk_finish<BF16, D>(a, b, hkv, C, qb);
}

// ============================================================ balanced kernel
// Every wave owns one contiguous slice of a global page line and streams it
// on its own.  Unit u = b * Hkv + h (sequence-major) owns positions
// [S_u, S_u + P_b) with P_b = ceil(C_b / 16) and S_u = Hkv * PS_b + h * P_b
// (PS = exclusive prefix of P over sequences).  With W positions in all and N
// working waves, wave w owns [w W / N, (w + 1) W / N); the one owning position
// x is ((x + 1) N - 1) / W.  N <= W, so every working wave owns a position and
// the slices touching u are exactly waves wave_of(S_u) .. wave_of(S_u + P_b - 1).
// The partial of (wave w, unit u) lives in slot w + u, unique because waves
// and units are both ordered along the line; slice_merge_kernel, launched
// next, merges them (merging inside this launch would leave the last waves
// reading partials at the end while the rest of the device idles).  Slices
// hold at least kMinSlicePages pages.  Neighbouring waves stream neighbouring page ranges of
// one unit, so the waves in flight at any moment read pages spread over the
// pool rather than the adjacent head tiles of one block, which HBM serves
// better (measured on MI355X: about 5.6 TB/s against 4.9 for whole units).
// Dynamic LDS: PS[0..B] (int32).
template <typename KT, int D, int RB, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void stream_balanced_kernel(AttnArgs a) {
  using T = StreamTile<KT, D>;
  __shared__ __attribute__((aligned(16))) char vlds[NW][T::WAVE_LDS];
  __shared__ int wave_tot[NW];
  extern __shared__ int ps[];       // [B + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int B = a.B;

  // ---- exclusive prefix of pages per sequence (every workgroup computes it)
  page_prefix<NW * 64>(a, ps, wave_tot, tid);
  const int64_t W = (int64_t)a.Hkv * __builtin_amdgcn_readfirstlane(ps[B]);
  const int64_t N = min((int64_t)gridDim.x * NW, max((int64_t)1, W / kMinSlicePages));
  const int64_t w = (int64_t)blockIdx.x * NW + wave;
  if (w >= N) return;               // no workgroup barrier follows
  const int Mmax = a.G * a.Qmax;

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
    const int L = C - qb;
    const int M = a.G * qb;
    StreamRows<D, RB> rows;
    load_rows(rows, a, b, hkv, qb, M, g, m);
    StreamState<D, RB> st;
    st.init();
    if (a.stream_pages)
      stream_pairs<KT, D, RB, true>(a, rows, st, b, hkv, L, min(C, k1 * kPage), k0, k1, 0, 1, vlds[wave], lane,
                                    (int)(x - x0), (int)(xe - x0));
    else
      stream_pairs<KT, D, RB, false>(a, rows, st, b, hkv, L, min(C, k1 * kPage), k0, k1, 0, 1, vlds[wave], lane,
                                     (int)(x - x0), (int)(xe - x0));
    reduce_row_sums(st);

    if (k0 == 0 && k1 == Pb) {
      store_final_rows(a, rows, st, b, g);        // the whole unit in this slice
    } else {
      auto addr = [&](int rb, float*& o, float*& l) {
        const int64_t r = (w + u) * Mmax + rb * 16 + m;
        o = a.part_o + r * D;
        l = a.part_lse + r;
      };
      store_partial_rows(rows, st, g, addr);        // merged by the second launch
    }
    x += k1 - k0;
  }
}

// ---------------------------------------------------------------- launchers
// Workgroups of stream_attn_kernel<KT, D, RB, NW> resident on the current
// device at once (compute units times occupancy).  Looked up once per device
// and kept in a per-device table (every thread that fills an entry writes the
// same value, so concurrent first calls are harmless); 0 when unknown.
constexpr int kMaxDevices = 64;
template <typename KT, int D, int RB, int NW>
static int resident_workgroups() {
  static int cache[kMaxDevices];          // 0 = not looked up yet
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, stream_attn_kernel<KT, D, RB, NW>, NW * 64, 0) !=
          hipSuccess)
    return 0;
  const int n = cus * per;
  if (dev >= 0 && dev < kMaxDevices) __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  return n;
}

template <typename KT, int D, int RB, int NW>
static hipError_t launch_stream_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  AttnArgs b = a;
  if (a.part_tokens == 0) {
    const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
    const int res = resident_workgroups<KT, D, RB, NW>();
    b.seq_order = res <= 0 ? 0 : wgs <= res ? 1 : 2;
  }
  hipLaunchKernelGGL((stream_attn_kernel<KT, D, RB, NW>), grid, dim3(NW * 64), 0, s, b);
  return hipGetLastError();
}

template <typename KT, int D>
static hipError_t launch_stream_d(const AttnArgs& a, int rb, int nw, dim3 grid, hipStream_t s) {
  if (rb == 1 && nw == 4) return launch_stream_t<KT, D, 1, 4>(a, grid, s);
  if (rb == 2 && nw == 4) return launch_stream_t<KT, D, 2, 4>(a, grid, s);
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

// Balanced kernel.  With a == nullptr: report the persistent grid size
// (workgroups) for the current device, from its compute-unit count and the
// kernel's occupancy.  Otherwise launch *nwg workgroups.
template <typename KT, int D, int RB, int NW>
static hipError_t balanced_t(const AttnArgs* a, int B, int* nwg, hipStream_t s) {
  const size_t dyn = (size_t)(B + 1) * sizeof(int);
  if (a == nullptr) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, stream_balanced_kernel<KT, D, RB, NW>, NW * 64, dyn);
    if (e != hipSuccess) return e;
    *nwg = cus * (per > 0 ? per : 1);
    return hipSuccess;
  }
  hipLaunchKernelGGL((stream_balanced_kernel<KT, D, RB, NW>), dim3((unsigned)*nwg), dim3(NW * 64), dyn, s, *a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_slice_merge(*a, D, *nwg * NW, s);
}

template <typename KT, int D>
static hipError_t balanced_d(const AttnArgs* a, int rb, int nw, int B, int* nwg, hipStream_t s) {
  if (nw != 4) return hipErrorInvalidValue;
  if (rb == 1) return balanced_t<KT, D, 1, 4>(a, B, nwg, s);
  if (rb == 2) return balanced_t<KT, D, 2, 4>(a, B, nwg, s);
  return hipErrorInvalidValue;
}

hipError_t stream_balanced(const AttnArgs* a, int kv_dtype, int D, int rb, int nw, int B, int* nwg,
                           hipStream_t s) {
  if (kv_dtype == 1) {
    if (D == 64) return balanced_d<BF16, 64>(a, rb, nw, B, nwg, s);
    if (D == 128) return balanced_d<BF16, 128>(a, rb, nw, B, nwg, s);
  } else if (kv_dtype == 2) {
    if (D == 64) return balanced_d<FP8, 64>(a, rb, nw, B, nwg, s);
    if (D == 128) return balanced_d<FP8, 128>(a, rb, nw, B, nwg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pta
