// Quantized GEMMs on gfx950 matrix cores (include/pta_gemm.h): the quantized
// GEMM operators the TACO-LLM pages list beside the attention kernels
// (17173xz.com article, section "TACO-LLM如何实现降本增效?"; 618zxw.cn article,
// section "LLM量子化技術による推論コストの削減"; design talk section
// "5. 支持 Quantization（模型量化）": low-bit weights on low-precision matrix
// instructions).  W8A8 first, W4A16, W8A16 and W4A8 below.
//
// W8A8:
//   * Waves of 64 x 32 WNB (2 x WNB blocks of v_mfma_scale_f32_32x32x64_f8f6f4
//     with unit block scales: e4m3fn x e4m3fn, float32 accumulators), WMW of
//     them along M and two along N: 128 x 128 workgroup tiles up to 128 rows,
//     128 x 256 up to 256 (each activation tile feeds twice the columns), and
//     256 x 256 with eight waves above (a third fewer bytes staged per product;
//     the staging, not the matrix cores, bounds these kernels), there with
//     128-byte k-steps when K is a multiple of 128 (gemm_w8a8_k128_kernel).  A lane supplies 32
//     consecutive k-bytes of its row of A and of its column of W^T (k = 32 h +
//     0..31 of the 64-step, h = lane / 32); any consistent assignment of k to
//     (lane half, byte) gives the same sums, and this one makes each operand two
//     16-byte LDS reads.
//   * k-steps of 64 bytes staged in LDS (A tile 8 or 16 KiB + W tile 8 or 16
//     KiB), four or three stages, moved by buffer_load_dwordx4 ... lds with the whole
//     offset in the range-checked vector offset, so rows past M or N read as
//     zero and ragged edges need no other handling.  16-byte units of a row are
//     swizzled by the row's bits 2..3, so the 16 rows one pass of an operand
//     read touches hit 16 distinct bank groups.
//   * Workgroups are numbered so that the M tiles of one N tile run one after
//     the other on the same XCD: its weight tile reaches that XCD's L2 from HBM
//     once for all of them.
//   * Epilogue: y = acc * a_scale[m] * w_scale[n] in float32, rounded to bf16.
#include "../../include/pta_gemm.h"
#include "pta_device.h"

#include <type_traits>

using namespace pta;

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BK = 64, NT = 256;

// Tile geometry for WNB 32-column blocks per wave and WMW waves along M (each
// 64 rows), two waves along N:
//   WMW 2, WNB 2: 128 x 128 workgroup tiles, 4 waves, four stages
//   WMW 2, WNB 4: 128 x 256, 4 waves, three stages (two workgroups per CU)
//   WMW 4, WNB 4: 256 x 256, 8 waves, four stages (one workgroup per CU): a third
//                 fewer bytes staged per product than 128 x 256
template <int WNB, int WMW = 2>
struct GemmGeom {
  static constexpr int BM = 64 * WMW;
  static constexpr int BN = 64 * WNB;                     // two waves side by side along N
  static constexpr int NWAVES = 2 * WMW, NT = 64 * NWAVES;
  static constexpr int NBUF = WNB == 2 || WMW == 4 ? 4 : 3;
  static constexpr int A_TILE = BM * BK;                  // 8 or 16 KiB
  static constexpr int W_TILE = BN * BK;
  static constexpr int W_REG = NBUF * A_TILE;             // W region after the A region
  static constexpr int CHUNKS_A = A_TILE / 1024, CHUNKS_W = W_TILE / 1024;
  static constexpr int LOADS = (CHUNKS_A + CHUNKS_W) / NWAVES;     // copies per wave per stage
  static constexpr int LDS_BYTES = W_REG + NBUF * W_TILE;
  static_assert(CHUNKS_A % NWAVES == 0 && CHUNKS_W % NWAVES == 0, "whole copy rounds per operand");
  // the read offsets' per-stage parts are immediates (W_REG rides in the address register)
  static_assert((NBUF - 1) * W_TILE + (WNB - 1) * 32 * BK < 65536 && (NBUF - 1) * A_TILE + 32 * BK < 65536,
                "stage offsets must be 16-bit immediates");
  static_assert(LDS_BYTES <= (WMW == 2 ? 81920 : 163840), "workgroups per compute unit");
};

__device__ __forceinline__ i32x4 gemm_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = (int32_t)(uint32_t)p;
  r[1] = (int32_t)(uint32_t)(p >> 32);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

// One 1 KiB chunk (16 rows x 64 bytes) of a tile into LDS at m0val (the s_nop
// covers the wait state an M0 write needs before an LDS-DMA load).
// The whole byte offset goes in the vector offset, which the buffer range
// check covers (the scalar offset is outside it): rows of a ragged tile past M
// or N read zero instead of memory past the operand.
__device__ __forceinline__ void gemm_copy(uint32_t m0val, const i32x4& rsrc, uint32_t off, uint32_t voff) {
  const uint32_t v = voff + off;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0val), "v"(v), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int L, int K>
__device__ __forceinline__ void gemm_wait_stages(int k) {   // at most k later stages of L copies in flight
  if constexpr (K == 0) {
    gemm_wait_vm<0>();
  } else {
    if (k >= K) gemm_wait_vm<K * L>();
    else gemm_wait_stages<L, K - 1>(k);
  }
}

template <int I, int N, typename F>
__device__ __forceinline__ void gemm_static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    gemm_static_for<I + 1, N>(f);
  }
}

template <int WNB, int WMW, bool TILED = false>
__global__ __launch_bounds__(128 * WMW) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w8a8_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* w, const float* w_scale, uint16_t* y, int M, int N,
    int K, int tm, int tn) {
  using Gm = GemmGeom<WNB, WMW>;
  constexpr int BM = Gm::BM, BN = Gm::BN, NBUF = Gm::NBUF, A_TILE = Gm::A_TILE, W_TILE = Gm::W_TILE,
                W_REG = Gm::W_REG, NWAVES = Gm::NWAVES;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WMW, wn = wave / WMW;
  // XCD-grouped order: workgroup b runs on XCD b % 8; there, slots take the tm
  // M tiles of one N tile in a row
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / tm) * 8 + xcd, mt = slot % tm;
  if (nt >= tn) return;
  const int m0 = mt * BM, n0 = nt * BN;

  const i32x4 ars = gemm_rsrc(a, (uint32_t)((uint64_t)M * (uint64_t)K));
  // TILED: weights rearranged by taco_gemm_w8a16_pack, whose 8 KiB block per
  // (128-column tile, 64-k stage) is this kernel's LDS image of those columns
  const i32x4 wrs = gemm_rsrc(w, TILED ? (uint32_t)((uint64_t)((N + 127) / 128) * 128u * (uint64_t)K)
                                       : (uint32_t)((uint64_t)N * (uint64_t)K));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];
  // copy lanes: row l / 4 of a chunk, physical unit l % 4 holding logical unit
  // (l % 4) ^ ((row >> 2) & 3), with row >> 2 & 3 = (l / 16) & 3 for every chunk
  const uint32_t voff = (uint32_t)((lane >> 2) * K + ((((lane & 3) ^ ((lane >> 4) & 3))) << 4));
  const uint32_t voffT = (uint32_t)(16 * lane);
  const int nk = K / BK;
  auto copy_stage = [&](int s, int buf) {
    const uint32_t kb = (uint32_t)(s * BK);
#pragma unroll
    for (int i = 0; i < Gm::LOADS; ++i) {
      const int c = wave + NWAVES * i;             // chunk c of the stage: A chunks, then W chunks
      if (i < Gm::CHUNKS_A / NWAVES)               // (whole rounds of A chunks: known per i)
        gemm_copy(lds0 + (uint32_t)(buf * A_TILE + c * 1024), ars, (uint32_t)(m0 + 16 * c) * (uint32_t)K + kb, voff);
      else if (TILED) {                            // chunk cw: block of columns n0 + 128 (cw / 8) on
        const int cw = c - Gm::CHUNKS_A;
        gemm_copy(lds0 + (uint32_t)(W_REG + buf * W_TILE + cw * 1024), wrs,
                  ((uint32_t)(n0 / 128 + (cw >> 3)) * (uint32_t)nk + (uint32_t)s) * 8192u + 1024u * (uint32_t)(cw & 7),
                  voffT);
      } else
        gemm_copy(lds0 + (uint32_t)(W_REG + buf * W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  (uint32_t)(n0 + 16 * (c - Gm::CHUNKS_A)) * (uint32_t)K + kb, voff);
    }
  };
  // operand read offsets (bytes) inside a tile: row 32 blk + l % 32 of the
  // wave's 64 rows, units 2 h and 2 h + 1 (swizzled)
  const int r32 = lane & 31, h = lane >> 5;
  uint32_t aoff[2], woff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t u = (uint32_t)(((2 * h + e) ^ ((r32 >> 2) & 3)) << 4);
    aoff[e] = (uint32_t)((64 * wm + r32) * BK) + u;
    woff[e] = (uint32_t)(W_REG + (32 * WNB * wn + r32) * BK) + u;
  }

  f32x16 acc[2][WNB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = {};

  const int pro = min(NBUF - 1, nk);
  for (int s = 0; s < pro; ++s) copy_stage(s, s);

  auto step = [&](auto bc, int s) {
    constexpr int BUF = decltype(bc)::value;
    gemm_wait_stages<Gm::LOADS, NBUF - 2>(min(NBUF - 2, nk - 1 - s));
    __syncthreads();                          // stage s in LDS; stage s - 1 consumed by every wave
    if (s + NBUF - 1 < nk) copy_stage(s + NBUF - 1, (BUF + NBUF - 1) % NBUF);
    i32x8 ao[2], wo[WNB];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(lds + aoff[0] + BUF * A_TILE + i * 32 * BK);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(lds + aoff[1] + BUF * A_TILE + i * 32 * BK);
      ao[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(lds + woff[0] + BUF * W_TILE + j * 32 * BK);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(lds + woff[1] + BUF * W_TILE + j * 32 * BK);
      wo[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[i], wo[j], acc[i][j], 0, 0, 0, 0x7f, 0, 0x7f);
  };
  for (int s = 0; s < nk; s += NBUF) {
    bool more = true;
    gemm_static_for<0, NBUF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (!more) return;
      if (s + i >= nk) {
        more = false;
        return;
      }
      step(std::integral_constant<int, i>{}, s + i);
    });
  }

  // epilogue: lane owns column n0 + 32 WNB wn + 32 j + l % 32 and rows 8 q + 4 h + r
#pragma unroll
  for (int j = 0; j < WNB; ++j) {
    const int n = n0 + 32 * WNB * wn + 32 * j + r32;
    if (n >= N) continue;
    const float sw = w_scale[n];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16(acc[i][j][e] * a_scale[m] * sw);
      }
  }
}


// 256 x 256 tiles with 128-byte k-steps (K a multiple of 128): each copy moves
// 8 rows x 128 bytes, whole 128-byte lines, where a 64-byte k-step moves 16
// half lines per copy and the copy path then carries about half the bytes per
// clock.  Eight waves of 64 x 128 as gemm_w8a8_kernel<4, 4>, two stages (the
// next one in flight), two 64-byte halves per stage.  LDS rows are 128 bytes:
// the 16-byte unit u of tile row r sits in slot u ^ ((r >> 1) & 7), so the 16
// rows of one read pass land in 16 distinct bank groups.
template <int N_>
struct GemmK128 {
  static constexpr int BM = 256, BN = 256, BKS = 128, NWAVES = 8, NT = 512, NBUF = 2;
  static constexpr int A_TILE = BM * BKS, W_TILE = BN * BKS;       // 32 KiB each
  static constexpr int W_REG = NBUF * A_TILE;
  static constexpr int CHUNKS_A = A_TILE / 1024, CHUNKS_W = W_TILE / 1024;
  static constexpr int LOADS = (CHUNKS_A + CHUNKS_W) / NWAVES;
  static constexpr int LDS_BYTES = W_REG + NBUF * W_TILE;          // 128 KiB: one workgroup per CU
  static_assert(CHUNKS_A % NWAVES == 0 && CHUNKS_W % NWAVES == 0, "whole copy rounds per operand");
  static_assert((NBUF - 1) * W_TILE + 3 * 32 * BKS < 65536, "stage offsets must be 16-bit immediates");
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w8a8_k128_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* w, const float* w_scale, uint16_t* y, int M, int N,
    int K, int tm, int tn) {
  using Gm = GemmK128<0>;
  constexpr int BM = Gm::BM, BN = Gm::BN, BKS = Gm::BKS, A_TILE = Gm::A_TILE, W_TILE = Gm::W_TILE,
                W_REG = Gm::W_REG, NWAVES = Gm::NWAVES, WNB = 4;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / tm) * 8 + xcd, mt = slot % tm;
  if (nt >= tn) return;
  const int m0 = mt * BM, n0 = nt * BN;

  const i32x4 ars = gemm_rsrc(a, (uint32_t)((uint64_t)M * (uint64_t)K));
  const i32x4 wrs = gemm_rsrc(w, (uint32_t)((uint64_t)N * (uint64_t)K));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];
  // copy lanes: chunk row l / 8 (tile row 8 c + l / 8), slot l % 8 holding logical
  // unit (l % 8) ^ ((row >> 1) & 7) = (l % 8) ^ (4 (c & 1) + l / 16); a wave's
  // chunks c = wave + 8 i all have the parity of the wave
  const uint32_t voff =
      (uint32_t)((lane >> 3) * K + (((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) << 4));
  const int nk = K / BKS;
  auto copy_stage = [&](int s, int buf) {
    const uint32_t kb = (uint32_t)(s * BKS);
#pragma unroll
    for (int i = 0; i < Gm::LOADS; ++i) {
      const int c = wave + NWAVES * i;
      if (i < Gm::CHUNKS_A / NWAVES)
        gemm_copy(lds0 + (uint32_t)(buf * A_TILE + c * 1024), ars, (uint32_t)(m0 + 8 * c) * (uint32_t)K + kb, voff);
      else
        gemm_copy(lds0 + (uint32_t)(W_REG + buf * W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  (uint32_t)(n0 + 8 * (c - Gm::CHUNKS_A)) * (uint32_t)K + kb, voff);
    }
  };
  // operand reads: row 32 blk + l % 32 of the wave's rows, logical units 4 q + 2 h + e
  // of half q of the stage
  const int r32 = lane & 31, h = lane >> 5, sw = (r32 >> 1) & 7;
  uint32_t aoff[2][2], woff[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t u = (uint32_t)(((4 * q + 2 * h + e) ^ sw) << 4);
      aoff[q][e] = (uint32_t)((64 * wm + r32) * BKS) + u;
      woff[q][e] = (uint32_t)(W_REG + (32 * WNB * wn + r32) * BKS) + u;
    }

  f32x16 acc[2][WNB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = {};

  copy_stage(0, 0);
  auto step = [&](auto bc, int s) {
    constexpr int BUF = decltype(bc)::value;
    gemm_wait_vm<0>();
    __syncthreads();                          // stage s in LDS; stage s - 1 consumed by every wave
    if (s + 1 < nk) copy_stage(s + 1, BUF ^ 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      i32x8 ao[2], wo[WNB];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(lds + aoff[q][0] + BUF * A_TILE + i * 32 * BKS);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(lds + aoff[q][1] + BUF * A_TILE + i * 32 * BKS);
        ao[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < WNB; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(lds + woff[q][0] + BUF * W_TILE + j * 32 * BKS);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(lds + woff[q][1] + BUF * W_TILE + j * 32 * BKS);
        wo[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[i], wo[j], acc[i][j], 0, 0, 0, 0x7f, 0, 0x7f);
    }
  };
  for (int s = 0; s < nk; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nk) step(std::integral_constant<int, 1>{}, s + 1);
  }

#pragma unroll
  for (int j = 0; j < WNB; ++j) {
    const int n = n0 + 32 * WNB * wn + 32 * j + r32;
    if (n >= N) continue;
    const float sw_n = w_scale[n];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16(acc[i][j][e] * a_scale[m] * sw_n);
      }
  }
}


// ------------------------------------------------------------------ W4A16
// bf16 activations x group-scaled signed int4 weights on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation):
//   * Workgroup tile 32 WM (M) x 128 (N), BK = 64 k per stage; each of the four
//     waves owns 32 columns and all 32 WM rows (WM 32-row blocks), so every
//     weight fragment it converts feeds WM products.
//   * k assignment: in a stage, lane half h of k-step ks covers the k-octet
//     4 h + ks of both operands (any consistent assignment gives the same
//     sums).  A lane's packed weights for the whole stage are then one 16-byte
//     LDS read (octets 4 h .. 4 h + 3 of its column), and its activations one
//     16-byte read per k-step and row block.
//   * Conversion is exact: each nibble is sign-extended (v_bfe_i32), converted
//     to float32 and packed to bf16 (integers -8..7 are exact in bf16), so the
//     only roundings are the matrix cores' float32 sums and the final bf16.
//   * Group scales apply in float32: each group's products accumulate apart
//     (the first product of a group starts from zero) and acc += s[n][g] * acc_g
//     at the group's end.  The scales of a group's 128 columns arrive by
//     LDS-DMA (buffer_load_dword ... lds, a strided gather) with the group's
//     first stage, into one of four slots (group & 3).
//   * Staging as the W8A8 kernel: buffer-resource LDS-DMA with the whole offset
//     in the range-checked vector offset (rows past M or N read zero), NBUF
//     stages, XCD-grouped tile order.  With weights rearranged by
//     taco_gemm_w4a16_pack (TILED) a stage's weight tile is one contiguous
//     4 KiB block, copied as is.  Swizzles: the 16-byte unit u of
//     activation row r sits at u ^ ((r >> 1) & 7) (rows are 128 bytes), the
//     unit u of weight row r at u ^ ((r >> 3) & 1) (rows are 32 bytes): the 16
//     lanes of one read pass touch 16 distinct bank groups.
template <int WM>
struct W4Geom {
  static constexpr int BM = 32 * WM, BN = 128, BK = 64;
  static constexpr int NBUF = WM == 4 ? 3 : 4;
  static constexpr int A_TILE = BM * BK * 2;               // bf16
  static constexpr int W_TILE = BN * BK / 2;               // packed int4 (4 KiB)
  static constexpr int W_REG = NBUF * A_TILE;
  static constexpr int S_REG = W_REG + NBUF * W_TILE;      // 4 scale slots of 128 floats
  static constexpr int CHUNKS_A = A_TILE / 1024, CHUNKS_W = W_TILE / 1024;
  static constexpr int LOADS = (CHUNKS_A + CHUNKS_W) / 4;  // copies per wave per stage
  static constexpr int LDS_BYTES = S_REG + 4 * 512;
  static_assert((CHUNKS_A + CHUNKS_W) % 4 == 0, "whole copies per wave");
  static_assert(LDS_BYTES <= 81920, "two workgroups per compute unit");
};

__device__ __forceinline__ void gemm_copy_dword(uint32_t m0val, const i32x4& rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0val), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Signed nibbles 0..7 of w (nibble i = bits 4 i .. 4 i + 3) as bf16, element i.
__device__ __forceinline__ bf16x8 int4x8_to_bf16(uint32_t w) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lo = (int)(w << (28 - 8 * j)) >> 28, hi = (int)(w << (24 - 8 * j)) >> 28;
    r[j] = pack_bf16x2((float)lo, (float)hi);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// Weight tiles in load order (the rearranged layout of taco_gemm_w4a16_pack):
// the 4 KiB block of 128-column tile nt and 64-k stage s sits at byte
// (nt * (K / 64) + s) * 4096 and is the LDS image of that stage's weight tile:
// byte 32 r + 16 p holds the 16 bytes of column 128 nt + r at k-bytes
// 32 s + 16 (p ^ ((r >> 3) & 1)) (zero past N).  A stage's weights then arrive
// as four contiguous 1 KiB copies, whole 128-byte lines, where the row-major
// layout moves 32 bytes of each of 32 rows per copy.
__global__ __launch_bounds__(256) void w4a16_pack_kernel(const uint8_t* w, uint8_t* wt, int N, int K,
                                                        int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one 16-byte unit of the tiled buffer
  if (u >= units) return;
  const int nk = K / 64;
  const int64_t blk = u >> 8;                                   // 256 units per 4 KiB block
  const int within = (int)(u & 255), r = within >> 1, p = within & 1;
  const int nt = (int)(blk / nk), st = (int)(blk % nk);
  const int n = nt * 128 + r;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (n < N)
    v = *reinterpret_cast<const uint4*>(w + (int64_t)n * (K / 2) + 32 * st + 16 * (p ^ ((r >> 3) & 1)));
  *reinterpret_cast<uint4*>(wt + u * 16) = v;
}

template <int WM, bool TILED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a16_kernel(
    const uint16_t* a, const uint8_t* w, const float* w_scale, uint16_t* y, int M, int N, int K, int G, int tm,
    int tn) {
  using Gm = W4Geom<WM>;
  constexpr int BM = Gm::BM, BN = Gm::BN, NBUF = Gm::NBUF;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / tm) * 8 + xcd, mt = slot % tm;
  if (nt >= tn) return;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KG = K / G;                                     // groups per row

  const i32x4 ars = gemm_rsrc(a, (uint32_t)((uint64_t)M * (uint64_t)K * 2u));
  const i32x4 wrs = gemm_rsrc(w, TILED ? (uint32_t)((uint64_t)tn * 128u * (uint64_t)K / 2u)
                                       : (uint32_t)((uint64_t)N * (uint64_t)K / 2u));
  const i32x4 srs = gemm_rsrc(w_scale, (uint32_t)((uint64_t)N * (uint64_t)KG * 4u));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];

  // copy lanes.  Activation chunk c (8 rows of 128 bytes): lane l fills row
  // 8 c + l / 8, physical unit l % 8, holding logical unit (l % 8) ^ ((row >> 1) & 7),
  // where (row >> 1) & 7 = (4 (c & 1) + l / 16) & 7.  Weight chunk (32 rows of
  // 32 bytes): lane l fills row l / 2, physical unit l % 2, holding logical unit
  // (l % 2) ^ ((l / 16) & 1).
  uint32_t voffA[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    voffA[par] = (uint32_t)((lane >> 3) * 2 * K + 16 * ((lane & 7) ^ ((4 * par + (lane >> 4)) & 7)));
  const uint32_t voffW =
      TILED ? (uint32_t)(16 * lane) : (uint32_t)((lane >> 1) * (K / 2) + 16 * ((lane & 1) ^ ((lane >> 4) & 1)));
  const int nk = K / Gm::BK, GS = G / Gm::BK;              // stages, stages per group
  auto copy_stage = [&](int s, int buf) {
    const uint32_t kb = (uint32_t)(s * Gm::BK);
#pragma unroll
    for (int i = 0; i < Gm::LOADS; ++i) {
      const int c = wave + 4 * i;
      if (c < Gm::CHUNKS_A)
        gemm_copy(lds0 + (uint32_t)(buf * Gm::A_TILE + c * 1024), ars,
                  (uint32_t)(m0 + 8 * c) * (uint32_t)(2 * K) + 2u * kb, voffA[c & 1]);
      else if (TILED)
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  ((uint32_t)nt * (uint32_t)nk + (uint32_t)s) * 4096u + 1024u * (uint32_t)(c - Gm::CHUNKS_A), voffW);
      else
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  (uint32_t)(n0 + 32 * (c - Gm::CHUNKS_A)) * (uint32_t)(K / 2) + kb / 2u, voffW);
    }
    if (wave == 0 && s % GS == 0) {
      const int g = s / GS;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        gemm_copy_dword(lds0 + (uint32_t)(Gm::S_REG + (g & 3) * 512 + 256 * j), srs,
                        ((uint32_t)(n0 + 64 * j + lane) * (uint32_t)KG + (uint32_t)g) * 4u);
    }
  };

  // operand read offsets: activation row 32 mb + l % 32, logical unit 4 h + ks;
  // weight row 32 wave + l % 32, logical unit h
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t arow = (uint32_t)(r32 * 128);
  const int asw = (r32 >> 1) & 7;                            // same for every row block (32 mb is even)
  const int wr = 32 * wave + r32;
  const uint32_t woff = (uint32_t)(Gm::W_REG + wr * 32 + 16 * (h ^ ((wr >> 3) & 1)));

  f32x16 acc[WM], accg[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) acc[i] = {};

  const int pro = min(NBUF - 1, nk);
  for (int s = 0; s < pro; ++s) copy_stage(s, s);

  auto step = [&](auto bc, int s) {
    constexpr int BUF = decltype(bc)::value;
    gemm_wait_stages<Gm::LOADS, NBUF - 2>(min(NBUF - 2, nk - 1 - s));
    __syncthreads();                          // stage s in LDS; stage s - 1 consumed by every wave
    if (s + NBUF - 1 < nk) copy_stage(s + NBUF - 1, (BUF + NBUF - 1) % NBUF);
    const bool first = s % GS == 0;
    const uint4 wq = *reinterpret_cast<const uint4*>(lds + woff + BUF * Gm::W_TILE);
    const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = int4x8_to_bf16(wd[ks]);
      const uint32_t au = (uint32_t)(16 * ((4 * h + ks) ^ asw));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(lds + BUF * Gm::A_TILE + mb * 32 * 128 + arow + au);
        if (ks == 0 && first) accg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, f32x16{}, 0, 0, 0);
        else accg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, accg[mb], 0, 0, 0);
      }
    }
    if (s % GS == GS - 1) {                   // the group's last stage: acc += s[n][g] * acc_g
      const float sc = *reinterpret_cast<const float*>(lds + Gm::S_REG + ((s / GS) & 3) * 512 + 4 * wr);
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = fmaf(sc, accg[mb][e], acc[mb][e]);
    }
  };
  for (int s = 0; s < nk; s += NBUF) {
    bool more = true;
    gemm_static_for<0, NBUF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (!more) return;
      if (s + i >= nk) {
        more = false;
        return;
      }
      step(std::integral_constant<int, i>{}, s + i);
    });
  }

  // epilogue: lane owns column n0 + 32 wave + l % 32 and rows 8 q + 4 h + r of each block
  const int n = n0 + wr;
  if (n < N) {
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16(acc[mb][e]);
      }
  }
}


// ------------------------------------------------------------------ W8A16
// bf16 activations x fp8 e4m3fn weights with one scale per output channel, on
// the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, float32 accumulation):
//   * Tiles, waves, k assignment, staging and tile order as the W4A16 kernel:
//     32 WM x 128 workgroup tiles, 64 k per stage, each wave 32 columns and all
//     32 WM rows; lane half h of k-step ks covers k-octet 4 h + ks, so a lane's
//     weights for a stage are the 32 bytes at k-bytes 32 h .. 32 h + 31 of its
//     column (two 16-byte LDS reads).
//   * Weights are decoded exactly (every finite e4m3fn value is a bf16 value;
//     v_cvt_scalef32_pk_bf16_fp8 with unit scale), so the only roundings are
//     the float32 sums and the final bf16; the channel scale multiplies the
//     float32 sum in the epilogue.
//   * A weight row of a stage is 64 bytes (four 16-byte units); unit u of row r
//     sits at u ^ ((r >> 2) & 3), so the 16 rows of one read pass touch 16
//     distinct bank groups.  Activation rows are swizzled as in W4A16.
template <int WM>
struct W8Geom {
  static constexpr int BM = 32 * WM, BN = 128, BK = 64;
  static constexpr int NBUF = WM == 4 ? 3 : 4;
  static constexpr int A_TILE = BM * BK * 2;               // bf16
  static constexpr int W_TILE = BN * BK;                   // fp8 codes (8 KiB)
  static constexpr int W_REG = NBUF * A_TILE;
  static constexpr int CHUNKS_A = A_TILE / 1024, CHUNKS_W = W_TILE / 1024;
  static constexpr int LOADS = (CHUNKS_A + CHUNKS_W) / 4;  // copies per wave per stage
  static constexpr int LDS_BYTES = W_REG + NBUF * W_TILE;
  static_assert((CHUNKS_A + CHUNKS_W) % 4 == 0, "whole copies per wave");
  static_assert(LDS_BYTES <= 81920, "two workgroups per compute unit");
};

// Eight e4m3fn codes (bytes of lo, then hi) as eight bf16, element i = byte i.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo),
                                               fp8x2_to_bf16x2<false>(hi), fp8x2_to_bf16x2<true>(hi)));
}

// Weight tiles of W8A16 in load order (taco_gemm_w8a16_pack): the 8 KiB block
// of 128-column tile nt and 64-k stage s sits at byte (nt * (K / 64) + s) * 8192
// and is the LDS image of that stage's weight tile: byte 64 r + 16 p holds the
// 16 bytes of column 128 nt + r at k-bytes 64 s + 16 (p ^ ((r >> 2) & 3)) (zero
// past N), so a stage arrives as eight contiguous 1 KiB copies of whole lines.
__global__ __launch_bounds__(256) void w8a16_pack_kernel(const uint8_t* w, uint8_t* wt, int N, int K, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one 16-byte unit of the tiled buffer
  if (u >= units) return;
  const int nk = K / 64;
  const int64_t blk = u >> 9;                                   // 512 units per 8 KiB block
  const int within = (int)(u & 511), r = within >> 2, p = within & 3;
  const int nt = (int)(blk / nk), st = (int)(blk % nk);
  const int n = nt * 128 + r;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (n < N) v = *reinterpret_cast<const uint4*>(w + (int64_t)n * K + 64 * st + 16 * (p ^ ((r >> 2) & 3)));
  *reinterpret_cast<uint4*>(wt + u * 16) = v;
}

template <int WM, bool TILED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w8a16_kernel(
    const uint16_t* a, const uint8_t* w, const float* w_scale, uint16_t* y, int M, int N, int K, int tm, int tn) {
  using Gm = W8Geom<WM>;
  constexpr int BM = Gm::BM, BN = Gm::BN, NBUF = Gm::NBUF;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / tm) * 8 + xcd, mt = slot % tm;
  if (nt >= tn) return;
  const int m0 = mt * BM, n0 = nt * BN;

  const i32x4 ars = gemm_rsrc(a, (uint32_t)((uint64_t)M * (uint64_t)K * 2u));
  const i32x4 wrs = gemm_rsrc(w, TILED ? (uint32_t)((uint64_t)tn * 128u * (uint64_t)K)
                                       : (uint32_t)((uint64_t)N * (uint64_t)K));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];

  // copy lanes.  Activation chunk c (8 rows of 128 bytes) as in W4A16.  Weight
  // chunk c (16 rows of 64 bytes): lane l fills row 16 c + l / 4, physical unit
  // l % 4, holding logical unit (l % 4) ^ ((row >> 2) & 3) = (l % 4) ^ ((l / 16) & 3);
  // TILED: a contiguous 1 KiB piece of the stage's rearranged 8 KiB block.
  uint32_t voffA[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    voffA[par] = (uint32_t)((lane >> 3) * 2 * K + 16 * ((lane & 7) ^ ((4 * par + (lane >> 4)) & 7)));
  const uint32_t voffW = TILED ? (uint32_t)(16 * lane) : (uint32_t)((lane >> 2) * K + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  const int nk = K / Gm::BK;
  auto copy_stage = [&](int s, int buf) {
    const uint32_t kb = (uint32_t)(s * Gm::BK);
#pragma unroll
    for (int i = 0; i < Gm::LOADS; ++i) {
      const int c = wave + 4 * i;
      if (c < Gm::CHUNKS_A)
        gemm_copy(lds0 + (uint32_t)(buf * Gm::A_TILE + c * 1024), ars,
                  (uint32_t)(m0 + 8 * c) * (uint32_t)(2 * K) + 2u * kb, voffA[c & 1]);
      else if (TILED)
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  ((uint32_t)nt * (uint32_t)nk + (uint32_t)s) * 8192u + 1024u * (uint32_t)(c - Gm::CHUNKS_A), voffW);
      else
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  (uint32_t)(n0 + 16 * (c - Gm::CHUNKS_A)) * (uint32_t)K + kb, voffW);
    }
  };

  // operand read offsets: activation row 32 mb + l % 32, logical unit 4 h + ks;
  // weight row 32 wave + l % 32, logical units 2 h and 2 h + 1
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t arow = (uint32_t)(r32 * 128);
  const int asw = (r32 >> 1) & 7;
  const int wr = 32 * wave + r32;
  const uint32_t woff0 = (uint32_t)(Gm::W_REG + wr * 64 + 16 * ((2 * h) ^ ((wr >> 2) & 3)));
  const uint32_t woff1 = (uint32_t)(Gm::W_REG + wr * 64 + 16 * ((2 * h + 1) ^ ((wr >> 2) & 3)));

  f32x16 acc[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) acc[i] = {};

  const int pro = min(NBUF - 1, nk);
  for (int s = 0; s < pro; ++s) copy_stage(s, s);

  auto step = [&](auto bc, int s) {
    constexpr int BUF = decltype(bc)::value;
    gemm_wait_stages<Gm::LOADS, NBUF - 2>(min(NBUF - 2, nk - 1 - s));
    __syncthreads();                          // stage s in LDS; stage s - 1 consumed by every wave
    if (s + NBUF - 1 < nk) copy_stage(s + NBUF - 1, (BUF + NBUF - 1) % NBUF);
    const uint4 w0 = *reinterpret_cast<const uint4*>(lds + woff0 + BUF * Gm::W_TILE);
    const uint4 w1 = *reinterpret_cast<const uint4*>(lds + woff1 + BUF * Gm::W_TILE);
    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = fp8x8_to_bf16(wd[2 * ks], wd[2 * ks + 1]);
      const uint32_t au = (uint32_t)(16 * ((4 * h + ks) ^ asw));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(lds + BUF * Gm::A_TILE + mb * 32 * 128 + arow + au);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[mb], 0, 0, 0);
      }
    }
  };
  for (int s = 0; s < nk; s += NBUF) {
    bool more = true;
    gemm_static_for<0, NBUF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (!more) return;
      if (s + i >= nk) {
        more = false;
        return;
      }
      step(std::integral_constant<int, i>{}, s + i);
    });
  }

  // epilogue: lane owns column n0 + 32 wave + l % 32 and rows 8 q + 4 h + r of each block
  const int n = n0 + wr;
  if (n < N) {
    const float sc = w_scale[n];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16(sc * acc[mb][e]);
      }
  }
}

// ------------------------------------------------------------------ W4A8
// int8 activations (per-row scales) x group-scaled int4 weights on the integer
// matrix cores (v_mfma_i32_32x32x32_i8, int32 accumulation):
//   * Tiles 32 WM x 128, 64 k per stage, each of four waves 32 columns and all
//     32 WM rows, weights in the W4A16 layout and staging (packed rows of 32
//     bytes per stage, group scales by LDS-DMA into four slots), activation
//     rows of 64 bytes per stage with unit u of row r at u ^ ((r >> 2) & 3).
//   * k assignment: in k-step ks (32 k) lane half h covers the 16 k at
//     16 (2 h + ks) of the stage, so a lane's weights for the stage are one
//     16-byte LDS read and its activations one 16-byte read per k-step and row
//     block.
//   * Widening is exact and cheap: a nibble moved to the top of its byte is the
//     int8 value 16 q, so (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 hold the
//     even and odd k of eight weights and one byte permute each restores k
//     order; the factor 16 comes out with the activation scale (a power of
//     two, exact).
//   * A group's products sum exactly in int32 (|16 q a| <= 2^14 per product);
//     at the group's end acc += s[n][g] * float(acc_g) in float32, and the
//     epilogue multiplies by a_scale[m] / 16 and rounds to bf16.
template <int WM>
struct W48Geom {
  static constexpr int BM = 32 * WM, BN = 128, BK = 64;
  static constexpr int NBUF = 4;
  static constexpr int A_TILE = BM * BK;                   // int8
  static constexpr int W_TILE = BN * BK / 2;               // packed int4 (4 KiB)
  static constexpr int W_REG = NBUF * A_TILE;
  static constexpr int S_REG = W_REG + NBUF * W_TILE;      // 4 scale slots of 128 floats
  static constexpr int CHUNKS_A = A_TILE / 1024, CHUNKS_W = W_TILE / 1024;
  static constexpr int LOADS = (CHUNKS_A + CHUNKS_W) / 4;  // copies per wave per stage
  static constexpr int LDS_BYTES = S_REG + 4 * 512;
  static_assert((CHUNKS_A + CHUNKS_W) % 4 == 0, "whole copies per wave");
  static_assert(LDS_BYTES <= 81920, "two workgroups per compute unit");
};

// Eight int4 weights (low nibble = even k) as eight int8 values 16 q, in k
// order, as two words.
__device__ __forceinline__ void int4x8_to_i8x16q(uint32_t w, uint32_t& k0to3, uint32_t& k4to7) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;   // k 0 2 4 6 / k 1 3 5 7
  k0to3 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  k4to7 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

template <int WM, bool TILED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a8_kernel(
    const uint8_t* a, const float* a_scale, const uint8_t* w, const float* w_scale, uint16_t* y, int M, int N, int K,
    int G, int tm, int tn) {
  using Gm = W48Geom<WM>;
  constexpr int BM = Gm::BM, BN = Gm::BN, NBUF = Gm::NBUF;
  __shared__ __attribute__((aligned(1024))) char lds[Gm::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / tm) * 8 + xcd, mt = slot % tm;
  if (nt >= tn) return;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KG = K / G;                                     // groups per row

  const i32x4 ars = gemm_rsrc(a, (uint32_t)((uint64_t)M * (uint64_t)K));
  const i32x4 wrs = gemm_rsrc(w, TILED ? (uint32_t)((uint64_t)tn * 128u * (uint64_t)K / 2u)
                                       : (uint32_t)((uint64_t)N * (uint64_t)K / 2u));
  const i32x4 srs = gemm_rsrc(w_scale, (uint32_t)((uint64_t)N * (uint64_t)KG * 4u));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&lds[0];

  // copy lanes.  Activation chunk c (16 rows of 64 bytes): lane l fills row
  // 16 c + l / 4, physical unit l % 4, holding logical unit (l % 4) ^ ((l / 16) & 3).
  // Weight chunk (32 rows of 32 bytes) as in W4A16, or (TILED) a contiguous
  // 1 KiB piece of the stage's rearranged 4 KiB block.
  const uint32_t voffA = (uint32_t)((lane >> 2) * K + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  const uint32_t voffW =
      TILED ? (uint32_t)(16 * lane) : (uint32_t)((lane >> 1) * (K / 2) + 16 * ((lane & 1) ^ ((lane >> 4) & 1)));
  const int nk = K / Gm::BK, GS = G / Gm::BK;              // stages, stages per group
  auto copy_stage = [&](int s, int buf) {
    const uint32_t kb = (uint32_t)(s * Gm::BK);
#pragma unroll
    for (int i = 0; i < Gm::LOADS; ++i) {
      const int c = wave + 4 * i;
      if (c < Gm::CHUNKS_A)
        gemm_copy(lds0 + (uint32_t)(buf * Gm::A_TILE + c * 1024), ars, (uint32_t)(m0 + 16 * c) * (uint32_t)K + kb,
                  voffA);
      else if (TILED)
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  ((uint32_t)nt * (uint32_t)nk + (uint32_t)s) * 4096u + 1024u * (uint32_t)(c - Gm::CHUNKS_A), voffW);
      else
        gemm_copy(lds0 + (uint32_t)(Gm::W_REG + buf * Gm::W_TILE + (c - Gm::CHUNKS_A) * 1024), wrs,
                  (uint32_t)(n0 + 32 * (c - Gm::CHUNKS_A)) * (uint32_t)(K / 2) + kb / 2u, voffW);
    }
    if (wave == 0 && s % GS == 0) {
      const int g = s / GS;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        gemm_copy_dword(lds0 + (uint32_t)(Gm::S_REG + (g & 3) * 512 + 256 * j), srs,
                        ((uint32_t)(n0 + 64 * j + lane) * (uint32_t)KG + (uint32_t)g) * 4u);
    }
  };

  // operand read offsets: activation row 32 mb + l % 32, logical unit 2 h + ks;
  // weight row 32 wave + l % 32, logical unit h
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t arow = (uint32_t)(r32 * 64);
  const int asw = (r32 >> 2) & 3;                            // same for every row block
  const int wr = 32 * wave + r32;
  const uint32_t woff = (uint32_t)(Gm::W_REG + wr * 32 + 16 * (h ^ ((wr >> 3) & 1)));

  f32x16 acc[WM];
  i32x16 accg[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) acc[i] = {};

  const int pro = min(NBUF - 1, nk);
  for (int s = 0; s < pro; ++s) copy_stage(s, s);

  auto step = [&](auto bc, int s) {
    constexpr int BUF = decltype(bc)::value;
    gemm_wait_stages<Gm::LOADS, NBUF - 2>(min(NBUF - 2, nk - 1 - s));
    __syncthreads();                          // stage s in LDS; stage s - 1 consumed by every wave
    if (s + NBUF - 1 < nk) copy_stage(s + NBUF - 1, (BUF + NBUF - 1) % NBUF);
    const bool first = s % GS == 0;
    const uint4 wq = *reinterpret_cast<const uint4*>(lds + woff + BUF * Gm::W_TILE);
    const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 b;
      uint32_t b0, b1, b2, b3;
      int4x8_to_i8x16q(wd[2 * ks], b0, b1);
      int4x8_to_i8x16q(wd[2 * ks + 1], b2, b3);
      b = i32x4{(int32_t)b0, (int32_t)b1, (int32_t)b2, (int32_t)b3};
      const uint32_t au = (uint32_t)(16 * ((2 * h + ks) ^ asw));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const i32x4 av = *reinterpret_cast<const i32x4*>(lds + BUF * Gm::A_TILE + mb * 32 * 64 + arow + au);
        if (ks == 0 && first) accg[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b, i32x16{}, 0, 0, 0);
        else accg[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b, accg[mb], 0, 0, 0);
      }
    }
    if (s % GS == GS - 1) {                   // the group's last stage: acc += s[n][g] * acc_g
      const float sc = *reinterpret_cast<const float*>(lds + Gm::S_REG + ((s / GS) & 3) * 512 + 4 * wr);
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = fmaf(sc, (float)accg[mb][e], acc[mb][e]);
    }
  };
  for (int s = 0; s < nk; s += NBUF) {
    bool more = true;
    gemm_static_for<0, NBUF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (!more) return;
      if (s + i >= nk) {
        more = false;
        return;
      }
      step(std::integral_constant<int, i>{}, s + i);
    });
  }

  // epilogue: lane owns column n0 + 32 wave + l % 32 and rows 8 q + 4 h + r of each block
  const int n = n0 + wr;
  if (n < N) {
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16(acc[mb][e] * (a_scale[m] * 0.0625f));
      }
  }
}
}  // namespace

extern "C" {

}  // extern "C"

namespace {

pta_status w8a8_call(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y, int32_t M,
                     int32_t N, int32_t K, void* stream, bool tiled) {
  if (!a || !a_scale || !w || !w_scale || !y) return PTA_ERR_NULL_PTR;
  if (M < 1 || N < 1 || K < BK || K % BK != 0) return PTA_ERR_BAD_DIMS;
  // every tile row (those past M or N included) must have a 32-bit buffer offset
  const uint64_t mpad = (uint64_t)((M + 255) / 256) * 256, npad = (uint64_t)((N + 255) / 256) * 256;
  if (mpad * (uint64_t)K >= ((uint64_t)1 << 32) || npad * (uint64_t)K >= ((uint64_t)1 << 32)) return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w)) % 16 != 0) return PTA_ERR_BAD_DIMS;
  // wide column tiles once the M tiles alone would not fill the device; 256-row
  // tiles past 256 rows
  const int kind = M > 256 ? 2 : (M > 128 ? 1 : 0);
  const int TBM = kind == 2 ? GemmGeom<4, 4>::BM : BM;
  const int BN = kind == 0 ? GemmGeom<2>::BN : GemmGeom<4>::BN;
  const int tm = (M + TBM - 1) / TBM, tn = (N + BN - 1) / BN;
  const int64_t blocks = (int64_t)8 * tm * ((tn + 7) / 8);
  if (blocks > 0x7fffffff) return PTA_ERR_BAD_DIMS;
  auto launch = [&](auto kern, int nt) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(nt), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t*>(a), a_scale, reinterpret_cast<const uint8_t*>(w), w_scale,
                       reinterpret_cast<uint16_t*>(y), M, N, K, tm, tn);
  };
  if (tiled) {   // the 64-k kernels only: the 128-k kernel stages 128-byte rows
    if (kind == 2) launch(gemm_w8a8_kernel<4, 4, true>, GemmGeom<4, 4>::NT);
    else if (kind == 1) launch(gemm_w8a8_kernel<4, 2, true>, GemmGeom<4, 2>::NT);
    else launch(gemm_w8a8_kernel<2, 2, true>, GemmGeom<2, 2>::NT);
  } else if (kind == 2 && K % 128 == 0) {
    launch(gemm_w8a8_k128_kernel, GemmK128<0>::NT);
  } else if (kind == 2) {
    launch(gemm_w8a8_kernel<4, 4>, GemmGeom<4, 4>::NT);
  } else if (kind == 1) {
    launch(gemm_w8a8_kernel<4, 2>, GemmGeom<4, 2>::NT);
  } else {
    launch(gemm_w8a8_kernel<2, 2>, GemmGeom<2, 2>::NT);
  }
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

}  // namespace

extern "C" {

pta_status taco_gemm_w8a8(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y,
                          int32_t M, int32_t N, int32_t K, void* stream) {
  return w8a8_call(a, a_scale, w, w_scale, y, M, N, K, stream, false);
}

pta_status taco_gemm_w8a8_tiled(const void* a, const float* a_scale, const void* w_tiled, const float* w_scale,
                                void* y, int32_t M, int32_t N, int32_t K, void* stream) {
  return w8a8_call(a, a_scale, w_tiled, w_scale, y, M, N, K, stream, true);
}

}  // extern "C"

namespace {

pta_status w4a16_call(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N,
                      int32_t K, int32_t group, void* stream, bool tiled) {
  if (!a || !w || !w_scale || !y) return PTA_ERR_NULL_PTR;
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || group < 64 || group % 64 != 0 || K % group != 0)
    return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w)) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w_scale) % 4 != 0)
    return PTA_ERR_BAD_DIMS;
  // row blocks of 64 rows up to 64 rows, else of 128
  const bool tall = M > 64;
  const int BM = tall ? W4Geom<4>::BM : W4Geom<2>::BM, BN = 128;
  // every tile row (those past M or N included) must have a 32-bit buffer offset
  const uint64_t mpad = (uint64_t)((M + BM - 1) / BM) * BM, npad = (uint64_t)((N + BN - 1) / BN) * BN;
  if (mpad * (uint64_t)K * 2u >= ((uint64_t)1 << 32) || npad * (uint64_t)K / 2u >= ((uint64_t)1 << 32) ||
      npad * (uint64_t)(K / group) * 4u >= ((uint64_t)1 << 32))
    return PTA_ERR_BAD_DIMS;
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int64_t blocks = (int64_t)8 * tm * ((tn + 7) / 8);
  if (blocks > 0x7fffffff) return PTA_ERR_BAD_DIMS;
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint16_t*>(a), reinterpret_cast<const uint8_t*>(w), w_scale,
                       reinterpret_cast<uint16_t*>(y), M, N, K, group, tm, tn);
  };
  if (tall) {
    if (tiled) launch(gemm_w4a16_kernel<4, true>);
    else launch(gemm_w4a16_kernel<4, false>);
  } else {
    if (tiled) launch(gemm_w4a16_kernel<2, true>);
    else launch(gemm_w4a16_kernel<2, false>);
  }
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

}  // namespace

extern "C" {

pta_status taco_gemm_w4a16(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N,
                           int32_t K, int32_t group, void* stream) {
  return w4a16_call(a, w, w_scale, y, M, N, K, group, stream, false);
}

size_t taco_gemm_w4a16_tiled_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 64 || K % 64 != 0) return 0;
  const uint64_t bytes = (uint64_t)((N + 127) / 128) * 128u * (uint64_t)K / 2u;
  return bytes < ((uint64_t)1 << 32) ? (size_t)bytes : 0;
}

pta_status taco_gemm_w4a16_pack(const void* w, void* w_tiled, int32_t N, int32_t K, void* stream) {
  if (!w || !w_tiled) return PTA_ERR_NULL_PTR;
  const size_t bytes = taco_gemm_w4a16_tiled_bytes(N, K);
  if (bytes == 0) return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(w_tiled)) % 16 != 0) return PTA_ERR_BAD_DIMS;
  const int64_t units = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(w4a16_pack_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint8_t*>(w), reinterpret_cast<uint8_t*>(w_tiled), N, K, units);
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

pta_status taco_gemm_w4a16_tiled(const void* a, const void* w_tiled, const float* w_scale, void* y, int32_t M,
                                 int32_t N, int32_t K, int32_t group, void* stream) {
  return w4a16_call(a, w_tiled, w_scale, y, M, N, K, group, stream, true);
}

}  // extern "C"

namespace {

pta_status w4a8_call(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y, int32_t M,
                     int32_t N, int32_t K, int32_t group, void* stream, bool tiled) {
  if (!a || !a_scale || !w || !w_scale || !y) return PTA_ERR_NULL_PTR;
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || group < 64 || group % 64 != 0 || K % group != 0)
    return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w)) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(a_scale) | reinterpret_cast<uintptr_t>(w_scale)) % 4 != 0)
    return PTA_ERR_BAD_DIMS;
  // row blocks of 64 rows up to 64 rows, else of 128
  const bool tall = M > 64;
  const int BM = tall ? W48Geom<4>::BM : W48Geom<2>::BM, BN = 128;
  // every tile row (those past M or N included) must have a 32-bit buffer offset
  const uint64_t mpad = (uint64_t)((M + BM - 1) / BM) * BM, npad = (uint64_t)((N + BN - 1) / BN) * BN;
  if (mpad * (uint64_t)K >= ((uint64_t)1 << 32) || npad * (uint64_t)K / 2u >= ((uint64_t)1 << 32) ||
      npad * (uint64_t)(K / group) * 4u >= ((uint64_t)1 << 32))
    return PTA_ERR_BAD_DIMS;
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int64_t blocks = (int64_t)8 * tm * ((tn + 7) / 8);
  if (blocks > 0x7fffffff) return PTA_ERR_BAD_DIMS;
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t*>(a), a_scale, reinterpret_cast<const uint8_t*>(w), w_scale,
                       reinterpret_cast<uint16_t*>(y), M, N, K, group, tm, tn);
  };
  if (tall) {
    if (tiled) launch(gemm_w4a8_kernel<4, true>);
    else launch(gemm_w4a8_kernel<4, false>);
  } else {
    if (tiled) launch(gemm_w4a8_kernel<2, true>);
    else launch(gemm_w4a8_kernel<2, false>);
  }
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

}  // namespace

extern "C" {

pta_status taco_gemm_w4a8(const void* a, const float* a_scale, const void* w, const float* w_scale, void* y,
                          int32_t M, int32_t N, int32_t K, int32_t group, void* stream) {
  return w4a8_call(a, a_scale, w, w_scale, y, M, N, K, group, stream, false);
}

pta_status taco_gemm_w4a8_tiled(const void* a, const float* a_scale, const void* w_tiled, const float* w_scale,
                                void* y, int32_t M, int32_t N, int32_t K, int32_t group, void* stream) {
  return w4a8_call(a, a_scale, w_tiled, w_scale, y, M, N, K, group, stream, true);
}

}  // extern "C"

namespace {

pta_status w8a16_call(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N, int32_t K,
                      void* stream, bool tiled) {
  if (!a || !w || !w_scale || !y) return PTA_ERR_NULL_PTR;
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0) return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w)) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w_scale) % 4 != 0)
    return PTA_ERR_BAD_DIMS;
  // row blocks of 64 rows up to 64 rows, else of 128
  const bool tall = M > 64;
  const int BM = tall ? W8Geom<4>::BM : W8Geom<2>::BM, BN = 128;
  // every tile row (those past M or N included) must have a 32-bit buffer offset
  const uint64_t mpad = (uint64_t)((M + BM - 1) / BM) * BM, npad = (uint64_t)((N + BN - 1) / BN) * BN;
  if (mpad * (uint64_t)K * 2u >= ((uint64_t)1 << 32) || npad * (uint64_t)K >= ((uint64_t)1 << 32))
    return PTA_ERR_BAD_DIMS;
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int64_t blocks = (int64_t)8 * tm * ((tn + 7) / 8);
  if (blocks > 0x7fffffff) return PTA_ERR_BAD_DIMS;
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint16_t*>(a), reinterpret_cast<const uint8_t*>(w), w_scale,
                       reinterpret_cast<uint16_t*>(y), M, N, K, tm, tn);
  };
  if (tall) {
    if (tiled) launch(gemm_w8a16_kernel<4, true>);
    else launch(gemm_w8a16_kernel<4, false>);
  } else {
    if (tiled) launch(gemm_w8a16_kernel<2, true>);
    else launch(gemm_w8a16_kernel<2, false>);
  }
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

}  // namespace

extern "C" {

pta_status taco_gemm_w8a16(const void* a, const void* w, const float* w_scale, void* y, int32_t M, int32_t N,
                           int32_t K, void* stream) {
  return w8a16_call(a, w, w_scale, y, M, N, K, stream, false);
}

size_t taco_gemm_w8a16_tiled_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 64 || K % 64 != 0) return 0;
  const uint64_t bytes = (uint64_t)((N + 127) / 128) * 128u * (uint64_t)K;
  return bytes < ((uint64_t)1 << 32) ? (size_t)bytes : 0;
}

pta_status taco_gemm_w8a16_pack(const void* w, void* w_tiled, int32_t N, int32_t K, void* stream) {
  if (!w || !w_tiled) return PTA_ERR_NULL_PTR;
  const size_t bytes = taco_gemm_w8a16_tiled_bytes(N, K);
  if (bytes == 0) return PTA_ERR_BAD_DIMS;
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(w_tiled)) % 16 != 0) return PTA_ERR_BAD_DIMS;
  const int64_t units = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(w8a16_pack_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint8_t*>(w), reinterpret_cast<uint8_t*>(w_tiled), N, K, units);
  return hipGetLastError() == hipSuccess ? PTA_OK : PTA_ERR_HIP;
}

pta_status taco_gemm_w8a16_tiled(const void* a, const void* w_tiled, const float* w_scale, void* y, int32_t M,
                                 int32_t N, int32_t K, void* stream) {
  return w8a16_call(a, w_tiled, w_scale, y, M, N, K, stream, true);
}

}  // extern "C"
