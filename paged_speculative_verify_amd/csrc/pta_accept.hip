// Acceptance of verified candidates and commit of their K/V rows.
//
// After the verify pass the target model's prediction at each candidate
// position decides which candidates are kept, so that one step generates
// several tokens (TACO-LLM design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践":
// the target model judges the candidate tokens; "2. 加速上限分析" counts the
// tokens hit per step).  Greedy rule: a root is accepted when its token equals
// the prediction after the committed prefix, any other node when its parent
// is accepted and its token equals the parent's prediction; the deepest
// accepted node (lowest index among equals) and its ancestors form the path
// that is committed.  The path's K/V rows move to consecutive positions right
// after the committed prefix (blocks are filled as tokens are kept, section
// "4. 支持 Paged Attention"), and the context length becomes prefix + path.
//
// One workgroup per sequence.  Wave 0 finds the path: lane i holds node i, its
// parent is the highest set bit of the mask row below i, and pointer jumping
// (six rounds for up to 64 nodes) gives every node the AND of its ancestors'
// matches and its depth; the best node is a wave maximum and the path is read
// back along the parents with uniform register reads.  Then all waves move
// the rows (a destination row can be the source of a later entry, never of an
// earlier one, so moves in path order are safe).
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

// 16 fp8 codes from pages of scale s_src re-encoded for a page of scale s_dst.
__device__ __forceinline__ uint4 fp8_reencode(uint4 w, float s_src, float s_dst) {
  uint32_t in[4] = {w.x, w.y, w.z, w.w}, out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t r = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = fp8x2_to_f32<false>((in[k] >> (8 * e)) & 0xffu)[0] * s_src;
      r |= f32_to_e4m3fn_sat(__fdiv_rn(x, s_dst)) << (8 * e);
    }
    out[k] = r;
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

template <typename KT>
__global__ __launch_bounds__(256) void accept_commit_kernel(AcceptArgs p) {
  __shared__ int s_path[64];
  __shared__ int s_n;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int C = p.ctx[b], q = p.qlen[b], L = C - q;
  const int tprev = p.target_prev[b];
  if (tid < 64) {
    const int i = tid;
    const bool live = i < q;
    const uint64_t bits = live ? load_mask_row(p.mask, b, i, q, p.Qmax) : 0ull;
    const uint64_t below = bits & ((1ull << i) - 1ull);           // i < 64
    const int par = below ? 63 - __builtin_clzll(below) : -1;
    const int tok = live ? p.cand[(int64_t)b * p.Qmax + i] : 0;
    const int want = (live && par >= 0) ? p.target[(int64_t)b * p.Qmax + par] : tprev;
    int acc = live && tok == want;
    int depth = 1, jp = par;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const int src = jp < 0 ? i : jp;
      const int acc_j = __shfl(acc, src, 64);
      const int dep_j = __shfl(depth, src, 64);
      const int jp_j = __shfl(jp, src, 64);
      if (jp >= 0) {
        acc = acc & acc_j;
        depth += dep_j;
        jp = jp_j;
      }
    }
    int key = acc ? depth * 128 + (127 - i) : -1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
    const int n = key < 0 ? 0 : key >> 7;
    const int best = key < 0 ? -1 : 127 - (key & 127);
    if (i == 0) {
      int cur = best;
      for (int k = n - 1; k >= 0; --k) {
        s_path[k] = cur;
        cur = __builtin_amdgcn_readlane(par, cur);
      }
      s_n = n;
      p.n_acc[b] = n;
      p.bonus[b] = n > 0 ? p.target[(int64_t)b * p.Qmax + best] : tprev;
      p.new_ctx[b] = L + n;
    }
  }
  __syncthreads();
  const int n = s_n;
  if (tid < p.Qmax) p.path[(int64_t)b * p.Qmax + tid] = tid < n ? s_path[tid] : -1;
  // Moves: thread t owns the same 16-byte pieces (K or V, head, piece) of every
  // row, so its own program order keeps the in-order rule; within a group of
  // eight path entries it reads all sources before writing (a destination is
  // never the source of an earlier entry, and later entries' sources lie past
  // every destination written so far), which keeps eight loads in flight.
  const int32_t* table = p.tables + (int64_t)b * p.MBS;
  const int pieces = p.D * KT::bytes / 16;
  const int per = p.Hkv * pieces;
  for (int k0 = 0; k0 < n; k0 += 8) {
    const int kn = min(8, n - k0);
    for (int it = tid; it < 2 * per; it += 256) {
      const int which = it / per, h = (it % per) / pieces, j = it % pieces;
      char* cache = reinterpret_cast<char*>(which ? p.v : p.k);
      uint4 buf[8];
      int64_t src_page[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < kn && s_path[k0 + e] != k0 + e) {
          const int src = L + s_path[k0 + e];
          src_page[e] = table[src / kPage];
          const int64_t off = ((src_page[e] * p.Hkv + h) * kPage + src % kPage) * (int64_t)(p.D * KT::bytes);
          buf[e] = *reinterpret_cast<const uint4*>(cache + off + 16 * j);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < kn && s_path[k0 + e] != k0 + e) {
          const int dst = L + k0 + e;
          const int64_t dpage = table[dst / kPage];
          const int64_t off = ((dpage * p.Hkv + h) * kPage + dst % kPage) * (int64_t)(p.D * KT::bytes);
          uint4 w = buf[e];
          if constexpr (KT::bytes == 1) {
            const float* scl = which ? p.v_scale : p.k_scale;
            const float s_src = scl[src_page[e] * p.Hkv + h], s_dst = scl[dpage * p.Hkv + h];
            if (s_src != s_dst) w = fp8_reencode(w, s_src, s_dst);
          }
          *reinterpret_cast<uint4*>(cache + off + 16 * j) = w;
        }
      }
    }
  }
}

hipError_t launch_accept(const AcceptArgs& p, int kv_dtype, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  if (kv_dtype == 0) hipLaunchKernelGGL(accept_commit_kernel<F32>, dim3((unsigned)p.B), dim3(256), 0, s, p);
  else if (kv_dtype == 1) hipLaunchKernelGGL(accept_commit_kernel<BF16>, dim3((unsigned)p.B), dim3(256), 0, s, p);
  else if (kv_dtype == 2) hipLaunchKernelGGL(accept_commit_kernel<FP8>, dim3((unsigned)p.B), dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pta
