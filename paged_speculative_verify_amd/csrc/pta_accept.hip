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
// the rows, one path entry at a time (a destination row can be the source of
// a later entry, never of an earlier one, so in-order moves are safe).
#include "pta_device.h"
#include "pta_launch.h"

namespace pta {

template <typename KT>
__device__ __forceinline__ void move_row(const AcceptArgs& p, void* cache, const float* scale, int64_t ps, int os,
                                         int64_t pd, int od, int tid) {
  const int n = p.Hkv * p.D;
  for (int e = tid; e < n; e += 256) {
    const int h = e / p.D, d = e % p.D;
    const int64_t si = ((ps * p.Hkv + h) * kPage + os) * p.D + d;
    const int64_t di = ((pd * p.Hkv + h) * kPage + od) * p.D + d;
    if constexpr (KT::bytes == 4) {
      reinterpret_cast<uint32_t*>(cache)[di] = reinterpret_cast<const uint32_t*>(cache)[si];
    } else if constexpr (KT::bytes == 2) {
      reinterpret_cast<uint16_t*>(cache)[di] = reinterpret_cast<const uint16_t*>(cache)[si];
    } else {
      uint8_t* c8 = reinterpret_cast<uint8_t*>(cache);
      const uint32_t code = c8[si];
      const float s_src = scale[ps * p.Hkv + h], s_dst = scale[pd * p.Hkv + h];
      if (s_src == s_dst) {
        c8[di] = (uint8_t)code;
      } else {
        const float x = fp8x2_to_f32<false>(code)[0] * s_src;
        c8[di] = (uint8_t)f32_to_e4m3fn_sat(__fdiv_rn(x, s_dst));
      }
    }
  }
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
  const int32_t* table = p.tables + (int64_t)b * p.MBS;
  for (int k = 0; k < n; ++k) {
    const int node = s_path[k];
    if (node != k) {
      const int src = L + node, dst = L + k;
      const int64_t ps = table[src / kPage], pd = table[dst / kPage];
      move_row<KT>(p, p.k, p.k_scale, ps, src % kPage, pd, dst % kPage, tid);
      move_row<KT>(p, p.v, p.v_scale, ps, src % kPage, pd, dst % kPage, tid);
    }
    __syncthreads();          // entry k fully moved before entry k + 1 reads
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
