/*
 * libpta — paged tree attention for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Every array argument is a DEVICE pointer, except the dims
 * struct, which is a HOST pointer read during the call.  The caller owns every
 * buffer (including the split-K workspace); the library never allocates,
 * frees, synchronises or keeps a pointer after a call returns.  Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = default stream).
 * Errors are returned as a status, never thrown: all host-checkable errors
 * are detected before any HIP call is made; a failed launch returns
 * PTA_ERR_HIP.  Global state: a per-device table of kernel occupancies,
 * filled on the first launch on each device (idempotent, so calls from
 * several threads are safe), and the device array behind
 * taco_paged_tree_attn_balanced_noalloc (PTA_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's first use on that GPU until the process ends);
 * nothing else persists between calls.
 *
 * What is computed (sources: the TACO-LLM pages):
 *   - KV cache split into fixed-size blocks of tokens; each sequence's
 *     consecutive logical blocks map to non-contiguous physical blocks through
 *     a block table (design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践",
 *     section "4. 支持 Paged Attention").
 *   - Lookahead verification: each sequence carries q_len >= 1 candidate
 *     tokens arranged as a tree; candidates sharing a prefix are computed in
 *     one tree attention (same talk, sections "优化方案设计思路" and
 *     "优化策略总结" item 1), which turns the per-sequence decode GEMV into a
 *     small GEMM ("整体方案分为两大部分", TurboAttention bullets).
 *   - FlashAttention-style streaming so on-chip resources do not depend on
 *     sequence length (same bullets; "优化策略总结" item 2), and a split over
 *     the sequence for long contexts (618zxw.cn article, section
 *     "長シーケンス推論最適化におけるTurboAttention").
 *   - 8-bit floating point KV storage with fast dequantisation inside the
 *     attention operator (618zxw.cn article, section "LLM量子化技術による
 *     推論コストの削減"; talk section "5. 支持 Quantization").
 *
 * Semantics (exact masked softmax attention; rounding aside):
 *   for sequence b: C = ctx_lens[b] (INCLUDES the q_b = q_lens[b] candidates,
 *   whose K/V occupy logical positions L..C-1, L = C - q_b).  Logical
 *   position t is slot t % 16 of physical block block_tables[b][t / 16].
 *   q-head h uses KV head h / (Hq / Hkv).  Candidate i (< q_b) sees every
 *   t < L, and t = L + j iff tree_mask[b][i][j] != 0.  Then
 *     s_t   = scale * <q[b][i][h][:], K_t>
 *     out   = sum_t softmax(s)_t * V_t        (rounded to the q dtype)
 *     lse   = ln sum_t exp(s_t)               (natural log, fp32)
 *   A row with no visible key gives out = 0, lse = -inf.
 *
 * Layouts (row-major, contiguous):
 *   q, out        [num_seqs][max_q_len][num_q_heads][head_dim]  (q dtype)
 *   k_cache,
 *   v_cache       [num_blocks][num_kv_heads][page_size][head_dim] (kv dtype)
 *   k_scale,
 *   v_scale       [num_blocks][num_kv_heads] float (fp8 KV only, else NULL):
 *                 stored value x is represented by code * scale
 *   block_tables  [num_seqs][max_blocks_per_seq] int32
 *   ctx_lens,
 *   q_lens        [num_seqs] int32
 *   tree_mask     [num_seqs][max_q_len][max_q_len] uint8 (may be NULL only
 *                 when max_q_len == 1)
 *   lse           [num_seqs][num_q_heads][max_q_len] float, or NULL
 * Rows i >= q_lens[b] of out and lse are not written.
 *
 * Caller contract checked only on the device (see taco_pta_validate):
 *   1 <= q_lens[b] <= max_q_len, q_lens[b] <= ctx_lens[b] <= max_ctx_len,
 *   ctx_lens[b] <= page_size * max_blocks_per_seq, and every table entry
 *   below ceil(ctx_lens[b] / page_size) is in [0, num_blocks).  Breaking it
 *   gives undefined results.  Table entries past that count and cache slots
 *   past ctx_lens[b] are never read for their values (they may hold NaN).
 */
#ifndef PTA_H
#define PTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PTA_OK = 0,
  PTA_ERR_NULL_PTR = 1,          /* a required pointer is NULL */
  PTA_ERR_BAD_DIMS = 2,          /* a size is out of range or inconsistent */
  PTA_ERR_BAD_DTYPE = 3,         /* unsupported dtype or dtype combination */
  PTA_ERR_UNSUPPORTED = 4,       /* valid request outside what is built (e.g. forced path) */
  PTA_ERR_WORKSPACE_TOO_SMALL = 5,
  PTA_ERR_HIP = 6                /* a HIP runtime call or launch failed */
} pta_status;

typedef enum { PTA_F32 = 0, PTA_BF16 = 1, PTA_FP8_E4M3FN = 2 } pta_dtype;

/* Kernel family selection.  AUTO picks per call from the rows per KV head
 * (G * max_q_len): vector ALU for small row counts, MFMA otherwise.  TILE
 * forces the shared-tile matrix-core family (every wave of a workgroup reads
 * the same LDS pages) for any row count up to 256 with bf16 q.  TILE16 is TILE
 * with the balanced entry's shared-tile grid held to its 16x16x32-product
 * kernel (the one also used when a bf16 cache tensor exceeds 4 GiB; otherwise
 * the balanced entry runs the 32x32x16-product kernel); same results within
 * rounding. */
typedef enum {
  PTA_PATH_AUTO = 0,
  PTA_PATH_VALU = 1,
  PTA_PATH_MFMA = 2,
  PTA_PATH_TILE = 3,
  PTA_PATH_TILE16 = 4
} pta_path;

typedef struct {
  int32_t num_seqs;            /* B >= 0 (0 is a no-op) */
  int32_t num_q_heads;         /* Hq >= 1, multiple of num_kv_heads */
  int32_t num_kv_heads;        /* Hkv >= 1 */
  int32_t head_dim;            /* 64 or 128 */
  int32_t page_size;           /* must be 16 */
  int32_t max_q_len;           /* row stride of q/out/tree_mask; 1..64 */
  int32_t max_blocks_per_seq;  /* block_tables row stride, >= 1 */
  int32_t max_ctx_len;         /* host-known bound on ctx_lens (grid sizing), >= 1 */
  int64_t num_blocks;          /* physical blocks in the pool, >= 1 */
  int32_t q_dtype;             /* pta_dtype: F32 or BF16; out has the same dtype */
  int32_t kv_dtype;            /* pta_dtype: F32 (needs F32 q), BF16 or FP8_E4M3FN (need BF16 q) */
  int32_t path;                /* pta_path */
  int32_t flags;               /* pta_flags bits; others must be 0 */
} pta_dims;

/* Hints in pta_dims.flags.
 *   PTA_FLAG_SHARED_PAGES: the block tables may name one physical page for
 *   several sequences (a shared prefix read through the whole-context or
 *   balanced entries).  Without it, page tiles that one workgroup alone reads
 *   are loaded with the nontemporal (streaming) cache hint, which measured
 *   8-11% faster on the decode-shaped and fp8 calls and 9% on the 70B verify;
 *   pages read by several sequences are then fetched from memory by each of
 *   them instead of hitting in the caches.  Results are identical either way. */
#define PTA_FLAG_SHARED_PAGES 1

/* Paged tree attention, one pass over each sequence's whole context.
 * scale: softmax scale (finite).  lse may be NULL. */
pta_status taco_paged_tree_attn(const pta_dims* dims, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* ctx_lens,
                                const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                                void* out, float* lse, void* stream);

/* The verify step's KV append fused into the whole-context attention call:
 * every sequence's q_lens[b] new K and V rows (the candidates, logical
 * positions L .. C - 1 with L = ctx_lens[b] - q_lens[b]) are written into their
 * paged slots of k_cache / v_cache, then attention runs as in
 * taco_paged_tree_attn over the updated cache, in one launch (the candidates'
 * K/V are appended before they are attended to, design talk "4. 支持 Paged
 * Attention": blocks are filled as tokens arrive).
 *   k_new, v_new  [num_seqs][max_q_len][num_kv_heads][head_dim], 16-byte
 *                 aligned (else PTA_ERR_BAD_DIMS), rows past q_lens ignored; new_dtype = PTA_BF16 for bf16 caches,
 *                 PTA_F32 or PTA_BF16 for fp8 caches, whose slots get
 *                 RNE-saturated e4m3fn codes of x / scale with the slot's
 *                 existing (block, KV head) scale (as taco_kv_append).
 * Served where the whole-context matrix-core stream kernel runs (bf16 q,
 * num_q_heads / num_kv_heads * max_q_len <= 32, no forced VALU or tile path),
 * else PTA_ERR_UNSUPPORTED (use taco_kv_append, then taco_paged_tree_attn).
 * Other arguments and errors as taco_paged_tree_attn. */
pta_status taco_paged_tree_attn_append(const pta_dims* dims, const void* q, const void* k_new,
                                       const void* v_new, int32_t new_dtype, void* k_cache, void* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, const int32_t* ctx_lens,
                                       const int32_t* q_lens, const uint8_t* tree_mask, float scale,
                                       void* out, float* lse, void* stream);

/* Bytes of device workspace taken by taco_paged_tree_attn_splitk for these dims
 * and partition length (0 on invalid input). */
size_t taco_paged_tree_attn_splitk_workspace_size(const pta_dims* dims, int32_t partition_tokens);

/* Split-K paged tree attention for long contexts: each sequence is cut into
 * partitions of partition_tokens logical positions (a positive multiple of
 * 32), attention over each partition runs as an independent work unit that
 * writes its normalised partial output and log-sum-exp into `workspace`, and
 * the last unit of each (sequence, KV head) to finish merges the partitions by
 * log-sum-exp into out/lse, inside the same kernel launch (the long-sequence
 * part of the 618zxw.cn article, section "長シーケンス推論最適化における
 * TurboAttention": the sequence is processed in independent parts that are
 * combined).  The merge reads partitions in index order, so results do not
 * depend on scheduling.  Arguments otherwise as taco_paged_tree_attn.
 *
 * workspace: caller-owned device memory, 256-byte aligned (else
 * PTA_ERR_BAD_DIMS), of at least workspace_bytes >=
 * taco_paged_tree_attn_splitk_workspace_size(dims, partition_tokens).  Its
 * first region (num_seqs * num_kv_heads int32 arrival counters, padded to 256
 * bytes) must be zero before the first call that uses this workspace (e.g. a
 * zero-filled allocation); every call leaves it zero again.  The rest of the
 * workspace needs no initialisation.  Calls that may run concurrently must not
 * share a workspace. */
pta_status taco_paged_tree_attn_splitk(const pta_dims* dims, const void* q, const void* k_cache,
                                       const void* v_cache, const float* k_scale,
                                       const float* v_scale, const int32_t* block_tables,
                                       const int32_t* ctx_lens, const int32_t* q_lens,
                                       const uint8_t* tree_mask, float scale, void* out,
                                       float* lse, int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Shared-prefix paged tree attention (the pages' prefix cache: sequences
 * whose block tables alias the same physical pages for a common prefix,
 * design talk "4. 支持 Paged Attention" and the 618zxw.cn article's Prefix
 * Cache).  Split-K with partition_tokens = shared_tokens, where partition 0
 * (logical positions 0 .. shared_tokens - 1) of every group of sequences is
 * worked once for all of the group's rows: the pages are read once per group
 * instead of once per sequence, and each member's later partitions are worked
 * as in taco_paged_tree_attn_splitk; the last unit of each (sequence, KV head)
 * merges its partitions by log-sum-exp in the same launch.
 *
 * prefix_leader: device int32 [num_seqs]; sequence b belongs to the group whose
 *   first sequence is prefix_leader[b]; a group is a run of consecutive
 *   sequences (prefix_leader[lead] == lead, then lead + 1, ... with the same
 *   leader), at most max_group of them.  A sequence with prefix_leader[b] == b
 *   and no followers is a group of one (its partition 0 is worked alone).
 * Caller contract (results are undefined otherwise; not checked on the
 *   device): within a group of two or more, the first shared_tokens / 16
 *   block-table entries of every member are equal, and every member's
 *   committed part (ctx_lens - q_lens) is at least shared_tokens.
 * max_group * (num_q_heads / num_kv_heads) * max_q_len must be at most 32 and
 *   q bf16 (the group's rows form one matrix-core stream unit), else
 *   PTA_ERR_UNSUPPORTED; shared_tokens a positive multiple of 32 (else
 *   PTA_ERR_BAD_DIMS).
 * workspace: as taco_paged_tree_attn_splitk with partition_tokens =
 *   shared_tokens (same size query, same zero-counter contract).  Other
 *   arguments as taco_paged_tree_attn. */
pta_status taco_paged_tree_attn_shared_prefix(const pta_dims* dims, const void* q, const void* k_cache,
                                              const void* v_cache, const float* k_scale,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* ctx_lens, const int32_t* q_lens,
                                              const uint8_t* tree_mask, const int32_t* prefix_leader,
                                              int32_t max_group, int32_t shared_tokens, float scale,
                                              void* out, float* lse, void* workspace,
                                              size_t workspace_bytes, void* stream);

/* Bytes of device workspace taken by taco_paged_tree_attn_balanced for these
 * dims on the current device (0 on invalid input or when the balanced mode
 * does not serve these dims). */
size_t taco_paged_tree_attn_balanced_workspace_size(const pta_dims* dims);

/* Work-balanced paged tree attention.  The pages of every (sequence, KV head)
 * unit are laid end to end and cut into equal contiguous slices worked by a
 * persistent grid sized to the current device, so ragged context lengths cost
 * no load imbalance (sequence-dimension parallelism, design talk
 * "优化策略总结" item 2; a sequence processed in parts that are combined,
 * 618zxw.cn article section "長シーケンス推論最適化におけるTurboAttention").
 * A slice holding a whole unit writes its rows directly; a slice that ends
 * inside a unit writes a normalised partial and log-sum-exp to the workspace,
 * and a second launch on the same stream merges each unit's partials in
 * slice order (results do not depend on scheduling).  Served for bf16 q with
 * num_seqs <= 16383 and either G * max_q_len <= 32 rows per KV head (the
 * matrix-core streaming path, one slice per wave) or, with bf16 KV, up to 256
 * rows (the shared-tile path: one workgroup per row group of up to 128 rows
 * per slice; also chosen for fewer rows by path PTA_PATH_TILE); otherwise
 * PTA_ERR_UNSUPPORTED.  Arguments as taco_paged_tree_attn.  workspace:
 * caller-owned device memory, 256-byte aligned (else PTA_ERR_BAD_DIMS), with
 * workspace_bytes >= taco_paged_tree_attn_balanced_workspace_size(dims); it
 * needs no initialisation, and calls that may run concurrently must not share
 * it. */
pta_status taco_paged_tree_attn_balanced(const pta_dims* dims, const void* q, const void* k_cache,
                                         const void* v_cache, const float* k_scale,
                                         const float* v_scale, const int32_t* block_tables,
                                         const int32_t* ctx_lens, const int32_t* q_lens,
                                         const uint8_t* tree_mask, float scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* The verify step's KV append fused into the balanced entry (as
 * taco_paged_tree_attn_append does for the whole-context one): every
 * sequence's q_lens[b] candidate K and V rows are written into their paged
 * slots (logical positions ctx_lens[b] - q_lens[b] ...), then attention runs as
 * in taco_paged_tree_attn_balanced over the updated cache, in the same grid.
 * Inside the grid, each slice writes the candidates that lie on its own pages
 * before it copies them, so the step needs no separate append launch.
 *   k_new, v_new  [num_seqs][max_q_len][num_kv_heads][head_dim] bf16, 16-byte
 *                 aligned (else PTA_ERR_BAD_DIMS), rows past q_lens ignored;
 *                 new_dtype must be PTA_BF16 (else PTA_ERR_BAD_DTYPE).
 * Served where the balanced entry runs its 32x32x16-product shared-tile grid
 * (bf16 q and KV, more than 32 rows per KV head or path PTA_PATH_TILE, caches
 * addressable with 32-bit offsets), else PTA_ERR_UNSUPPORTED (use
 * taco_kv_append, then taco_paged_tree_attn_balanced).  Workspace and other
 * arguments as taco_paged_tree_attn_balanced. */
pta_status taco_paged_tree_attn_balanced_append(const pta_dims* dims, const void* q, const void* k_new,
                                                const void* v_new, int32_t new_dtype, void* k_cache,
                                                void* v_cache, const int32_t* block_tables,
                                                const int32_t* ctx_lens, const int32_t* q_lens,
                                                const uint8_t* tree_mask, float scale, void* out, float* lse,
                                                void* workspace, size_t workspace_bytes, void* stream);

/* Largest balanced-entry workspace, in bytes, that
 * taco_paged_tree_attn_balanced_noalloc can serve (64 MiB). */
#define PTA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* taco_paged_tree_attn_balanced for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same kernels, same results and same arguments, minus the
 * workspace: it lives in a library-owned device array of
 * PTA_NOALLOC_SCRATCH_BYTES bytes per GPU.  The call allocates, frees and
 * synchronises nothing.
 *   - Needs taco_paged_tree_attn_balanced_workspace_size(dims) <=
 *     PTA_NOALLOC_SCRATCH_BYTES, else PTA_ERR_WORKSPACE_TOO_SMALL (the
 *     workloads this library is measured on take at most about 59 MB).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; it needs no initialisation (the grid writes every
 *     partial before the merge launch reads it).  Calls that may overlap on
 *     one GPU (other streams, other host threads) RACE and give undefined
 *     results; calls issued in order on one stream are safe.
 *   - The first call on a device looks up the address of that device's copy
 *     with the device current (a failure returns PTA_ERR_HIP).
 * Other arguments, semantics and errors as taco_paged_tree_attn_balanced. */
pta_status taco_paged_tree_attn_balanced_noalloc(const pta_dims* dims, const void* q, const void* k_cache,
                                                 const void* v_cache, const float* k_scale,
                                                 const float* v_scale, const int32_t* block_tables,
                                                 const int32_t* ctx_lens, const int32_t* q_lens,
                                                 const uint8_t* tree_mask, float scale, void* out,
                                                 float* lse, void* stream);

/* KV append: write num_tokens new K/V rows into their cache slots, as blocks
 * are handed out while tokens are generated (Paged Attention section of the
 * design talk).
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim] in new_dtype
 *                 (F32 or BF16; must equal kv_dtype unless kv_dtype is FP8)
 *   slot_mapping  [num_tokens] int64: slot = block * page_size + offset, or
 *                 negative to skip the token.  Slots must be < num_blocks *
 *                 page_size and distinct (duplicates race).
 *   fp8 caches store RNE-to-nearest-even e4m3fn of (x / scale) computed in
 *   float32, saturated to +-448, with the block's existing k_scale / v_scale.
 * Uses dims->num_kv_heads, head_dim, page_size, num_blocks, kv_dtype. */
pta_status taco_kv_append(const pta_dims* dims, const void* k_new, const void* v_new,
                          int32_t new_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                          void* k_cache, void* v_cache, const float* k_scale,
                          const float* v_scale, void* stream);

/* Acceptance and commit after a verify step (the step to the right of the
 * attention: the target model's prediction at each candidate decides which
 * candidates are kept, design talk section on Lookahead Decoding; several
 * tokens are generated per step, "2. 加速上限分析").  Greedy rule, per sequence:
 * parent(i) = the largest j < i with tree_mask[b][i][j] != 0 (-1: root); a
 * root is accepted iff cand_tokens[b][i] == target_prev[b]; another node iff
 * its parent is accepted and cand_tokens[b][i] == target_tokens[b][parent].
 * The committed path is the accepted node of greatest depth (lowest index
 * among equals) with its ancestors, in increasing index order.  Its K/V rows
 * move from logical position L + path[k] to L + k (L = ctx_lens[b] -
 * q_lens[b]) for every KV head, one entry after the other; fp8 rows are copied
 * when the source and destination (block, head) scales are equal, else
 * re-encoded as RNE_sat(value * s_src / s_dst) in float32.
 *   cand_tokens, target_tokens  [num_seqs][max_q_len] int32 (rows past q_lens ignored)
 *   target_prev   [num_seqs] int32: the prediction after the committed prefix
 *   ctx_lens, q_lens, tree_mask, block_tables: as for the attention call (read only)
 *   k_cache, v_cache (+ k_scale, v_scale for fp8): updated in place
 *   n_accepted    [num_seqs] int32 out: path length (0 when no root matches)
 *   accepted_path [num_seqs][max_q_len] int32 out: node indices, -1 after the path
 *   bonus_tokens  [num_seqs] int32 out: target_tokens at the path's last node,
 *                 or target_prev when the path is empty
 *   new_ctx_lens  [num_seqs] int32 out: L + n_accepted.  Cache rows past it are
 *                 untouched; blocks from ceil(new_ctx / page_size) on are free.
 * Errors: as taco_paged_tree_attn (dims, null pointers, dtype); the device
 * contract (lens, table entries) is the attention call's. */
pta_status taco_accept_commit(const pta_dims* dims, const int32_t* cand_tokens,
                              const int32_t* target_tokens, const int32_t* target_prev,
                              const int32_t* ctx_lens, const int32_t* q_lens,
                              const uint8_t* tree_mask, const int32_t* block_tables,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* v_scale, int32_t* n_accepted, int32_t* accepted_path,
                              int32_t* bonus_tokens, int32_t* new_ctx_lens, void* stream);

/* Device-side check of the caller contract above.  Writes into *d_flags (a
 * device int32, caller-owned; it is first cleared) the OR of:
 *   1 q_lens out of [1, max_q_len]     2 ctx_lens < q_lens or > max_ctx_len
 *   4 ctx_lens > page_size * max_blocks_per_seq
 *   8 a used block-table entry outside [0, num_blocks)
 * A debug/test aid: the attention entry points do not call it. */
pta_status taco_pta_validate(const pta_dims* dims, const int32_t* block_tables,
                             const int32_t* ctx_lens, const int32_t* q_lens, int32_t* d_flags,
                             void* stream);

/* Static, never NULL. */
const char* taco_pta_status_string(pta_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t taco_pta_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PTA_H */
