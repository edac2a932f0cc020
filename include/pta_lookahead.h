/* Lookahead cache: the host-side step to the left of the verify pass, which
 * proposes each sequence's candidate tokens and their tree (the tree_mask of
 * the attention call).  Design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践",
 * section "优化方案设计思路", part "1.基于批处理的 Lookahead Cache": every
 * sequence of a batch keeps a local cache, all of them share one global
 * cache, a query is answered by the longest match of the sequence's recent
 * tokens, the answer is a multi-branch forest, and the candidate length of
 * each sequence is adapted to its hit rate and to the batch size (also
 * "优化策略总结" item 1).
 *
 * Readings (the talk gives no data structure or formula):
 *   - a cache counts, for every token string p of length 1 .. window that
 *     occurs inside a sequence's history, the number of its occurrences; the
 *     local cache of a sequence counts its own history, the global cache the
 *     histories of every sequence ever appended (released ones included);
 *   - a query for sequence s takes the longest suffix of s's history, of
 *     length k <= min(max_match, window - 1), that has at least one
 *     continuation in either cache; the candidates are strings p + x that
 *     extend that suffix, scored local(p + x) + global(p + x), chosen best
 *     first (highest score, then lowest parent index, then lowest token id)
 *     while the budget lasts, each chosen node making its own continuations
 *     eligible.  Roots (parent -1) continue the committed context;
 *   - the hit rate is a per-sequence running mean in 16.16 fixed point,
 *     h <- (h + 65536 * accepted / proposed) / 2 after every step that
 *     proposed something (starting at 1.0); the budget is
 *     clamp(round(max_len * h), min_len, max_len), and when the batch's
 *     budgets add up to more than batch_cap each is scaled by
 *     batch_cap / total (floor), never below min_len.
 * Everything is integer arithmetic: results are exact and repeatable.
 *
 * Host memory only (plain host pointers); one cache must not be used from two
 * threads at once (its calls may run on the cache's own worker threads, see
 * taco_la_set_threads).  Errors are pta_status codes (pta.h); nothing is
 * changed when a call fails its argument checks. */
#ifndef PTA_LOOKAHEAD_H
#define PTA_LOOKAHEAD_H

#include <stdint.h>

#include "pta.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct taco_la_cache taco_la_cache;

/* A new, empty cache.  window: longest counted string (2 .. 64); max_match:
 * longest suffix matched by a query (1 .. window - 1).  NULL on bad arguments
 * or out of memory.  Free with taco_la_destroy. */
taco_la_cache* taco_la_create(int32_t window, int32_t max_match);
void taco_la_destroy(taco_la_cache* cache);

/* Run the cache's batch calls (taco_la_append_batch, taco_la_append,
 * taco_la_propose) on n threads: the calling thread and n - 1 workers owned by
 * the cache (1 .. 64; a new cache has 1, no workers).  An append batch splits
 * into one task per sequence (its local counts) and one per shard of the
 * global counts (strings grouped by their first token); a query batch into one
 * task per sequence.  Results do not depend on n.  Idle workers spin for about
 * a millisecond before they sleep (a call after a longer pause first wakes
 * them).  A child process after fork() finds none of the workers: there the
 * cache runs on the calling thread (and reports 1) until taco_la_set_threads
 * starts new ones.  PTA_ERR_BAD_DIMS for n outside 1 .. 64;
 * PTA_ERR_UNSUPPORTED when the system refuses a thread (the cache is then left
 * with 1). */
pta_status taco_la_set_threads(taco_la_cache* cache, int32_t n);

/* The cache's thread count (0 for a NULL cache). */
int32_t taco_la_threads(const taco_la_cache* cache);

/* Append n >= 0 tokens (ids >= 0) to the history of sequence seq (>= 0; a
 * sequence not seen before starts empty), counting the new strings in its
 * local cache and in the global cache.  PTA_ERR_NULL_PTR (cache, or tokens
 * with n > 0), PTA_ERR_BAD_DIMS (seq < 0, n < 0, a negative token). */
pta_status taco_la_append(taco_la_cache* cache, int32_t seq, const int32_t* tokens, int32_t n);

/* taco_la_append for num_seqs sequences in one call: seqs[i] gets lens[i]
 * tokens, taken in order from tokens (sum of lens entries).  Checks as
 * taco_la_append, all before any change. */
pta_status taco_la_append_batch(taco_la_cache* cache, int32_t num_seqs, const int32_t* seqs,
                                const int32_t* lens, const int32_t* tokens);

/* Drop sequence seq's history, local cache and hit rate (the global counts
 * stay).  Unknown seq: no-op. */
pta_status taco_la_release(taco_la_cache* cache, int32_t seq);

/* Propose candidates for num_seqs sequences.
 *   seqs     [num_seqs]  sequence ids (unknown ids have an empty history)
 *   budgets  [num_seqs]  candidates wanted per sequence (0 .. max_q)
 *   tokens   [num_seqs][max_q] out: candidate token ids, -1 past count
 *   parents  [num_seqs][max_q] out: parent index (< own index), -1 for a
 *            root, -1 past count
 *   counts   [num_seqs] out: candidates proposed (0 when nothing matches)
 * PTA_ERR_BAD_DIMS: num_seqs < 0, max_q < 1, a budget outside 0 .. max_q. */
pta_status taco_la_propose(taco_la_cache* cache, int32_t num_seqs, const int32_t* seqs,
                           const int32_t* budgets, int32_t max_q, int32_t* tokens, int32_t* parents,
                           int32_t* counts);

/* Feed back the last step (proposed[i] candidates of which accepted[i] were
 * accepted, 0 <= accepted <= proposed) and compute the next budgets with
 * 0 <= min_len <= max_len and batch_cap >= 0 (0: no batch limit). */
pta_status taco_la_update_budgets(taco_la_cache* cache, int32_t num_seqs, const int32_t* seqs,
                                  const int32_t* proposed, const int32_t* accepted, int32_t min_len,
                                  int32_t max_len, int32_t batch_cap, int32_t* budgets);

/* The attention call's tree_mask from parent arrays: mask[s][i][j] = 1 iff
 * i, j < counts[s] and j is i or an ancestor of i; every other byte 0.
 *   parents [num_seqs][max_q], counts [num_seqs], mask [num_seqs][max_q][max_q]
 * PTA_ERR_BAD_DIMS for a count outside 0 .. max_q or a parent not below its
 * node's index. */
pta_status taco_la_tree_mask(int32_t num_seqs, int32_t max_q, const int32_t* parents,
                             const int32_t* counts, uint8_t* mask);

#ifdef __cplusplus
}
#endif

#endif
