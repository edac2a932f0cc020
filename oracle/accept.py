"""Acceptance of verified candidates and commit of their K/V (test infrastructure).

After the verify forward pass the target model has predicted one next token
per candidate position; the candidates it agrees with are kept and several
tokens are generated in one step (53ai.com workshop transcript, talk
大模型倍速推理引擎 TACO-LLM 的设计与实践, section on Lookahead Decoding: the
target model judges which candidate tokens are correct; section
"TACO-LLM 性能效果", "2. 加速上限分析": with 7 lookahead candidates about 3.5
are hit per step).  The pages give no rule beyond that; the readings adopted
here are the plain greedy ones:

  * parent(i) = the largest j < i with tree_mask[i][j] != 0 (with an
    ancestor-or-self mask and parents numbered before children this is the
    tree parent); a node with no such j is a root.
  * A root r is accepted iff cand[r] == target_prev (the target's prediction
    after the committed prefix; a caller whose node 0 is the token sampled in
    the previous step passes target_prev = cand[0]).  A non-root i is accepted
    iff its parent is accepted and cand[i] == target[parent(i)].
  * The committed path is the accepted node of greatest depth (smallest index
    among equals) and its ancestors, in increasing index order; n_accepted is
    its length (0 if no root is accepted).  bonus = target[last node of the
    path], or target_prev when nothing is accepted: the token the next step
    starts from.
  * Commit: the K/V rows of path node k move from logical position L + path[k]
    to L + k (L = ctx_len - q_len), through the block table, for every KV head;
    the new context length is L + n_accepted.  Rows at positions past it are
    left as they are (their pages from ceil(new_ctx / 16) on are free for the
    caller's pool).  f32/bf16 rows are copied bit-exactly.  An fp8 row is
    copied as is when its source and destination (page, KV head) scales are
    equal; otherwise it is re-encoded: x = value(code) * s_src in float32,
    code' = RNE_sat(x / s_dst) with the division in float32.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_fp8_e4m3fn, encode_fp8_e4m3fn

PAGE = 16


def tree_parents(mask_rows: np.ndarray, q: int) -> np.ndarray:
    """parent[i] for i < q from the rows of an ancestor-or-self mask (-1 = root)."""
    par = np.full(q, -1, dtype=np.int64)
    for i in range(q):
        for j in range(i - 1, -1, -1):
            if mask_rows[i][j]:
                par[i] = j
                break
    return par


def accept_path(parents, cand, target, target_prev):
    """Greedy acceptance over one candidate tree: (path, bonus)."""
    q = len(parents)
    acc = [False] * q
    depth = [0] * q
    for i in range(q):                      # parents come before children
        p = int(parents[i])
        if p < 0:
            acc[i] = int(cand[i]) == int(target_prev)
            depth[i] = 1
        else:
            acc[i] = acc[p] and int(cand[i]) == int(target[p])
            depth[i] = depth[p] + 1
    best = -1
    for i in range(q):
        if acc[i] and (best < 0 or depth[i] > depth[best]):
            best = i
    if best < 0:
        return [], int(target_prev)
    path = []
    i = best
    while i >= 0:
        path.append(i)
        i = int(parents[i])
    path.reverse()
    return path, int(target[best])


def _fp8_move(code, s_src, s_dst):
    if np.float32(s_src) == np.float32(s_dst):
        return code
    x = decode_fp8_e4m3fn(np.asarray(code)).astype(np.float32) * np.float32(s_src)       # float32 product
    quot = (x / np.float32(s_dst)).astype(np.float32)                                   # float32 quotient
    return encode_fp8_e4m3fn(quot.astype(np.float64))


def accept_commit(ctx_lens, q_lens, tree_mask, cand, target, target_prev, block_tables,
                  k_cache, v_cache, *, kv_dtype: str, k_scale=None, v_scale=None):
    """Return (n_accepted [B], path [B, Qmax] (-1 padded), bonus [B], new_ctx [B],
    k_cache', v_cache') for a batch."""
    B, Qmax = np.asarray(cand).shape
    n_acc = np.zeros(B, dtype=np.int32)
    paths = np.full((B, Qmax), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    new_ctx = np.zeros(B, dtype=np.int32)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for b in range(B):
        C, q = int(ctx_lens[b]), int(q_lens[b])
        L = C - q
        rows = np.asarray(tree_mask[b]) if tree_mask is not None else np.ones((1, 1), dtype=np.uint8)
        par = tree_parents(rows, q)
        path, bon = accept_path(par, cand[b][:q], target[b][:q], target_prev[b])
        n_acc[b] = len(path)
        paths[b, :len(path)] = path
        bonus[b] = bon
        new_ctx[b] = L + len(path)
        for k, node in enumerate(path):           # increasing k: sources are never overwritten early
            if node == k:
                continue
            src, dst = L + node, L + k
            ps, os_ = int(block_tables[b][src // PAGE]), src % PAGE
            pd, od = int(block_tables[b][dst // PAGE]), dst % PAGE
            for cache, scl in ((k_out, k_scale), (v_out, v_scale)):
                if kv_dtype == "fp8":
                    for h in range(cache.shape[1]):
                        cache[pd, h, od, :] = _fp8_move(cache[ps, h, os_, :], scl[ps, h], scl[pd, h])
                else:
                    cache[pd, :, od, :] = cache[ps, :, os_, :]
    return n_acc, paths, bonus, new_ctx, k_out, v_out
