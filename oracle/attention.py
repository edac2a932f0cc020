"""Paged tree attention, written as its plain definition in float64.

What is computed (TACO-LLM pages):
  * The KV cache of each sequence is split into fixed-size blocks; a block
    table maps each sequence's consecutive logical blocks to non-contiguous
    physical blocks (design talk 大模型倍速推理引擎 TACO-LLM 的设计与实践,
    section "4. 支持 Paged Attention").
  * In a lookahead step the target model validates several candidate tokens
    in one forward pass; candidates that share a prefix are merged into one
    tree-attention computation (same talk, sections "优化方案设计思路" and
    "优化策略总结" item 1).
  * TurboAttention combines page management with a FlashAttention-style
    kernel (618zxw.cn article, section "長シーケンス推論最適化における
    TurboAttention"; talk, bullets on Paged Attention / FlashAttention in
    "整体方案分为两大部分").  Flash-style streaming and split-K only reorder
    the same exact softmax attention, so the oracle is that attention itself,
    materialised, two-pass, with no streaming.

Readings adopted where the pages are silent:
  * ctx_lens[b] counts the q_lens[b] candidates, whose K/V occupy the last
    q_lens[b] logical positions L..C-1 (L = C - q_b).
  * A candidate attends to every committed position t < L and to candidate
    positions L + j with tree_mask[b, i, j] != 0; positions t >= C are never
    used.
  * q-head h reads KV head h // (Hq // Hkv).
  * Physical cache layout [num_blocks, Hkv, page, D]; Q and out layout
    [B, Qmax, Hq, D]; rows i >= q_lens[b] are padding.
  * A row with no visible key gives out = 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import decode_bf16, decode_fp8_e4m3fn

PAGE = 16


def _decode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "fp8":
        return decode_fp8_e4m3fn(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def gather_page_rows(cache: np.ndarray, table_row: np.ndarray, kv_head: int, ctx_len: int,
                     dtype: str, scales: np.ndarray | None = None,
                     page_size: int = PAGE) -> np.ndarray:
    """Logical rows 0..ctx_len-1 of one KV head, in float64 [ctx_len, D].

    Logical position t lives in physical block table_row[t // page_size] at
    slot t % page_size (Paged Attention section of the design talk).  For fp8
    the stored code is decoded exactly and multiplied by that block's scale
    for this KV head.
    """
    t = np.arange(ctx_len, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // page_size]
    slot = t % page_size
    rows = _decode(cache[phys, kv_head, slot, :], dtype)
    if dtype == "fp8":
        if scales is None:
            raise ValueError("fp8 cache needs per-(block, KV head) scales")
        rows = rows * np.asarray(scales, dtype=np.float32).astype(np.float64)[phys, kv_head][:, None]
    return rows


def kv_head_of(q_head: int, group: int) -> int:
    """GQA: consecutive groups of `group` q-heads share one KV head."""
    return q_head // group


def visibility(ctx_len: int, q_len: int, tree_mask_b: np.ndarray) -> np.ndarray:
    """bool [q_len, ctx_len]: which logical key positions candidate i may attend.

    Committed prefix positions t < L are visible to every candidate; candidate
    position L + j is visible to candidate i iff tree_mask[i, j] is set (tree
    attention over shared prefixes, "优化策略总结" item 1 of the design talk).
    """
    L = ctx_len - q_len
    vis = np.zeros((q_len, ctx_len), dtype=bool)
    vis[:, :L] = True
    vis[:, L:] = np.asarray(tree_mask_b)[:q_len, :q_len] != 0
    return vis


def _attend(scores: np.ndarray, vis: np.ndarray, values: np.ndarray):
    """Masked softmax attention of score rows over value rows (float64).

    out_i = sum_t w_it V_t / sum_t w_it with w_it = exp(s_it - m_i) over the
    visible t, m_i = max over visible s_it; lse_i = m_i + ln(sum_t w_it).
    """
    n = scores.shape[0]
    out = np.zeros((n, values.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    any_vis = vis.any(axis=1)
    if not any_vis.any():
        return out, lse
    s = np.where(vis, scores, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    m_safe = np.where(any_vis, m, 0.0)
    w = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = w.sum(axis=1)
    num = w @ values
    out[any_vis] = num[any_vis] / l[any_vis, None]
    lse[any_vis] = m_safe[any_vis] + np.log(l[any_vis])
    return out, lse


def _inputs(q, k_cache, v_cache, q_dtype):
    q = np.asarray(q)
    if q.ndim != 4:
        raise ValueError("q must be [B, Qmax, Hq, D]")
    B, Qmax, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return _decode(q, q_dtype), B, Qmax, Hq, D, Hkv, Hq // Hkv


def paged_tree_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, scale, *,
                    q_dtype: str, kv_dtype: str, k_scale=None, v_scale=None,
                    page_size: int = PAGE):
    """Exact paged tree attention.

    Returns (out, lse): out float64 [B, Qmax, Hq, D] with NaN in padding rows,
    lse float64 [B, Hq, Qmax] (natural log) with NaN in padding rows.
    """
    qf, B, Qmax, Hq, D, Hkv, G = _inputs(q, k_cache, v_cache, q_dtype)
    out = np.full((B, Qmax, Hq, D), np.nan)
    lse = np.full((B, Hq, Qmax), np.nan)
    for b in range(B):
        C, Qb = int(ctx_lens[b]), int(q_lens[b])
        vis = visibility(C, Qb, tree_mask[b])
        K = [gather_page_rows(k_cache, block_tables[b], hk, C, kv_dtype, k_scale, page_size)
             for hk in range(Hkv)]
        V = [gather_page_rows(v_cache, block_tables[b], hk, C, kv_dtype, v_scale, page_size)
             for hk in range(Hkv)]
        for h in range(Hq):
            hk = kv_head_of(h, G)
            S = float(scale) * (qf[b, :Qb, h, :] @ K[hk].T)
            o, l = _attend(S, vis, V[hk])
            out[b, :Qb, h, :] = o
            lse[b, h, :Qb] = l
    return out, lse


def paged_tree_attn_partials(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                             scale, partition_tokens: int, *, q_dtype: str, kv_dtype: str,
                             k_scale=None, v_scale=None, page_size: int = PAGE):
    """Per-partition attention for split-K over long contexts.

    Partition p covers logical positions [p*T, (p+1)*T) clipped to ctx_len
    (T = partition_tokens).  Each partition yields its own normalised output
    O_p and log-sum-exp LSE_p over the keys it holds; partitions with no
    visible key (or past ctx_len) give O_p = 0, LSE_p = -inf.  This is the
    decomposition that lets on-chip resources stay independent of sequence
    length ("优化策略总结" item 2 of the design talk).

    Returns (O [B, Qmax, Hq, P, D], LSE [B, Hq, Qmax, P]) with
    P = ceil(max(ctx_lens) / T); padding rows are NaN.
    """
    T = int(partition_tokens)
    if T <= 0:
        raise ValueError("partition_tokens must be positive")
    qf, B, Qmax, Hq, D, Hkv, G = _inputs(q, k_cache, v_cache, q_dtype)
    P = max(1, math.ceil(int(np.max(ctx_lens)) / T))
    O = np.full((B, Qmax, Hq, P, D), np.nan)
    LSE = np.full((B, Hq, Qmax, P), np.nan)
    for b in range(B):
        C, Qb = int(ctx_lens[b]), int(q_lens[b])
        vis = visibility(C, Qb, tree_mask[b])
        O[b, :Qb] = 0.0
        LSE[b, :, :Qb] = -np.inf
        K = [gather_page_rows(k_cache, block_tables[b], hk, C, kv_dtype, k_scale, page_size)
             for hk in range(Hkv)]
        V = [gather_page_rows(v_cache, block_tables[b], hk, C, kv_dtype, v_scale, page_size)
             for hk in range(Hkv)]
        for h in range(Hq):
            hk = kv_head_of(h, G)
            S = float(scale) * (qf[b, :Qb, h, :] @ K[hk].T)
            for p in range(P):
                lo, hi = p * T, min((p + 1) * T, C)
                if lo >= hi:
                    continue
                o, l = _attend(S[:, lo:hi], vis[:, lo:hi], V[hk][lo:hi])
                O[b, :Qb, h, p, :] = o
                LSE[b, h, :Qb, p] = l
    return O, LSE


def merge_partials(O: np.ndarray, LSE: np.ndarray):
    """Combine per-partition results by log-sum-exp.

    LSE = ln sum_p exp(LSE_p);  out = sum_p exp(LSE_p - LSE) * O_p.
    Rows whose partitions are all empty give out = 0, LSE = -inf; NaN padding
    rows stay NaN.  Shapes as returned by paged_tree_attn_partials.
    """
    B, Qmax, Hq, P, D = O.shape
    out = np.full((B, Qmax, Hq, D), np.nan)
    lse = np.full((B, Hq, Qmax), np.nan)
    for b in range(B):
        for h in range(Hq):
            for i in range(Qmax):
                lp = LSE[b, h, i]
                if np.isnan(lp).any():
                    continue
                finite = np.isfinite(lp)
                if not finite.any():
                    out[b, i, h] = 0.0
                    lse[b, h, i] = -np.inf
                    continue
                mx = lp[finite].max()
                tot = mx + math.log(np.exp(lp[finite] - mx).sum())
                wts = np.where(finite, np.exp(np.where(finite, lp, 0.0) - tot), 0.0)
                out[b, i, h] = (wts[:, None] * np.nan_to_num(O[b, i, h])).sum(axis=0)
                lse[b, h, i] = tot
    return out, lse
