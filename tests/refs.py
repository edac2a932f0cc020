"""Independent references used to pin the oracle (test code only).

Nothing here calls the oracle's helpers.  Values are decoded with torch's own
bfloat16 / float8_e4m3fn types, pages are un-paged with a reshape of the
table's pages (not a per-token index), visibility comes from the candidates'
parent arrays (not the stored mask), and attention itself is torch's
scaled_dot_product_attention in float64 on the CPU.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

PAGE = 16


def torch_decode(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "f32":
        return t.to(torch.float64).numpy()
    if dtype == "bf16":
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "fp8":
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(dtype)


def unpage(pool: np.ndarray, table_row: np.ndarray, ctx_len: int, dtype: str,
           scales: np.ndarray | None = None) -> np.ndarray:
    """[Hkv, ctx_len, D] float64 from the pool by concatenating whole pages."""
    npages = -(-ctx_len // PAGE)
    ids = np.asarray(table_row[:npages], dtype=np.int64)
    tiles = torch_decode(pool[ids], dtype)                       # [P, Hkv, 16, D]
    if dtype == "fp8":
        tiles = tiles * np.asarray(scales, dtype=np.float64)[ids][:, :, None, None]
    hkv, d = tiles.shape[1], tiles.shape[3]
    seq = np.concatenate(list(tiles), axis=1) if npages else np.zeros((hkv, 0, d))
    return seq[:, :ctx_len, :]


def ancestors_or_self(parents: np.ndarray, i: int) -> list:
    out = []
    j = i
    while j >= 0:
        out.append(j)
        j = int(parents[j])
    return out


def vis_from_parents(ctx_len: int, q_len: int, parents: np.ndarray) -> np.ndarray:
    L = ctx_len - q_len
    vis = np.zeros((q_len, ctx_len), dtype=bool)
    vis[:, :L] = True
    for i in range(q_len):
        for j in ancestors_or_self(parents, i):
            vis[i, L + j] = True
    return vis


def sdpa(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, vis: np.ndarray, scale: float):
    """torch SDPA in float64; qrows [n, D], K/V [C, D], vis [n, C] -> [n, D]."""
    q = torch.from_numpy(qrows)[None, None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    m = torch.from_numpy(vis)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def workload_sdpa(w, use_stored_mask: bool = False) -> np.ndarray:
    """Whole-workload reference out [B, Qmax, Hq, D] (NaN padding rows)."""
    s = w.spec
    B, Qmax, Hq, D = w.q.shape
    Hkv = w.k_cache.shape[1]
    G = Hq // Hkv
    qd = torch_decode(w.q, s.q_dtype)
    out = np.full((B, Qmax, Hq, D), np.nan)
    for b in range(B):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        Kall = unpage(w.k_cache, w.block_tables[b], C, s.kv_dtype, w.k_scale)
        Vall = unpage(w.v_cache, w.block_tables[b], C, s.kv_dtype, w.v_scale)
        if use_stored_mask:
            L = C - Qb
            vis = np.concatenate([np.ones((Qb, L), bool), w.tree_mask[b, :Qb, :Qb] != 0], axis=1)
        else:
            vis = vis_from_parents(C, Qb, w.parents[b])
        for h in range(Hq):
            hk = h // G
            out[b, :Qb, h] = sdpa(qd[b, :Qb, h], Kall[hk], Vall[hk], vis, w.scale)
    return out
