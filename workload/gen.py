"""Seeded synthetic workloads for paged tree attention (inputs only).

The workloads follow the shapes the TACO-LLM pages motivate: a batch of
sequences whose KV cache lives in fixed-size pages reached through a block
table (design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践", section
"4. 支持 Paged Attention"), and per-sequence lookahead candidates arranged as a
token tree (same talk, sections "整体方案分为两大部分" and "优化策略总结").

Nothing here computes attention, a mask visibility rule beyond building the
ancestor-or-self relation of a sampled tree, or any step of the KV append.
Random streams: one ``numpy.random.SeedSequence`` per workload seed, with a
child stream per purpose and, for the K/V values, one grandchild per sequence,
so generation can run in threads and still be reproducible.

Stored element formats:
  f32   numpy float32
  bf16  numpy uint16 holding the upper half of the IEEE float32 pattern
        (round-to-nearest-even from float32)
  fp8   numpy uint8 holding OCP e4m3fn codes, with float32 scales per
        (page, KV head); codes are produced by torch's float8_e4m3fn cast
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

PAGE = 16                      # tokens per KV page
FP8_MAX = 448.0                # largest finite OCP e4m3fn magnitude
DTYPES = ("f32", "bf16", "fp8")


# --------------------------------------------------------------------------
# element-format helpers (conversions only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + (0x7FFF + ((u >> 16) & 1))) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp8_codes(x_over_scale: np.ndarray) -> np.ndarray:
    """float32 values already divided by their scale -> e4m3fn codes (torch cast)."""
    import torch
    t = torch.from_numpy(np.clip(x_over_scale, -FP8_MAX, FP8_MAX).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------------
# trees
# --------------------------------------------------------------------------
def _depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i, p in enumerate(parents):
        d[i] = 1 if p < 0 else d[p] + 1
    return d


def sample_tree_parents(rng: np.random.Generator, n: int, kind: str,
                        depth_cap: Optional[int]) -> np.ndarray:
    """Parent array of an n-node candidate tree; node 0 is the root (parent -1).

    kind "chain":  parent[i] = i - 1.
    kind "random": parent[i] uniform in {0..i-1}; when depth_cap is set, whole
                   trees whose deepest root-to-leaf path has more than
                   depth_cap nodes are rejected and redrawn.
    kind "flat":   every candidate is a root of its own (no shared path).
    """
    if kind == "chain":
        return np.arange(-1, n - 1, dtype=np.int32)
    if kind == "flat":
        return np.full(n, -1, dtype=np.int32)
    if kind != "random":
        raise ValueError(kind)
    for _ in range(100000):
        par = np.empty(n, dtype=np.int32)
        par[0] = -1
        for i in range(1, n):
            par[i] = rng.integers(0, i)
        if depth_cap is None or _depths(par).max() <= depth_cap:
            return par
    raise RuntimeError("tree rejection sampling did not converge")


def tree_mask_from_parents(parents: np.ndarray, qmax: int) -> np.ndarray:
    """Ancestor-or-self relation as a dense uint8 [qmax, qmax] matrix."""
    n = len(parents)
    m = np.zeros((qmax, qmax), dtype=np.uint8)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j] = 1
            j = int(parents[j])
    return m


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str = "bf16"
    kv_dtype: str = "bf16"
    ctx_list: Optional[tuple] = None          # explicit context lengths
    ctx_range: Optional[tuple] = None         # (lo, hi) inclusive, uniform integers
    q_len: int = 1                            # max candidates per sequence
    q_len_ragged: bool = False                # per-seq q_b uniform in [1, q_len]
    tree: str = "chain"                       # chain | random | flat
    depth_cap: Optional[int] = None
    pool_factor: float = 1.2                  # pool pages = ceil(f * pages used)
    pool_pages: Optional[int] = None          # explicit pool size (overrides f)
    scale: Optional[float] = None             # softmax scale; None -> 1/sqrt(D)
    split_tokens: Optional[int] = None        # split-K partition length
    seed: int = 0
    # shared prefix: consecutive groups of `share_group` sequences alias their first
    # `shared_prefix_pages` pages (same physical pages, same K/V); 0 = no sharing
    share_group: int = 1
    shared_prefix_pages: int = 0

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    # tiny decode: fp32, 16-page permuted pool, ctx {37, 80}, q=1, scale 1/8
    "tiny_decode": Spec("tiny_decode", 2, 4, 4, 64, "f32", "f32", ctx_list=(37, 80),
                        q_len=1, tree="chain", pool_pages=16, scale=1.0 / 8, seed=0),
    # Llama-3-8B-shaped decode
    "llama3_8b_decode": Spec("llama3_8b_decode", 64, 32, 8, 128, "bf16", "bf16",
                             ctx_range=(512, 4096), q_len=1, tree="chain", seed=1),
    # Llama-3.1-70B-shaped lookahead verify, 16-candidate random tree of depth <= 6
    "llama31_70b_verify": Spec("llama31_70b_verify", 32, 64, 8, 128, "bf16", "bf16",
                               ctx_range=(1024, 8192), q_len=16, tree="random",
                               depth_cap=6, seed=2),
    # long-sequence verify with 2048-token split-K partitions
    "long_splitk_verify": Spec("long_splitk_verify", 4, 64, 8, 128, "bf16", "bf16",
                               ctx_range=(32768, 131072), q_len=32, tree="random",
                               depth_cap=8, split_tokens=2048, seed=3),
    # fp8 e4m3fn KV with per-(page, KV head) scales, 8-candidate chain
    "fp8_kv_chain": Spec("fp8_kv_chain", 128, 32, 8, 128, "bf16", "fp8",
                         ctx_range=(2048, 16384), q_len=8, tree="chain", seed=4),
    # the decode shape with groups of 8 sequences sharing a 2048-token prefix (same physical
    # pages in their block tables), each with its own 512..2048-token continuation
    "shared_prefix_decode": Spec("shared_prefix_decode", 64, 32, 8, 128, "bf16", "bf16",
                                 ctx_range=(2560, 4096), q_len=1, tree="chain", seed=5,
                                 share_group=8, shared_prefix_pages=128),
}


@dataclass
class Workload:
    spec: Spec
    ctx_lens: np.ndarray            # int32 [B]
    q_lens: np.ndarray              # int32 [B]
    block_tables: np.ndarray        # int32 [B, MBS]
    num_blocks: int
    pages_used: np.ndarray          # int32 [B]  ceil(ctx/16)
    parents: np.ndarray             # int32 [B, Qmax], -1 root / padding
    tree_mask: np.ndarray           # uint8 [B, Qmax, Qmax]
    q: np.ndarray                   # [B, Qmax, Hq, D]  f32 or bf16 bits
    k_cache: np.ndarray             # [NB, Hkv, 16, D]  f32 / bf16 bits / fp8 codes
    v_cache: np.ndarray
    k_scale: Optional[np.ndarray]   # f32 [NB, Hkv] (fp8 only)
    v_scale: Optional[np.ndarray]
    scale: float
    pad_page: int                   # page id used for block-table padding
    contiguous_k: Optional[list] = field(default=None, repr=False)  # per seq [Hkv, C, D] float32
    contiguous_v: Optional[list] = field(default=None, repr=False)

    @property
    def max_q_len(self) -> int:
        return self.q.shape[1]

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def make(spec: Spec | str, *, seed: Optional[int] = None, poison: bool = False,
         keep_contiguous: bool = False, threads: int = 8, **overrides) -> Workload:
    """Build the workload for ``spec`` (a Spec or a CONFIGS key).

    poison=True fills every pool slot that no sequence owns (unassigned pages,
    tail slots past ctx_len, the block-table padding page) with NaN (fp8: code
    0x7F, also NaN) and padding Q rows with NaN, so that a kernel reading
    outside the valid region shows it in its output.
    """
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if overrides:
        spec = replace(spec, **overrides)
    if seed is not None:
        spec = replace(spec, seed=seed)
    B, Hq, Hkv, D = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    root = np.random.SeedSequence(spec.seed)
    s_ctx, s_pool, s_tree, s_q, s_kv = root.spawn(5)

    # 1. context lengths (they include the q_b candidates) and candidate counts
    rng = np.random.default_rng(s_ctx)
    Qmax = spec.q_len
    if spec.q_len_ragged:
        q_lens = rng.integers(1, Qmax + 1, size=B).astype(np.int32)
    else:
        q_lens = np.full(B, Qmax, dtype=np.int32)
    if spec.ctx_list is not None:
        if len(spec.ctx_list) != B:
            raise ValueError("ctx_list length must equal batch")
        ctx = np.asarray(spec.ctx_list, dtype=np.int32)
    else:
        lo, hi = spec.ctx_range
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    ctx = np.maximum(ctx, q_lens).astype(np.int32)
    share = spec.shared_prefix_pages > 0 and spec.share_group > 1
    SP = spec.shared_prefix_pages if share else 0
    if share:
        # the shared pages are whole pages of every member's committed prefix
        ctx = np.maximum(ctx, SP * PAGE + q_lens).astype(np.int32)
    group_of = np.arange(B) // max(1, spec.share_group)
    n_groups = int(group_of.max()) + 1 if B else 0

    # 2. pool and block tables: consecutive slices of one random permutation (with a shared
    #    prefix, each group's first pages come once, then every member's own pages)
    pages = ((ctx + PAGE - 1) // PAGE).astype(np.int32)
    used = int(pages.sum()) - (B - n_groups) * SP
    NB = spec.pool_pages if spec.pool_pages is not None else int(math.ceil(spec.pool_factor * used))
    if NB < used:
        raise ValueError("pool smaller than the pages in use")
    rng = np.random.default_rng(s_pool)
    perm = rng.permutation(NB).astype(np.int32)
    MBS = int(pages.max())
    pad_page = int(perm[used]) if NB > used else int(perm[0])
    tables = np.full((B, MBS), pad_page, dtype=np.int32)
    off = 0
    for b in range(B):
        if share and (b == 0 or group_of[b] != group_of[b - 1]):
            group_pages = perm[off:off + SP]
            off += SP
        if share:
            tables[b, :SP] = group_pages
        tables[b, SP:pages[b]] = perm[off:off + pages[b] - SP]
        off += pages[b] - SP

    # 3. candidate trees
    rng = np.random.default_rng(s_tree)
    parents = np.full((B, Qmax), -1, dtype=np.int32)
    mask = np.zeros((B, Qmax, Qmax), dtype=np.uint8)
    for b in range(B):
        par = sample_tree_parents(rng, int(q_lens[b]), spec.tree, spec.depth_cap)
        parents[b, :len(par)] = par
        mask[b] = tree_mask_from_parents(par, Qmax)

    # 4. Q  [B, Qmax, Hq, D]
    rng = np.random.default_rng(s_q)
    qf = rng.standard_normal((B, Qmax, Hq, D), dtype=np.float32)
    for b in range(B):
        qf[b, q_lens[b]:] = np.nan if poison else 0.0
    q = _storage(qf, spec.q_dtype)

    # 5. K and V, one stream per sequence, scattered into pool pages
    kv_dt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[spec.kv_dtype]
    fill = 0
    if poison:
        fill = {"f32": np.float32(np.nan).view(np.uint32), "bf16": 0x7FC0, "fp8": 0x7F}[spec.kv_dtype]
    k_cache = np.empty((NB, Hkv, PAGE, D), dtype=kv_dt)
    v_cache = np.empty((NB, Hkv, PAGE, D), dtype=kv_dt)
    if spec.kv_dtype == "f32":
        k_cache.view(np.uint32)[...] = fill
        v_cache.view(np.uint32)[...] = fill
    else:
        k_cache[...] = fill
        v_cache[...] = fill
    is_fp8 = spec.kv_dtype == "fp8"
    k_scale = np.ones((NB, Hkv), dtype=np.float32) if is_fp8 else None
    v_scale = np.ones((NB, Hkv), dtype=np.float32) if is_fp8 else None
    contig_k = [None] * B if keep_contiguous else None
    contig_v = [None] * B if keep_contiguous else None
    seq_streams = s_kv.spawn(B)
    group_streams = s_kv.spawn(n_groups) if share else None

    def fill_seq(b: int) -> None:
        g = np.random.default_rng(seq_streams[b])
        C, P = int(ctx[b]), int(pages[b])
        gp = np.random.default_rng(group_streams[group_of[b]]) if share else None
        for which, cache, scl in ((0, k_cache, k_scale), (1, v_cache, v_scale)):
            if share:
                # the group's prefix (the same draw for every member), then this sequence's own rows
                x = np.concatenate([gp.standard_normal((Hkv, SP * PAGE, D), dtype=np.float32),
                                    g.standard_normal((Hkv, C - SP * PAGE, D), dtype=np.float32)], axis=1)
            else:
                x = g.standard_normal((Hkv, C, D), dtype=np.float32)
            if spec.kv_dtype == "bf16":
                x = bf16_bits_to_f32(f32_to_bf16_bits(x))   # values the kernel sees
            if keep_contiguous:
                (contig_k if which == 0 else contig_v)[b] = x
            padded = np.zeros((Hkv, P * PAGE, D), dtype=np.float32)
            padded[:, :C] = x
            tiles = padded.reshape(Hkv, P, PAGE, D).transpose(1, 0, 2, 3)   # [P, Hkv, 16, D]
            phys = tables[b, :P]
            if is_fp8:
                amax = np.abs(tiles).max(axis=(2, 3))                       # [P, Hkv]
                s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
                codes = _fp8_codes(tiles / s[:, :, None, None])
                scl[phys] = s
                enc = codes
            elif spec.kv_dtype == "bf16":
                enc = f32_to_bf16_bits(tiles)
            else:
                enc = tiles
            tail = C - (P - 1) * PAGE
            if poison and tail < PAGE:
                enc = enc.copy()
                if spec.kv_dtype == "f32":
                    enc.view(np.uint32)[-1, :, tail:, :] = fill
                else:
                    enc[-1, :, tail:, :] = fill
            cache[phys] = enc

    with ThreadPoolExecutor(max_workers=max(1, min(threads, B))) as ex:
        list(ex.map(fill_seq, range(B)))

    return Workload(spec=spec, ctx_lens=ctx, q_lens=q_lens, block_tables=tables, num_blocks=NB,
                    pages_used=pages, parents=parents, tree_mask=mask, q=q, k_cache=k_cache,
                    v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, scale=spec.softmax_scale,
                    pad_page=pad_page, contiguous_k=contig_k, contiguous_v=contig_v)


def make_tokens(w: Workload, seed: int, p_match: float = 0.7, p_root: float = 1.0, vocab: int = 32000):
    """Synthetic token ids for an acceptance step: candidate ids cand [B, Qmax],
    the target model's predictions target [B, Qmax] and its prediction after the
    committed prefix target_prev [B] (all int32).  Each non-root candidate copies
    its parent's prediction with probability p_match, each root copies
    target_prev with probability p_root; everything else is a uniform draw."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xACC]))
    B, Qmax = w.parents.shape
    cand = rng.integers(0, vocab, (B, Qmax)).astype(np.int32)
    target = rng.integers(0, vocab, (B, Qmax)).astype(np.int32)
    tprev = rng.integers(0, vocab, B).astype(np.int32)
    u = rng.random((B, Qmax))
    for b in range(B):
        for i in range(int(w.q_lens[b])):
            p = int(w.parents[b, i])
            if p >= 0 and u[b, i] < p_match:
                cand[b, i] = target[b, p]
            elif p < 0 and u[b, i] < p_root:
                cand[b, i] = tprev[b]
    return cand, target, tprev


def permute_pool(w: Workload, seed: int) -> Workload:
    """Same logical workload with the physical pages relabelled by a random bijection."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(w.num_blocks).astype(np.int32)     # old page id -> new page id
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[sigma] = w.k_cache
    v[sigma] = w.v_cache
    ks = vs = None
    if w.k_scale is not None:
        ks = np.empty_like(w.k_scale)
        vs = np.empty_like(w.v_scale)
        ks[sigma] = w.k_scale
        vs[sigma] = w.v_scale
    return replace(w, block_tables=sigma[w.block_tables], k_cache=k, v_cache=v,
                   k_scale=ks, v_scale=vs, pad_page=int(sigma[w.pad_page]))
