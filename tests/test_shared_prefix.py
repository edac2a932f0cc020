"""Shared-prefix pages: block tables of several sequences alias the same physical pages
(the pages' prefix cache, "GPU/CPU 多级缓存" and the Prefix Cache memory management of the
618zxw.cn article).  Paging only reorganises the data, so aliasing must not change what the
definition computes; these pins check the generator's aliasing and the oracle against private
copies of the shared pages and against brute force on contiguous K/V."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import refs
from workload import Spec, make


def shared_spec(kv="bf16", q_len=1, tree="chain", seed=0, group=3, sp=2):
    return Spec("sp", 6, 8, 2, 32, "bf16", kv, ctx_range=(40, 90), q_len=q_len, tree=tree, seed=seed,
                share_group=group, shared_prefix_pages=sp)


def run_oracle(w, tables=None, k=None, v=None, ks=None, vs=None):
    return oracle.paged_tree_attn(w.q, w.k_cache if k is None else k, w.v_cache if v is None else v,
                                  w.block_tables if tables is None else tables, w.ctx_lens, w.q_lens,
                                  w.tree_mask, w.scale, q_dtype=w.spec.q_dtype, kv_dtype=w.spec.kv_dtype,
                                  k_scale=w.k_scale if ks is None else ks, v_scale=w.v_scale if vs is None else vs)


def private_copies(w):
    """The same workload with every member's shared pages copied to pages of its own."""
    s = w.spec
    SP, G = s.shared_prefix_pages, s.share_group
    B = w.q.shape[0]
    extra = [b for b in range(B) if b % G != 0]
    NB = w.num_blocks + len(extra) * SP
    k = np.concatenate([w.k_cache, np.zeros((NB - w.num_blocks,) + w.k_cache.shape[1:], w.k_cache.dtype)])
    v = np.concatenate([w.v_cache, np.zeros((NB - w.num_blocks,) + w.v_cache.shape[1:], w.v_cache.dtype)])
    ks = vs = None
    if w.k_scale is not None:
        ks = np.concatenate([w.k_scale, np.ones((NB - w.num_blocks, w.k_scale.shape[1]), np.float32)])
        vs = np.concatenate([w.v_scale, np.ones((NB - w.num_blocks, w.v_scale.shape[1]), np.float32)])
    tables = w.block_tables.copy()
    nxt = w.num_blocks
    for b in extra:
        for p in range(SP):
            src = int(w.block_tables[b, p])
            k[nxt], v[nxt] = w.k_cache[src], w.v_cache[src]
            if ks is not None:
                ks[nxt], vs[nxt] = w.k_scale[src], w.v_scale[src]
            tables[b, p] = nxt
            nxt += 1
    return tables, k, v, ks, vs


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_generator_aliases_only_the_shared_prefix(kv):
    w = make(shared_spec(kv=kv, seed=3), keep_contiguous=True)
    SP, G = 2, 3
    for g in range(2):
        tb = w.block_tables[G * g:G * g + G, :SP]
        assert (tb == tb[0]).all()
        for j in range(G):
            assert np.array_equal(w.contiguous_k[G * g + j][:, :SP * 16], w.contiguous_k[G * g][:, :SP * 16])
            assert np.array_equal(w.contiguous_v[G * g + j][:, :SP * 16], w.contiguous_v[G * g][:, :SP * 16])
    own = np.concatenate([w.block_tables[b, SP:w.pages_used[b]] for b in range(6)])
    shared = np.concatenate([w.block_tables[G * g, :SP] for g in range(2)])
    allp = np.concatenate([shared, own])
    assert len(np.unique(allp)) == len(allp)
    # the shared pages lie inside every member's committed prefix
    assert (w.ctx_lens - w.q_lens >= SP * 16).all()


@pytest.mark.parametrize("kv,q_len,tree", [("bf16", 1, "chain"), ("bf16", 5, "random"), ("fp8", 4, "chain")])
def test_aliasing_is_bit_identical_to_private_copies(kv, q_len, tree):
    w = make(shared_spec(kv=kv, q_len=q_len, tree=tree, seed=7))
    out, lse = run_oracle(w)
    t, k, v, ks, vs = private_copies(w)
    out2, lse2 = run_oracle(w, tables=t, k=k, v=v, ks=ks, vs=vs)
    assert np.array_equal(out, out2, equal_nan=True)
    assert np.array_equal(lse, lse2, equal_nan=True)


def test_shared_prefix_bruteforce():
    w = make(shared_spec(q_len=4, tree="random", seed=11), keep_contiguous=True)
    out, _ = run_oracle(w)
    ref = refs.workload_sdpa(w)
    v = ~np.isnan(ref)
    assert np.abs(out[v] - ref[v]).max() <= 1e-12
    assert np.isnan(out[~v]).all()


def test_shared_prefix_config_shape():
    from workload.gen import CONFIGS
    s = CONFIGS["shared_prefix_decode"]
    assert s.share_group == 8 and s.shared_prefix_pages * 16 == 2048 and s.batch % s.share_group == 0
