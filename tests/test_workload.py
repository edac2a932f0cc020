"""Checks of the seeded input generator (CPU)."""
from __future__ import annotations

import numpy as np

from workload import CONFIGS, Spec, make, permute_pool
from workload.gen import _depths, bf16_bits_to_f32


def test_deterministic():
    s = Spec("d", 3, 4, 2, 16, "bf16", "fp8", ctx_range=(5, 50), q_len=5, tree="random", seed=9)
    a, b = make(s), make(s)
    for f in ("ctx_lens", "q_lens", "block_tables", "tree_mask", "q", "k_cache", "v_cache", "k_scale"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_tree_invariants():
    s = Spec("t", 16, 2, 1, 8, "f32", "f32", ctx_range=(40, 60), q_len=16, tree="random", depth_cap=6, seed=1)
    w = make(s)
    for b in range(16):
        par = w.parents[b]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, 16))
        assert _depths(par).max() <= 6
        m = w.tree_mask[b]
        assert (np.diag(m) == 1).all()
        for i in range(16):
            # mask row = ancestor-or-self closure
            anc = set()
            j = i
            while j >= 0:
                anc.add(j)
                j = par[j]
            assert set(np.flatnonzero(m[i])) == anc


def test_chain_mask_is_lower_triangle():
    w = make(Spec("c", 2, 2, 1, 8, "f32", "f32", ctx_range=(10, 20), q_len=8, tree="chain"))
    assert np.array_equal(w.tree_mask[0], np.tril(np.ones((8, 8), np.uint8)))


def test_pool_is_bijection_and_tables_disjoint():
    w = make(Spec("p", 8, 2, 1, 8, "f32", "f32", ctx_range=(1, 100), q_len=1, seed=4))
    used = np.concatenate([w.block_tables[b, :w.pages_used[b]] for b in range(8)])
    assert len(set(used.tolist())) == len(used)
    assert w.num_blocks == int(np.ceil(1.2 * used.size))
    assert used.min() >= 0 and used.max() < w.num_blocks
    assert w.pad_page not in set(used.tolist())


def test_ctx_ranges_and_qlens():
    w = make(Spec("r", 64, 2, 1, 8, "f32", "f32", ctx_range=(30, 90), q_len=6, q_len_ragged=True, seed=2))
    assert w.ctx_lens.min() >= 30 and w.ctx_lens.max() <= 90
    assert w.q_lens.min() >= 1 and w.q_lens.max() <= 6


def test_fp8_scales_are_page_absmax_over_448():
    import torch
    w = make(Spec("f", 2, 2, 2, 16, "bf16", "fp8", ctx_range=(20, 40), q_len=2, seed=6))
    for b in range(2):
        for p in range(w.pages_used[b]):
            page = w.block_tables[b, p]
            vals = torch.from_numpy(w.k_cache[page]).view(torch.float8_e4m3fn).float().numpy()
            # the largest code in each (page, head) tile decodes to 448 (the scaled absmax)
            assert np.allclose(np.abs(vals).reshape(2, -1).max(axis=1), 448.0)
            assert (w.k_scale[page] > 0).all()


def test_bf16_values_are_rounded_normals():
    w = make(Spec("b", 2, 2, 2, 16, "bf16", "bf16", ctx_range=(20, 40), q_len=1, seed=7), keep_contiguous=True)
    x = w.contiguous_k[0]
    assert np.array_equal(bf16_bits_to_f32(w.k_cache[w.block_tables[0, 0], 0, :16]), x[0, :16])


def test_named_configs_shapes():
    w = make("tiny_decode")
    assert w.q.shape == (2, 1, 4, 64) and w.k_cache.shape == (16, 4, 16, 64)
    for name, s in CONFIGS.items():
        assert s.num_q_heads % s.num_kv_heads == 0, name


def test_permute_pool_relabels():
    w = make(Spec("pp", 2, 2, 1, 8, "f32", "f32", ctx_range=(20, 40), q_len=2, seed=8))
    w2 = permute_pool(w, 3)
    for b in range(2):
        for p in range(w.pages_used[b]):
            assert np.array_equal(w.k_cache[w.block_tables[b, p]], w2.k_cache[w2.block_tables[b, p]])
