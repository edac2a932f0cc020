"""Pins for the acceptance / commit oracle (CPU only).

The acceptance rule is checked against brute-force enumeration of every
root-to-node path on small trees, the parent recovery against the generator's
own parent arrays, and the commit against invariants of the cache contents.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
from oracle.accept import _fp8_move
from workload.gen import sample_tree_parents, tree_mask_from_parents

PAGE = 16


def brute_force_path(parents, cand, target, target_prev):
    """Enumerate every root-to-node path; keep those whose every token matches
    the prediction before it; return the longest (smallest last node on ties)."""
    q = len(parents)
    best = []
    for end in range(q):
        path = []
        i = end
        while i >= 0:
            path.append(i)
            i = int(parents[i])
        path.reverse()
        ok = cand[path[0]] == target_prev and all(cand[path[k]] == target[path[k - 1]]
                                                   for k in range(1, len(path)))
        if ok and len(path) > len(best):
            best = path
    bonus = target[best[-1]] if best else target_prev
    return best, bonus


def _all_parent_arrays(n):
    return itertools.product(*[range(-1, i) if i else [-1] for i in range(n)])


def test_tree_parents_recovers_generator_parents():
    rng = np.random.default_rng(0)
    for q in (1, 2, 7, 16, 32, 64):
        for kind in ("chain", "random", "flat"):
            par = sample_tree_parents(rng, q, kind, None)
            mask = tree_mask_from_parents(par, 64)
            assert np.array_equal(oracle.tree_parents(mask, q), par.astype(np.int64)), (q, kind)


def test_accept_path_equals_brute_force_small_trees():
    rng = np.random.default_rng(1)
    for q in range(1, 6):
        for par in _all_parent_arrays(q):
            par = np.array(par)
            for _ in range(6):
                cand = rng.integers(0, 3, q)
                target = rng.integers(0, 3, q)
                tp = int(rng.integers(0, 3))
                got = oracle.accept_path(par, cand, target, tp)
                want = brute_force_path(par, cand, target, tp)
                assert got[0] == want[0] and got[1] == want[1], (par, cand, target, tp)


def test_accept_path_special_cases():
    q = 8
    chain = np.arange(-1, q - 1)
    cand = np.arange(100, 100 + q)
    target = np.arange(101, 101 + q)            # every prediction is the next candidate
    path, bonus = oracle.accept_path(chain, cand, target, 100)
    assert path == list(range(q)) and bonus == 100 + q
    target2 = target.copy()
    target2[0] = 7                               # the root's child is rejected
    path, bonus = oracle.accept_path(chain, cand, target2, 100)
    assert path == [0] and bonus == 7
    path, bonus = oracle.accept_path(chain, cand, target, 5)   # root rejected
    assert path == [] and bonus == 5


def _commit_case(kv_dtype, seed):
    rng = np.random.default_rng(seed)
    B, Hkv, D, Qmax = 3, 2, 8, 6
    q_lens = np.array([6, 1, 4])
    L = np.array([21, 0, 16])
    ctx = L + q_lens
    nb = 12
    tables = np.array([rng.permutation(nb)[:4] for _ in range(B)], dtype=np.int32)
    masks = np.zeros((B, Qmax, Qmax), dtype=np.uint8)
    cand = rng.integers(0, 4, (B, Qmax)).astype(np.int32)
    target = rng.integers(0, 4, (B, Qmax)).astype(np.int32)
    for b in range(B):
        par = sample_tree_parents(rng, int(q_lens[b]), "random", None)
        masks[b] = tree_mask_from_parents(par, Qmax)
        # make acceptance likely: each child's token copies its parent's prediction
        for i in range(int(q_lens[b])):
            if par[i] >= 0 and rng.random() < 0.8:
                cand[b, i] = target[b, par[i]]
    tprev = cand[:, 0].copy()
    if kv_dtype == "fp8":
        k = rng.integers(0, 0x7F, (nb, Hkv, PAGE, D)).astype(np.uint8)
        v = rng.integers(0, 0x7F, (nb, Hkv, PAGE, D)).astype(np.uint8)
        ks = rng.choice([0.5, 0.75, 1.0], (nb, Hkv)).astype(np.float32)
        vs = rng.choice([0.5, 0.75, 1.0], (nb, Hkv)).astype(np.float32)
    else:
        k = rng.integers(0, 1 << 15, (nb, Hkv, PAGE, D)).astype(np.uint16)
        v = rng.integers(0, 1 << 15, (nb, Hkv, PAGE, D)).astype(np.uint16)
        ks = vs = None
    return dict(ctx=ctx, q=q_lens, L=L, tables=tables, masks=masks, cand=cand, target=target, tprev=tprev,
                k=k, v=v, ks=ks, vs=vs)


def _row(cache, tables, b, t):
    return cache[tables[b][t // PAGE], :, t % PAGE, :]


@pytest.mark.parametrize("seed", range(4))
def test_commit_moves_path_rows_bf16(seed):
    c = _commit_case("bf16", seed)
    n, paths, bonus, new_ctx, k2, v2 = oracle.accept_commit(
        c["ctx"], c["q"], c["masks"], c["cand"], c["target"], c["tprev"], c["tables"], c["k"], c["v"],
        kv_dtype="bf16")
    for b in range(3):
        L = int(c["L"][b])
        assert new_ctx[b] == L + n[b]
        for kk in range(int(n[b])):
            for old, new in ((c["k"], k2), (c["v"], v2)):
                assert np.array_equal(_row(new, c["tables"], b, L + kk), _row(old, c["tables"], b, L + paths[b, kk]))
        for t in list(range(L)) + list(range(L + int(n[b]), int(c["ctx"][b]))):
            for old, new in ((c["k"], k2), (c["v"], v2)):
                assert np.array_equal(_row(new, c["tables"], b, t), _row(old, c["tables"], b, t)), (b, t)
        assert (paths[b, int(n[b]):] == -1).all()


def test_fp8_move_rule():
    from oracle.formats import decode_fp8_e4m3fn
    import torch
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    assert np.array_equal(_fp8_move(codes, 0.75, 0.75), codes)
    got = _fp8_move(codes, 0.75, 0.5)
    x = (decode_fp8_e4m3fn(codes).astype(np.float32) * np.float32(0.75)) / np.float32(0.5)
    lib = torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, lib)


@pytest.mark.parametrize("seed", range(3))
def test_commit_fp8_rows(seed):
    c = _commit_case("fp8", seed)
    n, paths, bonus, new_ctx, k2, v2 = oracle.accept_commit(
        c["ctx"], c["q"], c["masks"], c["cand"], c["target"], c["tprev"], c["tables"], c["k"], c["v"],
        kv_dtype="fp8", k_scale=c["ks"], v_scale=c["vs"])
    from oracle.formats import decode_fp8_e4m3fn
    for b in range(3):
        L = int(c["L"][b])
        for kk in range(int(n[b])):
            src, dst = L + int(paths[b, kk]), L + kk
            for old, new, sc in ((c["k"], k2, c["ks"]), (c["v"], v2, c["vs"])):
                ps, pd = c["tables"][b][src // PAGE], c["tables"][b][dst // PAGE]
                a = decode_fp8_e4m3fn(old[ps, :, src % PAGE, :]) * sc[ps][:, None]
                z = decode_fp8_e4m3fn(new[pd, :, dst % PAGE, :]) * sc[pd][:, None]
                # re-encoding keeps the value to half an e4m3 step (relative 2^-4) of the destination scale
                assert np.all(np.abs(z - a) <= np.abs(a) * 2.0 ** -4 + sc[pd][:, None] * 2.0 ** -10)
