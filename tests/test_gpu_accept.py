"""GPU parity of taco_accept_commit against the oracle: every output and every
cache byte must match exactly (integer decisions and row moves; fp8 rows
re-encoded between pages of different scales follow the same float32 steps)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workload import Spec, make
from workload.device import to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_speculative_verify_amd as psv
    psv.load()
    return torch


def tokens(w, seed, p_match=0.7, p_root=0.9):
    """Synthetic candidate / prediction ids: a node copies its parent's prediction
    with probability p_match, and the root matches the prefix prediction with
    probability p_root."""
    rng = np.random.default_rng(seed)
    B, Qmax = w.q.shape[0], w.q.shape[1]
    cand = rng.integers(0, 50, (B, Qmax)).astype(np.int32)
    target = rng.integers(0, 50, (B, Qmax)).astype(np.int32)
    tprev = rng.integers(0, 50, B).astype(np.int32)
    for b in range(B):
        q = int(w.q_lens[b])
        mask = w.tree_mask[b] if Qmax > 1 else np.ones((1, 1), np.uint8)
        par = oracle.tree_parents(mask, q)
        for i in range(q):
            if par[i] >= 0 and rng.random() < p_match:
                cand[b, i] = target[b, par[i]]
            if par[i] < 0 and rng.random() < p_root:
                cand[b, i] = tprev[b]
    return cand, target, tprev


def spec(name, B, Hq, Hkv, D, qd, kvd, ctx, q_len, tree="random", depth=None, ragged=False, seed=0):
    return Spec(name, B, Hq, Hkv, D, qd, kvd, ctx_range=ctx, q_len=q_len, q_len_ragged=ragged,
                tree=tree, depth_cap=depth, seed=seed)


CASES = [
    ("tree16_bf16", spec("a", 6, 16, 4, 128, "bf16", "bf16", (16, 700), 16, "random", 6, seed=1)),
    ("tree32_bf16_ragged", spec("a", 5, 16, 8, 128, "bf16", "bf16", (1, 900), 32, "random", ragged=True, seed=2)),
    ("chain8_fp8", spec("a", 7, 32, 8, 128, "bf16", "fp8", (8, 600), 8, "chain", seed=3)),
    ("tree12_fp8_d64", spec("a", 4, 8, 2, 64, "bf16", "fp8", (12, 300), 12, "random", seed=4)),
    ("forest_f32", spec("a", 3, 4, 2, 64, "f32", "f32", (10, 200), 10, "flat", seed=5)),
    ("tree64_bf16", spec("a", 2, 4, 4, 128, "bf16", "bf16", (64, 400), 64, "random", seed=6)),
    ("decode_bf16", spec("a", 9, 32, 8, 128, "bf16", "bf16", (1, 500), 1, "chain", seed=7)),
    ("verify70b_shape", spec("a", 32, 64, 8, 128, "bf16", "bf16", (1024, 2048), 16, "random", 6, seed=8)),
]


def _bits(t, kv_dtype):
    import torch
    view = {"bf16": torch.int16, "fp8": torch.uint8, "f32": torch.int32}[kv_dtype]
    return t.view(view).cpu().numpy()


@pytest.mark.parametrize("cid,sp", CASES, ids=[c[0] for c in CASES])
def test_accept_commit_parity(torch_cuda, cid, sp):
    import paged_speculative_verify_amd as psv
    torch = torch_cuda
    w = make(sp, poison=True)
    cand, target, tprev = tokens(w, 100 + sp.seed)
    say(cid, "B", w.q.shape[0], "q", sp.q_len, sp.kv_dtype)
    d = to_device(w)
    dev = d.q.device
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    n, path, bonus, new_ctx = psv.taco_accept_commit(T(cand), T(target), T(tprev), d.ctx_lens, d.q_lens,
                                                     d.tree_mask, d.block_tables, d.k_cache, d.v_cache,
                                                     k_scale=d.k_scale, v_scale=d.v_scale)
    torch.cuda.synchronize()
    r_n, r_path, r_bonus, r_ctx, r_k, r_v = oracle.accept_commit(
        w.ctx_lens, w.q_lens, w.tree_mask if w.q.shape[1] > 1 else None, cand, target, tprev, w.block_tables,
        w.k_cache, w.v_cache, kv_dtype=sp.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    assert np.array_equal(n.cpu().numpy(), r_n)
    assert np.array_equal(path.cpu().numpy(), r_path)
    assert np.array_equal(bonus.cpu().numpy(), r_bonus)
    assert np.array_equal(new_ctx.cpu().numpy(), r_ctx)
    view = {"bf16": np.int16, "fp8": np.uint8, "f32": np.int32}[sp.kv_dtype]
    assert np.array_equal(_bits(d.k_cache, sp.kv_dtype), np.ascontiguousarray(r_k).view(view))
    assert np.array_equal(_bits(d.v_cache, sp.kv_dtype), np.ascontiguousarray(r_v).view(view))
    say(cid, "accepted", r_n.tolist()[:8])


def test_accept_commit_then_attention_sees_committed_rows(torch_cuda):
    """After a commit, attention over the new context (one query per sequence
    at the last committed position) matches the oracle on the committed cache."""
    import paged_speculative_verify_amd as psv
    torch = torch_cuda
    sp = spec("c", 5, 16, 4, 128, "bf16", "bf16", (40, 900), 12, "random", seed=9)
    w = make(sp)
    cand, target, tprev = tokens(w, 7)
    d = to_device(w)
    dev = d.q.device
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    n, path, bonus, new_ctx = psv.taco_accept_commit(T(cand), T(target), T(tprev), d.ctx_lens, d.q_lens,
                                                     d.tree_mask, d.block_tables, d.k_cache, d.v_cache)
    _, _, _, r_ctx, r_k, r_v = oracle.accept_commit(w.ctx_lens, w.q_lens, w.tree_mask, cand, target, tprev,
                                                    w.block_tables, w.k_cache, w.v_cache, kv_dtype="bf16")
    q1 = d.q[:, :1].contiguous()
    ones = torch.ones(w.q.shape[0], dtype=torch.int32, device=dev)
    out = psv.taco_paged_tree_attn(q1, d.k_cache, d.v_cache, d.block_tables, new_ctx, ones, None, d.scale)
    torch.cuda.synchronize()
    B = w.q.shape[0]
    ref, _ = oracle.paged_tree_attn(np.ascontiguousarray(w.q[:, :1]), r_k, r_v, w.block_tables, r_ctx,
                                    np.ones(B, dtype=np.int32), np.ones((B, 1, 1), dtype=np.uint8), w.scale,
                                    q_dtype="bf16", kv_dtype="bf16")
    err = np.abs(out.to(torch.float64).cpu().numpy() - ref).max()
    assert err <= 1e-2, err
