"""One whole verify step on the GPU, every piece through the C ABI, checked against the oracle:
the lookahead cache proposes each sequence's candidate tree from synthetic token streams, its
tree mask drives the fused KV append + paged tree attention call, and taco_accept_commit keeps
the candidates that match the streams' true continuation and compacts their K/V rows."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workload import Spec, make
from workload.device import out_to_f64, to_device
from workload.gen import f32_to_bf16_bits
from workload.tokens import synthetic_streams

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kv,seed", [("bf16", 301), ("fp8", 302)])
def test_verify_step_end_to_end(kv, seed):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_speculative_verify_amd as psv
    Qmax, H = 8, 240
    # pages for contexts with room for 8 candidates; the step's q_b comes from the cache
    w = make(Spec("step", 6, 16, 4, 128, "bf16", kv, ctx_range=(40, 900), q_len=Qmax, tree="chain", seed=seed))
    B, _, Hq, D = w.q.shape
    Hkv = w.k_cache.shape[1]
    L = (w.ctx_lens - w.q_lens).astype(np.int32)

    streams = synthetic_streams(B, H + Qmax + 1, vocab=60, seed=seed)
    cache = psv.LookaheadCache(12, 6, threads=3 if kv == "fp8" else 1)   # the threaded cache on one case
    cache.append_batch(range(B), [s[:H] for s in streams])
    tok, par, cnt = cache.propose(range(B), [Qmax] * B, Qmax)
    for b in range(B):                        # nothing matched: a single guess, as plain decode would verify
        if cnt[b] == 0:
            tok[b, 0], par[b, 0], cnt[b] = 0, -1, 1
    mask = psv.taco_la_tree_mask(par, cnt)
    # the step's shapes: q_b candidates after the committed L_b tokens
    w.q_lens = cnt.astype(np.int32)
    w.ctx_lens = (L + cnt).astype(np.int32)
    w.tree_mask = mask
    truth = np.array([s[H:H + Qmax + 1] for s in streams], np.int32)
    depth = np.zeros((B, Qmax), np.int32)
    for b in range(B):
        for i in range(int(cnt[b])):
            depth[b, i] = 1 if par[b, i] < 0 else depth[b, par[b, i]] + 1
    cand = np.where(tok >= 0, tok, 0).astype(np.int32)
    target = np.take_along_axis(truth, depth, axis=1).astype(np.int32)     # true token after node i's path
    tprev = truth[:, 0].copy()
    say("step", kv, "candidates", list(cnt))

    # the oracle's step: append, attention over the updated cache, acceptance and commit
    rng = np.random.default_rng(seed + 7)
    xk = rng.standard_normal((B, Qmax, Hkv, D)).astype(np.float32)
    xv = rng.standard_normal((B, Qmax, Hkv, D)).astype(np.float32)
    new_dt = "bf16"
    pos = [(b, j) for b in range(B) for j in range(int(cnt[b]))]
    slots = np.array([int(w.block_tables[b, (L[b] + j) // 16]) * 16 + (L[b] + j) % 16 for b, j in pos], np.int64)
    ref_k, ref_v = oracle.kv_append(w.k_cache, w.v_cache, f32_to_bf16_bits(np.stack([xk[b, j] for b, j in pos])),
                                    f32_to_bf16_bits(np.stack([xv[b, j] for b, j in pos])), slots,
                                    cache_dtype=kv, new_dtype=new_dt, k_scale=w.k_scale, v_scale=w.v_scale)
    ref, _ = oracle.paged_tree_attn(w.q, ref_k, ref_v, w.block_tables, w.ctx_lens, w.q_lens, w.tree_mask, w.scale,
                                    q_dtype="bf16", kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale)
    n_acc, path, bonus, new_ctx, k2, v2 = oracle.accept_commit(
        w.ctx_lens, w.q_lens, w.tree_mask, cand, target, tprev, w.block_tables, ref_k, ref_v, kv_dtype=kv,
        k_scale=w.k_scale, v_scale=w.v_scale)

    # the same step on the GPU
    d = to_device(w)
    kn = torch.from_numpy(f32_to_bf16_bits(xk)).cuda().view(torch.bfloat16)
    vn = torch.from_numpy(f32_to_bf16_bits(xv)).cuda().view(torch.bfloat16)
    out = torch.full_like(d.q, float("nan"))
    psv.taco_paged_tree_attn_append(d.q, kn, vn, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                    d.tree_mask, d.scale, out=out, k_scale=d.k_scale, v_scale=d.v_scale,
                                    max_ctx_len=d.max_ctx_len)
    g = psv.taco_accept_commit(torch.from_numpy(cand).cuda(), torch.from_numpy(target).cuda(),
                               torch.from_numpy(tprev).cuda(), d.ctx_lens, d.q_lens, d.tree_mask, d.block_tables,
                               d.k_cache, d.v_cache, k_scale=d.k_scale, v_scale=d.v_scale)
    torch.cuda.synchronize()
    o = out_to_f64(out)
    valid = ~np.isnan(ref)
    err = np.abs(o[valid] - ref[valid]).max()
    assert err <= (3e-2 if kv == "fp8" else 1e-2), err
    assert np.array_equal(g[0].cpu().numpy(), n_acc) and np.array_equal(g[1].cpu().numpy(), path)
    assert np.array_equal(g[2].cpu().numpy(), bonus) and np.array_equal(g[3].cpu().numpy(), new_ctx)
    assert np.array_equal(d.k_cache.view(torch.uint8).cpu().numpy().reshape(-1), k2.view(np.uint8).reshape(-1))
    assert np.array_equal(d.v_cache.view(torch.uint8).cpu().numpy().reshape(-1), v2.view(np.uint8).reshape(-1))
    # acceptance is the longest prefix of the true continuation spelled by a path of the tree
    for b in range(B):
        best = 0
        for i in range(int(cnt[b])):
            j, ok = i, True
            while j >= 0:
                ok &= cand[b, j] == truth[b, depth[b, j] - 1]
                j = par[b, j]
            if ok:
                best = max(best, int(depth[b, i]))
        assert n_acc[b] == best
    say("step", kv, "max abs err", err, "accepted", list(n_acc))
