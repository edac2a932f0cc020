"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max |out - oracle| over valid rows): 1e-5 for fp32 inputs, 1e-2
for bf16, 3e-2 for fp8 KV; LSE is checked to 1e-4 / 2e-2 / 4e-2.  Indexing
and masking are checked bit-exactly with probes whose exact answer is a
stored integer, and by bit-identity under a relabelling of physical pages.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

import oracle
from workload import Spec, make, permute_pool
from workload.device import out_to_f64, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}
LSE_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 4e-2}


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


def tol_key(spec):
    return "fp8" if spec.kv_dtype == "fp8" else spec.q_dtype


def run_gpu(torch, w, split=None, path="auto", want_lse=True, mode=None, workspace=None, shared_pages=None):
    """mode: "whole", "split" (split-K with `split` tokens) or "balanced"; by default
    "split" when split is given, else "whole".  shared_pages (the cache hint): by default set
    exactly when the workload's block tables alias a shared prefix."""
    import paged_speculative_verify_amd as psv
    d = to_device(w)
    out = torch.full_like(d.q, float("nan"))
    B, Qmax, Hq, D = w.q.shape
    lse = torch.full((B, Hq, Qmax), float("nan"), dtype=torch.float32, device=d.q.device) if want_lse else None
    mode = mode or ("whole" if split is None else "split")
    if shared_pages is None:
        shared_pages = w.spec.shared_prefix_pages > 0 and w.spec.share_group > 1
    hint = dict(shared_pages=bool(shared_pages))
    if mode == "shared":
        sg = w.spec.share_group
        leader = torch.from_numpy(np.array([(b // sg) * sg for b in range(B)], dtype=np.int32)).to(d.q.device)
        psv.taco_paged_tree_attn_shared_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                               d.tree_mask, leader, sg, split, d.scale, out=out, lse=lse,
                                               k_scale=d.k_scale, v_scale=d.v_scale, max_ctx_len=d.max_ctx_len,
                                               path=path, **hint)
    elif mode == "balanced":
        psv.taco_paged_tree_attn_balanced(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                          d.q_lens, d.tree_mask, d.scale, out=out, lse=lse,
                                          k_scale=d.k_scale, v_scale=d.v_scale, workspace=workspace,
                                          max_ctx_len=d.max_ctx_len, path=path, **hint)
    elif mode == "whole":
        psv.taco_paged_tree_attn(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                 d.tree_mask, d.scale, out=out, lse=lse, k_scale=d.k_scale,
                                 v_scale=d.v_scale, max_ctx_len=d.max_ctx_len, path=path, **hint)
    else:
        psv.taco_paged_tree_attn_splitk(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                        d.q_lens, d.tree_mask, d.scale, split, out=out, lse=lse,
                                        k_scale=d.k_scale, v_scale=d.v_scale,
                                        max_ctx_len=d.max_ctx_len, path=path, **hint)
    torch.cuda.synchronize()
    return out_to_f64(out), (lse.cpu().numpy().astype(np.float64) if want_lse else None)


def run_oracle(w, rows=None):
    s = w.spec
    sel = slice(None) if rows is None else rows
    return oracle.paged_tree_attn(w.q[sel], w.k_cache, w.v_cache, w.block_tables[sel], w.ctx_lens[sel],
                                  w.q_lens[sel], w.tree_mask[sel], w.scale, q_dtype=s.q_dtype,
                                  kv_dtype=s.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)


def assert_parity(w, out, lse, ref, ref_lse, seqs=None):
    key = tol_key(w.spec)
    if seqs is not None:
        out, lse = out[seqs], (lse[seqs] if lse is not None else None)
    valid = ~np.isnan(ref)
    # rows past q_len are untouched (still NaN), valid rows are finite
    assert np.isnan(out[~valid]).all(), "padding rows were written"
    assert np.isfinite(out[valid]).all(), "non-finite output in a valid row"
    err = np.abs(out[valid] - ref[valid]).max()
    assert err <= TOL[key], f"max abs err {err} > {TOL[key]}"
    if lse is not None:
        lv = ~np.isnan(ref_lse)
        assert np.isnan(lse[~lv]).all()
        lerr = np.abs(lse[lv] - ref_lse[lv]).max()
        assert lerr <= LSE_TOL[key], f"lse err {lerr}"
    return err


def spec(name, B, Hq, Hkv, D, qd, kvd, ctx, q_len, tree="random", depth=None, ragged=False, seed=0,
         **kw):
    return Spec(name, B, Hq, Hkv, D, qd, kvd, ctx_range=ctx, q_len=q_len, q_len_ragged=ragged,
                tree=tree, depth_cap=depth, seed=seed, **kw)


# -------------------------------------------------------------- small cases
CASES = [
    # (id, spec, split, path)
    ("tiny_decode_f32", "tiny_decode", None, "auto"),
    ("tiny_decode_f32_split32", "tiny_decode", 32, "auto"),
    ("decode_bf16_valu", spec("d", 6, 32, 8, 128, "bf16", "bf16", (1, 700), 1, "chain", seed=1), None, "valu"),
    ("decode_bf16_mfma", spec("d", 6, 32, 8, 128, "bf16", "bf16", (1, 700), 1, "chain", seed=1), None, "mfma"),
    ("decode_bf16_d64_valu", spec("d", 5, 8, 2, 64, "bf16", "bf16", (3, 300), 1, "chain", seed=2), None, "valu"),
    ("decode_bf16_split_valu", spec("d", 6, 32, 8, 128, "bf16", "bf16", (100, 3000), 1, "chain", seed=3), 256, "valu"),
    ("decode_f32_d128_mr8", spec("d", 3, 8, 1, 128, "f32", "f32", (20, 400), 1, "chain", seed=4), None, "valu"),
    ("small_tree_valu_mr8", spec("t", 4, 4, 2, 128, "bf16", "bf16", (8, 200), 4, "random", seed=5), None, "valu"),
    ("small_tree_mfma", spec("t", 4, 4, 2, 128, "bf16", "bf16", (8, 200), 4, "random", seed=5), None, "mfma"),
    ("verify_tree16_g8", spec("v", 4, 64, 8, 128, "bf16", "bf16", (16, 900), 16, "random", 6, seed=6), None, "auto"),
    ("verify_tree16_g8_split", spec("v", 4, 64, 8, 128, "bf16", "bf16", (16, 900), 16, "random", 6, seed=6), 128, "auto"),
    ("verify_tree32_g8_split", spec("l", 2, 64, 8, 128, "bf16", "bf16", (300, 3000), 32, "random", 8, seed=7), 2048, "auto"),
    ("verify_tree32_split64", spec("l", 2, 64, 8, 128, "bf16", "bf16", (33, 700), 32, "random", 8, seed=8), 64, "auto"),
    ("ragged_tree_mfma", spec("r", 7, 16, 2, 128, "bf16", "bf16", (1, 500), 12, "random", ragged=True, seed=9), None, "auto"),
    ("ragged_tree_d64", spec("r", 5, 16, 4, 64, "bf16", "bf16", (1, 300), 20, "random", ragged=True, seed=10), None, "auto"),
    ("fp8_chain8_mfma", spec("f", 6, 32, 8, 128, "bf16", "fp8", (8, 1500), 8, "chain", seed=11), None, "auto"),
    ("fp8_chain8_split", spec("f", 6, 32, 8, 128, "bf16", "fp8", (8, 1500), 8, "chain", seed=11), 512, "auto"),
    ("fp8_decode_valu", spec("f", 6, 32, 8, 128, "bf16", "fp8", (1, 900), 1, "chain", seed=12), None, "valu"),
    ("fp8_d64_tree", spec("f", 4, 16, 2, 64, "bf16", "fp8", (5, 400), 6, "random", seed=13), None, "auto"),
    ("gqa1_tree64", spec("w", 2, 4, 4, 128, "bf16", "bf16", (64, 400), 64, "random", seed=14), None, "mfma"),
    ("flat_forest", spec("ff", 3, 16, 2, 128, "bf16", "bf16", (10, 200), 10, "flat", seed=15), None, "auto"),
    # whole ranges of more than 256 pages: the block-table ring is refilled in the loop
    ("long_tree32_whole", spec("lw", 2, 64, 8, 128, "bf16", "bf16", (5000, 9000), 32, "random", 8, seed=16), None, "auto"),
    ("long_tree16_split8192", spec("lw", 3, 64, 8, 128, "bf16", "bf16", (9000, 12000), 16, "random", 6, seed=17), 8192, "auto"),
    # the shared-tile family forced for small row counts
    ("decode_bf16_tile", spec("d", 6, 32, 8, 128, "bf16", "bf16", (1, 700), 1, "chain", seed=1), None, "tile"),
    ("decode_bf16_tile_split", spec("d", 6, 32, 8, 128, "bf16", "bf16", (100, 3000), 1, "chain", seed=3), 256, "tile"),
    ("decode_d64_tile", spec("d", 5, 8, 2, 64, "bf16", "bf16", (3, 300), 1, "chain", seed=2), None, "tile"),
    ("fp8_chain8_tile", spec("f", 6, 32, 8, 128, "bf16", "fp8", (8, 1500), 8, "chain", seed=11), None, "tile"),
]


@pytest.mark.parametrize("cid,sp,split,path", CASES, ids=[c[0] for c in CASES])
def test_parity_small(torch_cuda, cid, sp, split, path):
    w = make(sp, poison=True)
    say(cid, "B", w.q.shape[0], "ctx", w.ctx_lens.tolist()[:8], "split", split, "path", path)
    out, lse = run_gpu(torch_cuda, w, split=split, path=path)
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)


def test_split_matches_unsplit(torch_cuda):
    w = make(spec("s", 3, 64, 8, 128, "bf16", "bf16", (200, 2500), 16, "random", 6, seed=21))
    say("split_vs_unsplit")
    a, _ = run_gpu(torch_cuda, w)
    b, _ = run_gpu(torch_cuda, w, split=256)
    v = ~np.isnan(a)
    assert np.abs(a[v] - b[v]).max() <= 1e-2


def test_permutation_and_repeat_bit_identical(torch_cuda):
    for sp, path in ((spec("p", 4, 32, 8, 128, "bf16", "bf16", (30, 800), 1, "chain", seed=31), "valu"),
                     (spec("p", 4, 64, 8, 128, "bf16", "bf16", (30, 800), 16, "random", 6, seed=32), "mfma"),
                     (spec("p", 4, 32, 8, 128, "bf16", "fp8", (30, 800), 8, "chain", seed=33), "mfma")):
        w = make(sp)
        say("permutation", sp.kv_dtype, path)
        a, la = run_gpu(torch_cuda, w, path=path)
        a2, la2 = run_gpu(torch_cuda, w, path=path)
        b, lb = run_gpu(torch_cuda, permute_pool(w, 5), path=path)
        assert np.array_equal(a, a2, equal_nan=True) and np.array_equal(la, la2, equal_nan=True)
        assert np.array_equal(a, b, equal_nan=True) and np.array_equal(la, lb, equal_nan=True)


def _probe_workload(sp, seed=3):
    """One-hot probe: per (seq, head, candidate) one visible key dominates by a score gap of
    >= 1000; V channel 0/1 hold (position mod 256, head + 3*seq) so the output names the
    exact logical position and head that were read."""
    from tests.test_oracle_pins import enc
    from tests import refs
    rng = np.random.default_rng(seed)
    w = make(sp)
    kv, qd = sp.kv_dtype, sp.q_dtype
    B, Qmax, Hq, D = w.q.shape
    Hkv = w.k_cache.shape[1]
    G = Hq // Hkv
    wrap = 16 if kv == "fp8" else 256
    if w.k_scale is not None:
        w.k_scale[...] = 1.0
        w.v_scale[...] = 1.0
    w.q[...] = 0
    w.k_cache[...] = 0
    w.v_cache[...] = 0
    want = np.full((B, Qmax, Hq, 2), np.nan)
    one = enc(1.0, kv)
    for b in range(B):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        vis = refs.vis_from_parents(C, Qb, w.parents[b])
        for t in range(C):
            page, slot = w.block_tables[b, t // 16], t % 16
            for hk in range(Hkv):
                w.v_cache[page, hk, slot, 0] = enc(t % wrap, kv)
                w.v_cache[page, hk, slot, 1] = enc((hk + 3 * b) % wrap, kv)
        for h in range(Hq):
            hk = h // G
            for i in range(Qb):
                t = int(rng.choice(np.flatnonzero(vis[i])))
                page, slot = w.block_tables[b, t // 16], t % 16
                ch = 2 + (h % G) * Qmax + i
                w.k_cache[page, hk, slot, ch] = one
                w.q[b, i, h, ch] = enc(2.0 ** math.ceil(math.log2(1000.0 / w.scale)), qd)
                want[b, i, h] = (t % wrap, (hk + 3 * b) % wrap)
    return w, want


@pytest.mark.parametrize("cid,sp,path", [
    ("probe_decode_valu", spec("o", 3, 8, 4, 64, "bf16", "bf16", (5, 300), 1, "chain", seed=41), "valu"),
    ("probe_tree_mfma", spec("o", 3, 4, 1, 128, "bf16", "bf16", (12, 300), 12, "random", seed=42), "mfma"),
    ("probe_tree_valu", spec("o", 3, 2, 1, 64, "bf16", "bf16", (12, 300), 4, "random", seed=43), "valu"),
    ("probe_fp8_mfma", spec("o", 2, 4, 1, 128, "bf16", "fp8", (8, 200), 8, "chain", seed=44), "mfma"),
    ("probe_f32", spec("o", 2, 2, 2, 64, "f32", "f32", (5, 200), 3, "random", seed=45), "valu"),
])
def test_one_hot_indexing_bit_exact(torch_cuda, cid, sp, path):
    w, want = _probe_workload(sp)
    say(cid)
    for split in (None, 32):
        out, _ = run_gpu(torch_cuda, w, split=split, path=path, want_lse=False)
        v = ~np.isnan(want[..., 0])
        assert np.array_equal(out[..., :2][v], want[v]), (cid, split)


@pytest.mark.parametrize("cid,sp,path", [
    # 96 rows per KV head (G 8 x 12 candidates): the balanced shared-tile grid, 32x32x16 kernel
    ("probe_bal_wide", spec("o", 3, 8, 1, 128, "bf16", "bf16", (12, 700), 12, "random", seed=46), "auto"),
    ("probe_bal_wide_d64_rows64", spec("o", 3, 8, 1, 64, "bf16", "bf16", (8, 500), 6, "random", seed=47), "auto"),
    ("probe_bal_tile16", spec("o", 3, 8, 1, 128, "bf16", "bf16", (12, 700), 12, "random", seed=48), "tile16"),
], ids=["probe_bal_wide", "probe_bal_wide_d64_rows64", "probe_bal_tile16"])
def test_one_hot_indexing_bit_exact_balanced(torch_cuda, cid, sp, path):
    """The balanced entry's slices, page walk and slice merge read exactly the intended
    (page, slot, head): every output equals its one dominant V row bit for bit."""
    w, want = _probe_workload(sp)
    say(cid)
    out, _ = run_gpu(torch_cuda, w, mode="balanced", path=path, want_lse=False)
    v = ~np.isnan(want[..., 0])
    assert np.array_equal(out[..., :2][v], want[v]), cid


@pytest.mark.parametrize("path,D", [("auto", 64), ("auto", 128), ("tile16", 128)])
def test_mask_bit_exact_balanced(torch_cuda, path, D):
    """The mask probe through the balanced shared-tile grid (256 rows per KV head)."""
    from tests.test_oracle_pins import enc
    w = make(spec("mb", 3, 16, 1, D, "bf16", "bf16", (20, 400), 16, "random", 5, seed=52))
    say("mask probe balanced", path, D)
    w.k_cache[...] = 0
    w.v_cache[...] = 0
    for b in range(3):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        for j in range(Qb):
            t = C - Qb + j
            w.v_cache[w.block_tables[b, t // 16], :, t % 16, j] = enc(1.0, "bf16")
    out, _ = run_gpu(torch_cuda, w, mode="balanced", path=path, want_lse=False)
    for b in range(3):
        Qb = int(w.q_lens[b])
        got = out[b, :Qb, :, :Qb] > 0
        want = (w.tree_mask[b, :Qb, :Qb] != 0)[:, None, :].repeat(out.shape[2], axis=1)
        assert np.array_equal(got, want)
        assert (out[b, :Qb, :, Qb:] == 0).all()


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_mask_bit_exact(torch_cuda, path):
    """K = 0, prefix V = 0, candidate j's V = e_j: out_i[j] > 0 exactly where the mask is set."""
    from tests.test_oracle_pins import enc
    Hq = 16 if path == "mfma" else 2
    q_len = 16 if path == "mfma" else 4
    w = make(spec("m", 3, Hq, 2 if path == "valu" else 1, 64, "bf16", "bf16", (20, 200), q_len, "random",
                  5, seed=51))
    say("mask probe", path)
    w.k_cache[...] = 0
    w.v_cache[...] = 0
    for b in range(3):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        for j in range(Qb):
            t = C - Qb + j
            w.v_cache[w.block_tables[b, t // 16], :, t % 16, j] = enc(1.0, "bf16")
    out, _ = run_gpu(torch_cuda, w, path=path, want_lse=False)
    for b in range(3):
        Qb = int(w.q_lens[b])
        got = out[b, :Qb, :, :Qb] > 0
        want = (w.tree_mask[b, :Qb, :Qb] != 0)[:, None, :].repeat(out.shape[2], axis=1)
        assert np.array_equal(got, want)
        assert (out[b, :Qb, :, Qb:] == 0).all()


def test_kv_append_parity(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    from workload.gen import f32_to_bf16_bits
    for kv, new_dt in (("bf16", "bf16"), ("f32", "f32"), ("fp8", "bf16"), ("fp8", "f32")):
        w = make(spec("a", 5, 8, 4, 128, "bf16" if kv != "f32" else "f32", kv, (10, 300), 6, "chain", seed=61))
        say("kv_append", kv, new_dt)
        rng = np.random.default_rng(62)
        pos = [(b, int(w.ctx_lens[b]) - int(w.q_lens[b]) + j) for b in range(5) for j in range(int(w.q_lens[b]))]
        slots = np.array([w.block_tables[b, t // 16] * 16 + t % 16 for b, t in pos] + [-1, -7], np.int64)
        x = (rng.standard_normal((len(slots), 4, 128)) * 3).astype(np.float32)
        x[0, 0, :4] = [1e6, -1e6, 0.0, -0.0]
        new = x if new_dt == "f32" else f32_to_bf16_bits(x)
        ref_k, ref_v = oracle.kv_append(w.k_cache, w.v_cache, new, new[:, ::-1].copy(), slots,
                                        cache_dtype=kv, new_dtype=new_dt, k_scale=w.k_scale, v_scale=w.v_scale)
        d = to_device(w)
        nv = torch.bfloat16 if new_dt == "bf16" else None
        kn = torch.from_numpy(new).cuda()
        vn = torch.from_numpy(new[:, ::-1].copy()).cuda()
        if nv is not None:
            kn, vn = kn.view(nv), vn.view(nv)
        psv.taco_kv_append(kn, vn, torch.from_numpy(slots).cuda(), d.k_cache, d.v_cache,
                           k_scale=d.k_scale, v_scale=d.v_scale)
        torch.cuda.synchronize()
        gk = d.k_cache.view(torch.uint8).cpu().numpy().view(ref_k.dtype).reshape(ref_k.shape)
        gv = d.v_cache.view(torch.uint8).cpu().numpy().view(ref_v.dtype).reshape(ref_v.shape)
        assert np.array_equal(gk.view(np.uint8), ref_k.view(np.uint8))
        assert np.array_equal(gv.view(np.uint8), ref_v.view(np.uint8))


# taco_paged_tree_attn_append: the candidates' K/V rows written by the attention launch itself.
FUSED_CASES = [
    ("decode_bf16", spec("fa", 6, 32, 8, 128, "bf16", "bf16", (1, 700), 1, "chain", seed=191), "bf16"),
    ("tree4_bf16", spec("fa", 5, 16, 4, 128, "bf16", "bf16", (4, 500), 4, "random", seed=192), "bf16"),
    ("ragged_tree8_d64", spec("fa", 5, 16, 4, 64, "bf16", "bf16", (8, 300), 8, "random", ragged=True,
                              seed=193), "bf16"),
    ("fp8_chain8_f32_rows", spec("fa", 6, 32, 8, 128, "bf16", "fp8", (8, 900), 8, "chain", seed=194), "f32"),
    ("fp8_decode_bf16_rows", spec("fa", 6, 32, 8, 128, "bf16", "fp8", (1, 900), 1, "chain", seed=195), "bf16"),
    # candidates straddling a 32-token page pair: two waves each write and read their own part
    ("cross_pairs_q8", spec("fa", 24, 16, 4, 128, "bf16", "bf16", (8, 200), 8, "random", seed=197), "bf16"),
    ("fp8_cross_pairs_q8", spec("fa", 24, 16, 4, 128, "bf16", "fp8", (8, 200), 8, "chain", seed=198), "f32"),
]


def check_fused_append(cid, sp, new_dt, call):
    """Poisoned workload whose candidates' slots still hold the old rows; call(d, k_new, v_new,
    out, lse) must write the new rows into the cache (byte-exact against the oracle's append) and
    attend over them (parity against the oracle over the appended cache)."""
    import torch
    from workload.gen import f32_to_bf16_bits
    w = make(sp, poison=True)
    B, Qmax, Hq, D = w.q.shape
    Hkv = w.k_cache.shape[1]
    kv = sp.kv_dtype
    if "cross_pairs" in cid:
        first, last = w.ctx_lens - w.q_lens, w.ctx_lens - 1
        assert (first // 32 != last // 32).any()
    rng = np.random.default_rng(sp.seed + 1)
    # new keys twice the spread of the cache's, so the candidates carry weight; new values as the
    # cache's, so outputs stay in the range the bf16 tolerance is set for
    xk = (rng.standard_normal((B, Qmax, Hkv, D)) * 2).astype(np.float32)
    xv = rng.standard_normal((B, Qmax, Hkv, D)).astype(np.float32)
    enc = (lambda x: x) if new_dt == "f32" else f32_to_bf16_bits
    pos = [(b, j) for b in range(B) for j in range(int(w.q_lens[b]))]
    slots = np.array([int(w.block_tables[b, (int(w.ctx_lens[b]) - int(w.q_lens[b]) + j) // 16]) * 16
                      + (int(w.ctx_lens[b]) - int(w.q_lens[b]) + j) % 16 for b, j in pos], np.int64)
    rows_k = enc(np.stack([xk[b, j] for b, j in pos]))
    rows_v = enc(np.stack([xv[b, j] for b, j in pos]))
    ref_k, ref_v = oracle.kv_append(w.k_cache, w.v_cache, rows_k, rows_v, slots, cache_dtype=kv,
                                    new_dtype=new_dt, k_scale=w.k_scale, v_scale=w.v_scale)
    ref, ref_lse = oracle.paged_tree_attn(w.q, ref_k, ref_v, w.block_tables, w.ctx_lens, w.q_lens, w.tree_mask,
                                          w.scale, q_dtype=sp.q_dtype, kv_dtype=kv, k_scale=w.k_scale,
                                          v_scale=w.v_scale)
    # the case can see a stale read: attention over the old rows misses every sequence's result
    stale, _ = oracle.paged_tree_attn(w.q, w.k_cache, w.v_cache, w.block_tables, w.ctx_lens, w.q_lens,
                                      w.tree_mask, w.scale, q_dtype=sp.q_dtype, kv_dtype=kv, k_scale=w.k_scale,
                                      v_scale=w.v_scale)
    assert all(np.nanmax(np.abs(ref[b] - stale[b])) > TOL[tol_key(sp)] for b in range(B))
    say(cid, "B", B, "q", sp.q_len, "kv", kv, "new rows", new_dt)
    d = to_device(w)                                  # the candidates' slots still hold the old rows
    kn = torch.from_numpy(np.ascontiguousarray(enc(xk))).cuda()
    vn = torch.from_numpy(np.ascontiguousarray(enc(xv))).cuda()
    if new_dt == "bf16":
        kn, vn = kn.view(torch.bfloat16), vn.view(torch.bfloat16)
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full((B, Hq, Qmax), float("nan"), dtype=torch.float32, device=d.q.device)
    call(d, kn, vn, out, lse)
    torch.cuda.synchronize()
    gk = d.k_cache.view(torch.uint8).cpu().numpy()
    gv = d.v_cache.view(torch.uint8).cpu().numpy()
    assert np.array_equal(gk.reshape(-1), ref_k.view(np.uint8).reshape(-1)), "K cache after the call"
    assert np.array_equal(gv.reshape(-1), ref_v.view(np.uint8).reshape(-1)), "V cache after the call"
    err = assert_parity(w, out_to_f64(out), lse.cpu().numpy().astype(np.float64), ref, ref_lse)
    say(cid, "max abs err", err)
    return w


@pytest.mark.parametrize("cid,sp,new_dt", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_append_parity(torch_cuda, cid, sp, new_dt):
    import paged_speculative_verify_amd as psv

    def call(d, kn, vn, out, lse):
        psv.taco_paged_tree_attn_append(d.q, kn, vn, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                        d.tree_mask, d.scale, out=out, lse=lse, k_scale=d.k_scale,
                                        v_scale=d.v_scale, max_ctx_len=d.max_ctx_len)
    check_fused_append(cid, sp, new_dt, call)


def test_fused_append_unsupported_path(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    w = make(spec("fa", 3, 64, 8, 128, "bf16", "bf16", (20, 200), 16, "random", seed=196))   # 128 rows: tile path
    d = to_device(w)
    B, Qmax, Hq, D = w.q.shape
    kn = torch.zeros((B, Qmax, 8, D), dtype=torch.bfloat16, device=d.q.device)
    with pytest.raises(psv.PtaError):
        psv.taco_paged_tree_attn_append(d.q, kn, kn, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                        d.tree_mask, d.scale, max_ctx_len=d.max_ctx_len)


# the append fused into the balanced entry's 32x32x16 grid: more than 32 rows per KV head;
# long contexts over few units make slices of one or two pages, so a sequence's candidates
# often fall on pages of two slices (each slice writes and reads only its own)
BALANCED_FUSED_CASES = [
    ("g8_q8", spec("fb", 3, 64, 8, 128, "bf16", "bf16", (300, 900), 8, "random", seed=211)),
    ("g16_q16_two_row_groups", spec("fb", 2, 64, 4, 128, "bf16", "bf16", (500, 900), 16, "random", seed=212)),
    ("ragged_q16_d64", spec("fb", 5, 32, 4, 64, "bf16", "bf16", (1, 400), 16, "random", ragged=True, seed=213)),
    ("g8_q32_chain", spec("fb", 2, 64, 8, 128, "bf16", "bf16", (33, 1500), 32, "chain", seed=214)),
]


@pytest.mark.parametrize("cid,sp", BALANCED_FUSED_CASES, ids=[c[0] for c in BALANCED_FUSED_CASES])
def test_balanced_fused_append_parity(torch_cuda, cid, sp):
    import torch
    import paged_speculative_verify_amd as psv
    seen = {}

    def call(d, kn, vn, out, lse):
        need = psv.taco_paged_tree_attn_balanced_workspace_size(d.q, d.k_cache, d.block_tables,
                                                                max_ctx_len=d.max_ctx_len)
        seen["ws"] = torch.zeros(need, dtype=torch.uint8, device=d.q.device)
        psv.taco_paged_tree_attn_balanced_append(d.q, kn, vn, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                                 d.q_lens, d.tree_mask, d.scale, out=out, lse=lse,
                                                 workspace=seen["ws"], max_ctx_len=d.max_ctx_len)
        seen.update(d=d, kn=kn, vn=vn, out=out)
    w = check_fused_append(cid, sp, "bf16", call)
    # a second call on the appended cache and the same workspace: same bytes, same outputs
    d, ws = seen["d"], seen["ws"]
    k_before = d.k_cache.clone()
    out2 = torch.full_like(d.q, float("nan"))
    psv.taco_paged_tree_attn_balanced_append(d.q, seen["kn"], seen["vn"], d.k_cache, d.v_cache, d.block_tables,
                                             d.ctx_lens, d.q_lens, d.tree_mask, d.scale, out=out2, workspace=ws,
                                             max_ctx_len=d.max_ctx_len)
    torch.cuda.synchronize()
    assert torch.equal(d.k_cache.view(torch.int16), k_before.view(torch.int16))
    a, b = seen["out"].float().cpu().numpy(), out2.float().cpu().numpy()
    for i in range(w.q.shape[0]):
        qb = int(w.q_lens[i])
        assert np.array_equal(a[i, :qb], b[i, :qb]), "repeat call"


def test_balanced_fused_append_unsupported(torch_cuda):
    """Served only by the 32x32x16 grid: fp8 KV (streaming balanced grid) and the 16x16x32
    path are refused, and so are rows in another dtype."""
    import torch
    import paged_speculative_verify_amd as psv
    for kv, path in (("fp8", "auto"), ("bf16", "tile16")):
        w = make(spec("fb", 3, 64, 8, 128, "bf16", kv, (20, 200), 8, "random", seed=215))
        d = to_device(w)
        B, Qmax, Hq, D = w.q.shape
        kn = torch.zeros((B, Qmax, 8, D), dtype=torch.bfloat16, device=d.q.device)
        say("balanced fused unsupported", kv, path)
        with pytest.raises(psv.PtaError) as e:
            psv.taco_paged_tree_attn_balanced_append(d.q, kn, kn, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                                     d.q_lens, d.tree_mask, d.scale, max_ctx_len=d.max_ctx_len,
                                                     path=path)
        assert e.value.status == 4, e.value


# The cache hint (PTA_FLAG_SHARED_PAGES) changes how page tiles are loaded, never what is
# computed: both settings give the same bits, on the streaming kernel (decode, fp8), the wide
# kernel with one row group (streamed) and two (cached either way), the 16x16x32 tile kernels
# (whole entry, and the balanced entry on path tile16: the hint leaves them alone), and
# shared-prefix tables.
HINT_CASES = [
    ("decode_stream", spec("h", 6, 32, 8, 128, "bf16", "bf16", (1, 700), 1, "chain", seed=231), "whole", "auto"),
    ("fp8_chain_stream", spec("h", 6, 32, 8, 128, "bf16", "fp8", (8, 900), 8, "chain", seed=232), "whole",
     "auto"),
    ("wide_one_row_group", spec("h", 3, 64, 8, 128, "bf16", "bf16", (300, 900), 16, "random", seed=233),
     "balanced", "auto"),
    ("wide_two_row_groups", spec("h", 2, 64, 8, 128, "bf16", "bf16", (500, 900), 32, "random", 8, seed=234),
     "balanced", "auto"),
    ("tile_whole", spec("h", 3, 64, 8, 128, "bf16", "bf16", (300, 900), 16, "random", seed=236), "whole",
     "auto"),
    ("tile16_balanced", spec("h", 3, 64, 8, 128, "bf16", "bf16", (300, 900), 16, "random", seed=237),
     "balanced", "tile16"),
    ("shared_prefix_tables", spec("h", 16, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=235,
                                  share_group=4, shared_prefix_pages=8), "whole", "auto"),
]


@pytest.mark.parametrize("cid,sp,mode,path", HINT_CASES, ids=[c[0] for c in HINT_CASES])
def test_cache_hint_same_results(torch_cuda, cid, sp, mode, path):
    w = make(sp, poison=True)
    say("cache hint", cid, mode, path)
    o1, l1 = run_gpu(torch_cuda, w, mode=mode, path=path, shared_pages=False)
    o2, l2 = run_gpu(torch_cuda, w, mode=mode, path=path, shared_pages=True)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
    ref, ref_lse = run_oracle(w)
    assert_parity(w, o1, l1, ref, ref_lse)


def test_validate_flags(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    w = make(spec("c", 4, 8, 2, 64, "bf16", "bf16", (20, 100), 4, "chain", seed=71))
    say("validate")
    d = to_device(w)
    args = dict(max_q_len=4, num_blocks=w.num_blocks, max_ctx_len=int(w.ctx_lens.max()))
    assert psv.taco_pta_validate(d.block_tables, d.ctx_lens, d.q_lens, **args) == 0
    bt = d.block_tables.clone()
    bt[1, 0] = w.num_blocks
    assert psv.taco_pta_validate(bt, d.ctx_lens, d.q_lens, **args) == 8
    ql = d.q_lens.clone()
    ql[2] = 5
    assert psv.taco_pta_validate(d.block_tables, d.ctx_lens, ql, **args) & 1
    cl = d.ctx_lens.clone()
    cl[0] = 2
    assert psv.taco_pta_validate(d.block_tables, cl, d.q_lens, **args) & 2


def test_empty_batch_and_errors(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    w = make(spec("e", 2, 8, 2, 64, "bf16", "bf16", (20, 100), 4, "chain", seed=81))
    d = to_device(w)
    say("errors and empty batch")
    with pytest.raises(psv.PtaError):      # max_ctx_len beyond page_size * max_blocks_per_seq
        psv.taco_paged_tree_attn(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                 d.tree_mask, d.scale, max_ctx_len=10 ** 9)
    with pytest.raises(psv.PtaError):      # 8 * 4 = 32 rows on the vector-ALU path
        psv.taco_paged_tree_attn(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                 d.tree_mask, d.scale, path="valu")
    e = lambda t: t[:0]
    out = psv.taco_paged_tree_attn(e(d.q), d.k_cache, d.v_cache, e(d.block_tables), e(d.ctx_lens),
                                   e(d.q_lens), e(d.tree_mask), d.scale)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


# -------------------------------------------------------------- full-size configs, sampled sequences
# (case id, workload, entry override or None for the workload's launch configuration, split, sampled sequences)
FULL = [
    ("llama3_8b_decode", "llama3_8b_decode", None, None, [0, 17, 42, 63]),
    ("llama31_70b_verify", "llama31_70b_verify", None, None, [0, 5, 9, 17, 24, 31]),
    ("long_splitk_verify", "long_splitk_verify", None, None, [1, 2]),
    # fixed 2048-token partitions: up to 64 partials per (sequence, KV head) merged in the launch
    ("long_splitk_verify_split2048", "long_splitk_verify", "split", 2048, [0, 3]),
    ("fp8_kv_chain", "fp8_kv_chain", None, None, [0, 31, 64, 77, 100, 127]),
    ("shared_prefix_decode", "shared_prefix_decode", None, None, [0, 9, 63]),
]


@pytest.mark.parametrize("cid,name,mode,split,seqs", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(torch_cuda, cid, name, mode, split, seqs):
    import bench
    w = make(name)
    cfg = bench.launch_config(name)
    if mode is not None:
        cfg["mode"], cfg["split"] = mode, split
    say("full", cid, "entry", cfg["mode"], "split", cfg["split"], "path", cfg["path"], "sampled seqs", seqs)
    out, lse = run_gpu(torch_cuda, w, split=cfg["split"], path=cfg["path"], mode=cfg["mode"])
    ref, ref_lse = run_oracle(w, rows=np.array(seqs))
    err = assert_parity(w, out, lse, ref, ref_lse, seqs=np.array(seqs))
    say("full", cid, "max abs err", err)
    # every other row is finite and every padding row untouched
    B = w.q.shape[0]
    for b in range(B):
        qb = int(w.q_lens[b])
        assert np.isfinite(out[b, :qb]).all()
        assert np.isnan(out[b, qb:]).all()


# The exact prepared call bench.py times (entry, kernel family, KV append fused into the launch or
# launched before it), at the workload's full size, on the same input set the bench builds first.
# The candidates' cache slots are poisoned before the step, so a step whose append did not run,
# or ran after the pages were read, fails.
TIMED = [
    ("llama3_8b_decode", [0, 17, 42, 63]),
    ("shared_prefix_decode", [0, 9, 63]),
    ("llama31_70b_verify", [0, 9, 31]),
    ("long_splitk_verify", [0, 3]),
    ("fp8_kv_chain", [0, 77, 127]),
]


@pytest.mark.parametrize("name,seqs", TIMED, ids=[t[0] for t in TIMED])
def test_full_size_timed_call(torch_cuda, name, seqs):
    import argparse

    import torch
    import bench
    import paged_speculative_verify_amd as psv
    cfg = bench.resolve_cfg(name, argparse.Namespace(path=None, split=None, shared_entry=False,
                                                     private_pages=False, separate_append=False))
    say("timed", name, "entry", cfg["mode"], "fused append", bool(cfg.get("fuse_append")), "seqs", seqs)
    ds = bench.build_sets(psv, torch, name, cfg, 1)[0]
    w, d = ds.w, ds.d
    pages, offs = [], []
    for b in range(w.q.shape[0]):
        for t in range(int(w.ctx_lens[b]) - int(w.q_lens[b]), int(w.ctx_lens[b])):
            pages.append(int(w.block_tables[b, t // 16]))
            offs.append(t % 16)
    P = torch.tensor(pages, dtype=torch.int64, device=d.q.device)
    O = torch.tensor(offs, dtype=torch.int64, device=d.q.device)
    poison = 0x7F if w.spec.kv_dtype == "fp8" else float("nan")
    d.k_cache[P, :, O] = poison
    d.v_cache[P, :, O] = poison
    ds.out.fill_(float("nan"))
    ds.lse.fill_(float("nan"))
    ds.append_call()
    ds.attn_call()
    torch.cuda.synchronize()
    view = torch.uint8 if w.spec.kv_dtype == "fp8" else torch.int16
    for cache, host in ((d.k_cache, w.k_cache), (d.v_cache, w.v_cache)):
        got = cache[P, :, O].contiguous().view(view).cpu().numpy()
        want = np.stack([host[p, :, o] for p, o in zip(pages, offs)])
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), "candidate rows"
    out = out_to_f64(ds.out)
    lse = ds.lse.cpu().numpy().astype(np.float64)
    ref, ref_lse = run_oracle(w, rows=np.array(seqs))
    err = assert_parity(w, out, lse, ref, ref_lse, seqs=np.array(seqs))
    say("timed", name, "max abs err", err)
    for b in range(w.q.shape[0]):
        qb = int(w.q_lens[b])
        assert np.isfinite(out[b, :qb]).all() and np.isnan(out[b, qb:]).all()


# The whole-context stream grid takes its sequences in an order of their context lengths: long/short
# pairs when the grid is resident at once, longest first when it is larger, grid order past 256
# sequences.  Every sequence must still be computed exactly once, ties (equal lengths) included.
ORDER_CASES = [
    ("pairs_even", spec("o", 40, 32, 8, 128, "bf16", "bf16", (1, 600), 1, "chain", seed=161)),
    ("pairs_odd_ties", spec("o", 41, 32, 8, 128, "bf16", "bf16", (50, 52), 1, "chain", seed=162)),
    ("longest_first", spec("o", 90, 32, 8, 128, "bf16", "bf16", (1, 400), 1, "chain", seed=163)),
    ("longest_first_fp8_chain", spec("o", 80, 32, 8, 128, "bf16", "fp8", (8, 300), 8, "chain", seed=164)),
    ("grid_order_past_256", spec("o", 300, 4, 1, 128, "bf16", "bf16", (1, 100), 1, "chain", seed=165)),
]


@pytest.mark.parametrize("cid,sp", ORDER_CASES, ids=[c[0] for c in ORDER_CASES])
def test_whole_grid_sequence_order(torch_cuda, cid, sp):
    w = make(sp, poison=True)
    say(cid, "B", w.q.shape[0], "Hkv", w.k_cache.shape[1], "ctx", w.ctx_lens.tolist()[:8])
    out, lse = run_gpu(torch_cuda, w, mode="whole")
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)


# Shared-prefix pages: groups of sequences alias their first pages in the block tables.
SHARED_CASES = [
    ("shared_decode_whole", spec("s", 24, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=171,
                                 share_group=8, shared_prefix_pages=12), "whole"),
    ("shared_decode_balanced", spec("s", 24, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=171,
                                    share_group=8, shared_prefix_pages=12), "balanced"),
    ("shared_tree16_balanced", spec("s", 8, 64, 8, 128, "bf16", "bf16", (200, 700), 16, "random", 6, seed=172,
                                    share_group=4, shared_prefix_pages=8), "balanced"),
    ("shared_fp8_chain_whole", spec("s", 16, 32, 8, 128, "bf16", "fp8", (200, 700), 8, "chain", seed=173,
                                    share_group=4, shared_prefix_pages=8), "whole"),
]


@pytest.mark.parametrize("cid,sp,mode", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_shared_prefix_parity(torch_cuda, cid, sp, mode):
    w = make(sp, poison=True)
    say(cid, "B", w.q.shape[0], "group", sp.share_group, "shared pages", sp.shared_prefix_pages, "mode", mode)
    out, lse = run_gpu(torch_cuda, w, mode=mode)
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)


# taco_paged_tree_attn_shared_prefix: partition 0 of each group worked once for all members' rows.
def leaders_by_group(B, alias, size):
    """Leaders of runs of `size` consecutive sequences inside each run of `alias` sequences that
    alias the same prefix pages (a group must never span two aliasing runs)."""
    lead = []
    for b in range(B):
        g0 = (b // alias) * alias
        lead.append(g0 + ((b - g0) // size) * size)
    return np.array(lead, dtype=np.int32)


SHARED_ENTRY_CASES = [
    # (id, spec, group sizes handed to the entry (None: the workload's groups), max_group)
    ("decode_groups8", spec("se", 24, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=181,
                            share_group=8, shared_prefix_pages=12), None, 8),
    ("tree2_groups4", spec("se", 16, 32, 8, 128, "bf16", "bf16", (200, 700), 2, "random", seed=182,
                           share_group=4, shared_prefix_pages=8), None, 4),
    ("fp8_decode_groups8", spec("se", 16, 32, 8, 128, "bf16", "fp8", (300, 900), 1, "chain", seed=183,
                                share_group=8, shared_prefix_pages=8), None, 8),
    ("ragged_last_group", spec("se", 20, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=184,
                               share_group=8, shared_prefix_pages=10), None, 8),
    # the workload's groups of 8 handed over as groups of 3, 3 and 2: any split of a run of aliased
    # sequences into consecutive groups is valid
    ("split_groups3", spec("se", 16, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=185,
                           share_group=8, shared_prefix_pages=12), 3, 8),
    # groups of one: every sequence works its own partition 0
    ("groups_of_one", spec("se", 8, 32, 8, 128, "bf16", "bf16", (300, 900), 1, "chain", seed=186,
                           share_group=8, shared_prefix_pages=12), 1, 8),
]


@pytest.mark.parametrize("cid,sp,gsize,max_group", SHARED_ENTRY_CASES, ids=[c[0] for c in SHARED_ENTRY_CASES])
def test_shared_prefix_entry_parity(torch_cuda, cid, sp, gsize, max_group):
    import paged_speculative_verify_amd as psv
    torch = torch_cuda
    w = make(sp, poison=True)
    d = to_device(w)
    B, Qmax, Hq, D = w.q.shape
    lead = leaders_by_group(B, sp.share_group, gsize or sp.share_group)
    T = sp.shared_prefix_pages * 16
    say(cid, "B", B, "groups of", gsize or sp.share_group, "shared tokens", T, "max_group", max_group)
    leader = torch.from_numpy(lead).to(d.q.device)
    ws = torch.zeros(psv.taco_paged_tree_attn_splitk_workspace_size(d.q, d.k_cache, d.block_tables, T,
                                                                     max_ctx_len=d.max_ctx_len),
                     dtype=torch.uint8, device=d.q.device)
    outs = []
    for _ in range(2):                       # the workspace's counters are left zero for reuse
        out = torch.full_like(d.q, float("nan"))
        lse = torch.full((B, Hq, Qmax), float("nan"), dtype=torch.float32, device=d.q.device)
        psv.taco_paged_tree_attn_shared_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                               d.tree_mask, leader, max_group, T, d.scale, out=out, lse=lse,
                                               k_scale=d.k_scale, v_scale=d.v_scale, workspace=ws,
                                               max_ctx_len=d.max_ctx_len)
        torch.cuda.synchronize()
        outs.append((out_to_f64(out), lse.cpu().numpy().astype(np.float64)))
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, outs[0][0], outs[0][1], ref, ref_lse)
    assert np.array_equal(outs[0][0], outs[1][0], equal_nan=True), "repeat call differs"
    assert int(ws[:B * 8 * 4].view(torch.int32).abs().sum()) == 0, "arrival counters not left zero"
    say(cid, "max abs err", err)


def test_shared_prefix_entry_rejects_too_many_rows(torch_cuda):
    import paged_speculative_verify_amd as psv
    torch = torch_cuda
    w = make(spec("se", 8, 32, 8, 128, "bf16", "bf16", (300, 600), 1, "chain", seed=187,
                  share_group=8, shared_prefix_pages=8))
    d = to_device(w)
    leader = torch.zeros(8, dtype=torch.int32, device=d.q.device)
    with pytest.raises(psv.PtaError):        # 9 sequences x 4 rows exceed one 32-row unit
        psv.taco_paged_tree_attn_shared_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                               d.tree_mask, leader, 9, 128, d.scale, max_ctx_len=d.max_ctx_len)


def test_splitk_workspace_reused_across_calls(torch_cuda):
    """One zero-filled workspace serves several split-K calls in a row (the
    fused merge resets its arrival counters), with changing partition lengths
    and batches, and every call matches the oracle."""
    import torch
    import paged_speculative_verify_amd as psv
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for n, (sp, split) in enumerate([
            (spec("w", 5, 32, 8, 128, "bf16", "bf16", (40, 3000), 1, "chain", seed=91), 256),
            (spec("w", 3, 32, 8, 128, "bf16", "bf16", (40, 3000), 1, "chain", seed=92), 64),
            (spec("w", 4, 64, 8, 128, "bf16", "bf16", (40, 2000), 16, "random", 6, seed=93), 128),
            (spec("w", 5, 32, 8, 128, "bf16", "fp8", (40, 3000), 8, "chain", seed=94), 512),
            (spec("w", 5, 32, 8, 128, "bf16", "bf16", (40, 3000), 1, "chain", seed=91), 256)]):
        w = make(sp, poison=True)
        say("workspace reuse", n, sp.kv_dtype, "q", sp.q_len, "split", split)
        d = to_device(w)
        need = psv.taco_paged_tree_attn_splitk_workspace_size(d.q, d.k_cache, d.block_tables, split,
                                                               max_ctx_len=d.max_ctx_len)
        assert 0 < need <= ws.numel()
        out = torch.full_like(d.q, float("nan"))
        B, Qmax, Hq, D = w.q.shape
        lse = torch.full((B, Hq, Qmax), float("nan"), dtype=torch.float32, device="cuda")
        psv.taco_paged_tree_attn_splitk(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                        d.tree_mask, d.scale, split, out=out, lse=lse, k_scale=d.k_scale,
                                        v_scale=d.v_scale, workspace=ws, max_ctx_len=d.max_ctx_len)
        torch.cuda.synchronize()
        ref, ref_lse = run_oracle(w)
        assert_parity(w, out_to_f64(out), lse.cpu().numpy().astype(np.float64), ref, ref_lse)
        counters = ws[:B * w.k_cache.shape[1] * 4].view(torch.int32)
        assert int(counters.abs().sum()) == 0, "arrival counters not reset"


# -------------------------------------------------------------- work-balanced entry point
BALANCED = [
    ("bal_decode_bf16", spec("b", 9, 32, 8, 128, "bf16", "bf16", (1, 2500), 1, "chain", seed=101)),
    ("bal_decode_long_ragged", spec("b", 5, 32, 8, 128, "bf16", "bf16", (1, 9000), 1, "chain", seed=102)),
    ("bal_tree_g2", spec("b", 7, 16, 8, 128, "bf16", "bf16", (5, 1500), 8, "random", 4, True, seed=103)),
    ("bal_fp8_chain8", spec("b", 6, 32, 8, 128, "bf16", "fp8", (8, 3000), 8, "chain", seed=104)),
    ("bal_d64", spec("b", 6, 16, 4, 64, "bf16", "bf16", (2, 2000), 4, "random", ragged=True, seed=105)),
    ("bal_fp8_d64", spec("b", 4, 8, 2, 64, "bf16", "fp8", (3, 1200), 6, "random", seed=106)),
    ("bal_tiny_units", spec("b", 40, 8, 2, 128, "bf16", "bf16", (1, 20), 1, "chain", seed=107)),
    ("bal_one_seq", spec("b", 1, 8, 1, 128, "bf16", "bf16", (30000, 30000), 2, "chain", seed=108)),
    # shared-tile family (more than 32 rows per KV head, bf16 KV)
    ("bal_tile_tree16", spec("bt", 5, 64, 8, 128, "bf16", "bf16", (16, 3000), 16, "random", 6, seed=121)),
    ("bal_tile_tree32_rg2", spec("bt", 2, 64, 8, 128, "bf16", "bf16", (300, 9000), 32, "random", 8, seed=122)),
    ("bal_tile_ragged_rg2", spec("bt", 6, 32, 4, 128, "bf16", "bf16", (1, 2500), 32, "random", ragged=True,
                                 seed=123)),
    ("bal_tile_d64", spec("bt", 5, 16, 4, 64, "bf16", "bf16", (1, 1800), 20, "random", ragged=True, seed=124)),
    ("bal_tile_rows48", spec("bt", 6, 8, 2, 128, "bf16", "bf16", (12, 2200), 12, "random", seed=125)),
    ("bal_tile_tiny_units", spec("bt", 50, 16, 2, 128, "bf16", "bf16", (8, 40), 8, "chain", seed=126)),
    # many (sequence, KV head) units, most of them cut into two or three slices
    ("bal_tile_inline_merge", spec("bt", 40, 32, 4, 128, "bf16", "bf16", (16, 3000), 16, "random", 6,
                                   seed=127)),
]


@pytest.mark.parametrize("cid,sp", BALANCED, ids=[c[0] for c in BALANCED])
def test_balanced_parity(torch_cuda, cid, sp):
    w = make(sp, poison=True)
    say(cid, "B", w.q.shape[0], "ctx", w.ctx_lens.tolist()[:8], "q", sp.q_len, sp.kv_dtype)
    out, lse = run_gpu(torch_cuda, w, mode="balanced")
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)


# the 16x16x32-product shared-tile kernel (path tile16; also what the balanced entry runs when a
# cache tensor exceeds 4 GiB) on the shared-tile cases
TILE16 = [c for c in BALANCED if c[0].startswith("bal_tile")]


@pytest.mark.parametrize("cid,sp", TILE16, ids=[c[0] + "_tile16" for c in TILE16])
def test_balanced_tile16_parity(torch_cuda, cid, sp):
    w = make(sp, poison=True)
    say(cid, "tile16")
    out, lse = run_gpu(torch_cuda, w, mode="balanced", path="tile16")
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "tile16 max abs err", err)


def test_balanced_repeat_and_workspace_reuse(torch_cuda):
    """The same workspace serves repeated calls; results are bit-identical from call to call
    and unchanged by a relabelling of physical pages."""
    import torch
    import paged_speculative_verify_amd as psv
    w = make(spec("r", 8, 32, 8, 128, "bf16", "bf16", (100, 6000), 1, "chain", seed=111))
    d = to_device(w)
    need = psv.taco_paged_tree_attn_balanced_workspace_size(d.q, d.k_cache, d.block_tables,
                                                            max_ctx_len=d.max_ctx_len)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say("balanced repeat, workspace", need)
    a1, l1 = run_gpu(torch_cuda, w, mode="balanced", workspace=ws)
    a2, l2 = run_gpu(torch_cuda, w, mode="balanced", workspace=ws)
    b1, m1 = run_gpu(torch_cuda, permute_pool(w, 7), mode="balanced", workspace=ws)
    assert np.array_equal(a1, a2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
    assert np.array_equal(a1, b1, equal_nan=True) and np.array_equal(l1, m1, equal_nan=True)
    ref, ref_lse = run_oracle(w)
    assert_parity(w, a1, l1, ref, ref_lse)


def test_balanced_rejects_unserved_dims(torch_cuda):
    import paged_speculative_verify_amd as psv
    w = make("tiny_decode")                     # fp32 q: not served by the matrix-core stream
    d = to_device(w)
    with pytest.raises(psv.PtaError):
        psv.taco_paged_tree_attn_balanced(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                          d.q_lens, d.tree_mask, d.scale, max_ctx_len=d.max_ctx_len)
    w = make(spec("x", 2, 64, 8, 128, "bf16", "fp8", (20, 100), 16, "random", seed=112))   # 128 rows, fp8
    d = to_device(w)
    with pytest.raises(psv.PtaError):
        psv.taco_paged_tree_attn_balanced(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                          d.q_lens, d.tree_mask, d.scale, k_scale=d.k_scale,
                                          v_scale=d.v_scale, max_ctx_len=d.max_ctx_len)


def test_balanced_tile_repeat_and_workspace_reuse(torch_cuda):
    """Shared-tile balanced grid with two row groups: repeated calls on one workspace are
    bit-identical and unchanged by a relabelling of physical pages."""
    import torch
    import paged_speculative_verify_amd as psv
    w = make(spec("rt", 3, 64, 8, 128, "bf16", "bf16", (500, 12000), 32, "random", 8, seed=131))
    d = to_device(w)
    need = psv.taco_paged_tree_attn_balanced_workspace_size(d.q, d.k_cache, d.block_tables,
                                                            max_ctx_len=d.max_ctx_len)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say("balanced tile repeat, workspace", need)
    a1, l1 = run_gpu(torch_cuda, w, mode="balanced", workspace=ws)
    a2, l2 = run_gpu(torch_cuda, w, mode="balanced", workspace=ws)
    b1, m1 = run_gpu(torch_cuda, permute_pool(w, 9), mode="balanced", workspace=ws)
    assert np.array_equal(a1, a2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
    assert np.array_equal(a1, b1, equal_nan=True) and np.array_equal(l1, m1, equal_nan=True)
    ref, ref_lse = run_oracle(w)
    assert_parity(w, a1, l1, ref, ref_lse)


@pytest.mark.parametrize("cid,sp", [
    ("bal_decode_tile", spec("bd", 9, 32, 8, 128, "bf16", "bf16", (1, 2500), 1, "chain", seed=141)),
    ("bal_chain8_tile", spec("bd", 6, 32, 8, 128, "bf16", "bf16", (8, 3000), 8, "chain", seed=142)),
], ids=["bal_decode_tile", "bal_chain8_tile"])
def test_balanced_tile_path_small_rows(torch_cuda, cid, sp):
    w = make(sp, poison=True)
    say(cid, "B", w.q.shape[0], "ctx", w.ctx_lens.tolist()[:8], "q", sp.q_len)
    out, lse = run_gpu(torch_cuda, w, mode="balanced", path="tile")
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)


# -------------------------------------------------------------- sign and zero of the scale
# The matrix-core paths fold a negative scale into the sign of Q and clamp a zero scale to
# the smallest normal float; both must still give the plain softmax(scale * q.k) result.
SCALE_CASES = [
    ("stream_whole", spec("sc", 4, 16, 4, 128, "bf16", "bf16", (20, 900), 4, "random", seed=151), "whole", "mfma"),
    ("stream_fp8_bal", spec("sc", 4, 32, 8, 128, "bf16", "fp8", (20, 900), 4, "chain", seed=152), "balanced",
     "auto"),
    ("tile_whole", spec("sc", 3, 32, 4, 128, "bf16", "bf16", (20, 900), 16, "random", seed=153), "whole", "tile"),
    ("tile_bal", spec("sc", 3, 32, 4, 128, "bf16", "bf16", (20, 900), 16, "random", seed=154), "balanced", "auto"),
    ("tile_fp8", spec("sc", 3, 32, 4, 128, "bf16", "fp8", (20, 900), 16, "random", seed=155), "whole", "tile"),
]


@pytest.mark.parametrize("scale", [-0.0883883, 0.0], ids=["negative", "zero"])
@pytest.mark.parametrize("cid,sp,mode,path", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_scale_sign_and_zero(torch_cuda, cid, sp, mode, path, scale):
    import dataclasses
    w = make(dataclasses.replace(sp, scale=scale), poison=True)
    say(cid, "scale", scale, "mode", mode, "path", path)
    out, lse = run_gpu(torch_cuda, w, mode=mode, path=path)
    ref, ref_lse = run_oracle(w)
    err = assert_parity(w, out, lse, ref, ref_lse)
    say(cid, "max abs err", err)
