"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin is written as a check function that raises AssertionError, so the
mutation tests at the end can plant a plausible mistake in the oracle and
show that at least one pin catches it.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import oracle.attention as oatt
from workload import Spec, make, permute_pool, tree_mask_from_parents
from workload.gen import f32_to_bf16_bits
from tests import refs


def small(name="s", B=2, Hq=4, Hkv=2, D=16, q_dtype="f32", kv_dtype="f32", ctx=(20, 50),
          q_len=4, tree="random", depth=None, seed=0, ragged=False, **kw):
    return Spec(name, B, Hq, Hkv, D, q_dtype, kv_dtype, ctx_range=ctx, q_len=q_len,
                q_len_ragged=ragged, tree=tree, depth_cap=depth, seed=seed, **kw)


def run_oracle(w, **kw):
    s = w.spec
    return oracle.paged_tree_attn(w.q, w.k_cache, w.v_cache, w.block_tables, w.ctx_lens,
                                  w.q_lens, w.tree_mask, w.scale, q_dtype=s.q_dtype,
                                  kv_dtype=s.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale, **kw)


# ---------------------------------------------------------------- check functions
def enc(value, dtype):
    """Store a float value in a cache/q element format (exact for the probe values used)."""
    v = np.float32(value)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(np.array([v]))[0]
    if dtype == "fp8":
        return torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    raise ValueError(dtype)


def check_fp8_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.fp8_e4m3fn_table()
    nan_l, nan_o = np.isnan(lib), np.isnan(ours)
    assert (nan_l == nan_o).all()
    assert np.array_equal(lib[~nan_l], ours[~nan_o])
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def check_fp8_encode(x: np.ndarray):
    x32 = np.clip(x.astype(np.float32), -448, 448)
    lib = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.encode_fp8_e4m3fn(x32.astype(np.float64))
    # +-0 may differ only in sign bit handling of exact zero; compare values and codes
    assert np.array_equal(lib, ours), (x32[lib != ours][:8], lib[lib != ours][:8], ours[lib != ours][:8])


def check_bruteforce(w, tol=1e-12, **kw):
    out, _ = run_oracle(w, **kw)
    ref = refs.workload_sdpa(w)
    valid = ~np.isnan(ref)
    assert (np.isnan(out) == ~valid).all()
    err = np.abs(out[valid] - ref[valid]).max()
    assert err <= tol, err


def check_decode_equivalence(w):
    """q_len = 1: ordinary single-token decode over all C positions."""
    assert (w.q_lens == 1).all()
    out, lse = run_oracle(w)
    qd = refs.torch_decode(w.q, w.spec.q_dtype)
    Hq, Hkv = w.q.shape[2], w.k_cache.shape[1]
    for b in range(w.q.shape[0]):
        C = int(w.ctx_lens[b])
        K = refs.unpage(w.k_cache, w.block_tables[b], C, w.spec.kv_dtype, w.k_scale)
        V = refs.unpage(w.v_cache, w.block_tables[b], C, w.spec.kv_dtype, w.v_scale)
        for h in range(Hq):
            s = w.scale * (K[h // (Hq // Hkv)] @ qd[b, 0, h])
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ V[h // (Hq // Hkv)]
            assert np.abs(out[b, 0, h] - ref).max() <= 1e-12
            assert abs(lse[b, h, 0] - (s.max() + math.log(p.sum()))) <= 1e-12


def check_chain_is_causal(w):
    """A linear chain of candidates is bottom-right-aligned causal attention."""
    out, _ = run_oracle(w)
    qd = refs.torch_decode(w.q, w.spec.q_dtype)
    Hq, Hkv = w.q.shape[2], w.k_cache.shape[1]
    for b in range(w.q.shape[0]):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        K = refs.unpage(w.k_cache, w.block_tables[b], C, w.spec.kv_dtype, w.k_scale)
        V = refs.unpage(w.v_cache, w.block_tables[b], C, w.spec.kv_dtype, w.v_scale)
        # query i sits at absolute position C - Qb + i and sees positions <= its own
        causal = np.arange(C)[None, :] <= (C - Qb + np.arange(Qb))[:, None]
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            ref = refs.sdpa(qd[b, :Qb, h], K[hk], V[hk], causal, w.scale)
            assert np.abs(out[b, :Qb, h] - ref).max() <= 1e-12


def check_node_is_path(w):
    """Tree node i equals decode over prefix + its ancestors + itself, as one contiguous sequence."""
    out, _ = run_oracle(w)
    qd = refs.torch_decode(w.q, w.spec.q_dtype)
    Hq, Hkv = w.q.shape[2], w.k_cache.shape[1]
    for b in range(w.q.shape[0]):
        C, Qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        L = C - Qb
        K = refs.unpage(w.k_cache, w.block_tables[b], C, w.spec.kv_dtype, w.k_scale)
        V = refs.unpage(w.v_cache, w.block_tables[b], C, w.spec.kv_dtype, w.v_scale)
        for i in range(Qb):
            path = sorted(refs.ancestors_or_self(w.parents[b], i))
            idx = list(range(L)) + [L + j for j in path]
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                s = w.scale * (K[hk][idx] @ qd[b, i, h])
                p = np.exp(s - s.max())
                ref = (p / p.sum()) @ V[hk][idx]
                assert np.abs(out[b, i, h] - ref).max() <= 1e-12


def check_permutation_bit_identical(w, seed=7):
    out1, lse1 = run_oracle(w)
    out2, lse2 = run_oracle(permute_pool(w, seed))
    assert np.array_equal(out1, out2, equal_nan=True)
    assert np.array_equal(lse1, lse2, equal_nan=True)


def check_split_identity(w, T):
    s = w.spec
    O, LSE = oracle.paged_tree_attn_partials(
        w.q, w.k_cache, w.v_cache, w.block_tables, w.ctx_lens, w.q_lens, w.tree_mask, w.scale, T,
        q_dtype=s.q_dtype, kv_dtype=s.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    out_m, lse_m = oracle.merge_partials(O, LSE)
    out, lse = run_oracle(w)
    assert (np.isnan(out) == np.isnan(out_m)).all()
    v = ~np.isnan(out)
    assert np.abs(out[v] - out_m[v]).max() <= 1e-12
    v = ~np.isnan(lse)
    assert np.abs(lse[v] - lse_m[v]).max() <= 1e-12


def check_closed_forms(w):
    """K = 0 -> uniform weights: out = mean of visible V rows; lse = ln(#visible)."""
    w0 = make(w.spec)
    w0.k_cache[...] = 0
    out, lse = run_oracle(w0)
    Hq, Hkv = w0.q.shape[2], w0.k_cache.shape[1]
    for b in range(w0.q.shape[0]):
        C, Qb = int(w0.ctx_lens[b]), int(w0.q_lens[b])
        V = refs.unpage(w0.v_cache, w0.block_tables[b], C, w0.spec.kv_dtype, w0.v_scale)
        vis = refs.vis_from_parents(C, Qb, w0.parents[b])
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Qb):
                ref = V[hk][vis[i]].mean(axis=0)
                assert np.abs(out[b, i, h] - ref).max() <= 1e-12
                assert abs(lse[b, h, i] - math.log(vis[i].sum())) <= 1e-12


def check_constant_v(w):
    """All V rows equal c -> out = c whatever the weights."""
    wc = make(w.spec)
    c = np.linspace(-2, 2, wc.v_cache.shape[-1])
    if wc.spec.kv_dtype == "f32":
        wc.v_cache[...] = c.astype(np.float32)
    else:
        wc.v_cache[...] = f32_to_bf16_bits(c.astype(np.float32))
        c = refs.torch_decode(f32_to_bf16_bits(c.astype(np.float32)), "bf16")
    out, _ = run_oracle(wc)
    valid = ~np.isnan(out[..., 0])
    assert np.abs(out[valid] - c).max() <= 1e-12


def check_one_hot_probe(w, seed=3):
    """Make one visible key dominate by a score gap >= 1000: out equals that V row exactly.

    V row t of KV head hk holds integers encoding (hk, t) in two channels, so
    the output names the logical position read.
    """
    rng = np.random.default_rng(seed)
    wp = make(w.spec)
    kv, qd = wp.spec.kv_dtype, wp.spec.q_dtype
    B, Qmax, Hq, D = wp.q.shape
    Hkv = wp.k_cache.shape[1]
    G = Hq // Hkv
    assert D >= 2 + G * Qmax, "probe needs one channel per (group member, candidate)"
    wrap = 16 if kv == "fp8" else 256          # integers exact in the storage format
    if wp.k_scale is not None:
        wp.k_scale[...] = 1.0
        wp.v_scale[...] = 1.0
    wp.q[...] = 0
    wp.k_cache[...] = 0
    wp.v_cache[...] = 0
    targets = {}
    for b in range(B):
        C, Qb = int(wp.ctx_lens[b]), int(wp.q_lens[b])
        vis = refs.vis_from_parents(C, Qb, wp.parents[b])
        for t in range(C):
            page, slot = wp.block_tables[b, t // 16], t % 16
            for hk in range(Hkv):
                wp.v_cache[page, hk, slot, 0] = enc(t % wrap, kv)
                wp.v_cache[page, hk, slot, 1] = enc((hk + 3 * b) % wrap, kv)
        for h in range(Hq):
            hk = h // G
            for i in range(Qb):
                t = int(rng.choice(np.flatnonzero(vis[i])))
                targets[(b, i, h)] = (t, hk)
                # key t of head hk gets a private channel set to 1; the q row puts ~1000/scale
                # there, a score gap past fp64 exp underflow, so the result is exact in any precision
                page, slot = wp.block_tables[b, t // 16], t % 16
                ch = 2 + (h % G) * Qmax + i
                wp.k_cache[page, hk, slot, ch] = enc(1.0, kv)
                wp.q[b, i, h, ch] = enc(2.0 ** math.ceil(math.log2(1000.0 / wp.scale)), qd)
    out, _ = run_oracle(wp)
    for (b, i, h), (t, hk) in targets.items():
        assert out[b, i, h, 0] == t % wrap and out[b, i, h, 1] == (hk + 3 * b) % wrap, \
            ((b, i, h), out[b, i, h, :2], t)


def check_mask_probe(w):
    """K = 0, prefix V = 0, candidate j's V = e_j: out_i[j] > 0 iff mask[i, j]."""
    wm = make(w.spec)
    wm.k_cache[...] = 0
    wm.v_cache[...] = 0
    if wm.k_scale is not None:
        wm.k_scale[...] = 1.0
        wm.v_scale[...] = 1.0
    B, Qmax, Hq, D = wm.q.shape
    assert D >= Qmax
    for b in range(B):
        C, Qb = int(wm.ctx_lens[b]), int(wm.q_lens[b])
        L = C - Qb
        for j in range(Qb):
            t = L + j
            wm.v_cache[wm.block_tables[b, t // 16], :, t % 16, j] = enc(1.0, wm.spec.kv_dtype)
    out, _ = run_oracle(wm)
    for b in range(B):
        Qb = int(wm.q_lens[b])
        ref_mask = tree_mask_from_parents(wm.parents[b, :Qb], Qb) != 0
        for h in range(Hq):
            got = out[b, :Qb, h, :Qb] > 0
            assert np.array_equal(got, ref_mask)


def check_gqa_is_replicated_mha(w):
    out, _ = run_oracle(w)
    Hq, Hkv = w.q.shape[2], w.k_cache.shape[1]
    G = Hq // Hkv
    k = np.repeat(w.k_cache, G, axis=1)
    v = np.repeat(w.v_cache, G, axis=1)
    ks = np.repeat(w.k_scale, G, axis=1) if w.k_scale is not None else None
    vs = np.repeat(w.v_scale, G, axis=1) if w.v_scale is not None else None
    s = w.spec
    out2, _ = oracle.paged_tree_attn(w.q, k, v, w.block_tables, w.ctx_lens, w.q_lens, w.tree_mask,
                                     w.scale, q_dtype=s.q_dtype, kv_dtype=s.kv_dtype,
                                     k_scale=ks, v_scale=vs)
    assert np.array_equal(out, out2, equal_nan=True)


# ---------------------------------------------------------------- tests
def test_fp8_table_matches_library():
    check_fp8_table()


def test_fp8_encode_matches_library():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.standard_normal(20000) * 0.01,
        rng.uniform(-448, 448, 20000),
        # every representable value and every midpoint between neighbours (ties)
        oracle.fp8_e4m3fn_table()[:0x7F],
        (oracle.fp8_e4m3fn_table()[:0x7E] + oracle.fp8_e4m3fn_table()[1:0x7F]) / 2,
        -(oracle.fp8_e4m3fn_table()[1:0x7E] + oracle.fp8_e4m3fn_table()[2:0x7F]) / 2,
        [0.0, 2.0 ** -10, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5, 447.9, 448.0],
    ])
    check_fp8_encode(x)


def test_fp8_encode_saturates_and_nan():
    codes = oracle.encode_fp8_e4m3fn(np.array([1e6, -1e6, 470.0, np.nan]))
    assert list(codes) == [0x7E, 0xFE, 0x7E, 0x7F]


def test_bf16_decode_matches_library():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    lib = refs.torch_decode(bits, "bf16")
    assert np.array_equal(ours, lib, equal_nan=True)


@pytest.mark.parametrize("spec", [
    small(seed=1),
    small(q_dtype="bf16", kv_dtype="bf16", Hq=8, Hkv=2, D=64, ctx=(17, 70), q_len=6, seed=2),
    small(q_dtype="bf16", kv_dtype="fp8", Hq=4, Hkv=1, D=32, ctx=(1, 40), q_len=1, seed=3),
    small(q_dtype="bf16", kv_dtype="fp8", Hq=4, Hkv=2, D=16, ctx=(30, 60), q_len=5, ragged=True, seed=4),
    small(B=3, ctx=(6, 33), q_len=6, ragged=True, tree="flat", seed=5),
])
def test_bruteforce_sdpa(spec):
    check_bruteforce(make(spec))


def test_bruteforce_with_poison():
    """Padding pages, tail slots and padding Q rows hold NaN; the result is unaffected."""
    spec = small(q_dtype="bf16", kv_dtype="bf16", ctx=(3, 45), q_len=3, ragged=True, seed=11)
    w = make(spec, poison=True)
    check_bruteforce(w)


def test_tiny_decode_config_bruteforce():
    w = make("tiny_decode")
    assert list(w.ctx_lens) == [37, 80] and w.num_blocks == 16
    check_bruteforce(w)
    check_decode_equivalence(w)


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(B=st.integers(1, 3), C_hi=st.integers(1, 70), q=st.integers(1, 6), D=st.sampled_from([8, 64]),
       G=st.sampled_from([1, 2, 4]), Hkv=st.sampled_from([1, 2]), ragged=st.booleans(),
       tree=st.sampled_from(["random", "chain", "flat"]), seed=st.integers(0, 10 ** 6),
       kv=st.sampled_from(["f32", "bf16", "fp8"]))
def test_bruteforce_fuzz(B, C_hi, q, D, G, Hkv, ragged, tree, seed, kv):
    qd = "f32" if kv == "f32" else "bf16"
    spec = Spec("fz", B, G * Hkv, Hkv, D, qd, kv, ctx_range=(1, max(1, C_hi)), q_len=q,
                q_len_ragged=ragged, tree=tree, seed=seed)
    check_bruteforce(make(spec))


def test_decode_equivalence():
    check_decode_equivalence(make(small(q_len=1, tree="chain", ctx=(1, 90), seed=21)))
    check_decode_equivalence(make(small(q_dtype="bf16", kv_dtype="fp8", q_len=1, tree="chain",
                                        ctx=(5, 90), seed=22)))


def test_chain_is_causal():
    check_chain_is_causal(make(small(q_len=6, tree="chain", ctx=(6, 80), seed=31)))
    check_chain_is_causal(make(small(q_dtype="bf16", kv_dtype="bf16", q_len=5, tree="chain",
                                     ragged=True, ctx=(5, 40), seed=32)))


def _all_parent_arrays(n):
    return itertools.product(*[range(i) for i in range(1, n)])


def test_node_is_path_exhaustive_small_trees():
    """Every parent array of a 5-candidate tree (4! = 24 trees)."""
    base = make(small(B=1, q_len=5, tree="chain", ctx=(40, 40), seed=41))
    for rest in _all_parent_arrays(5):
        par = np.array((-1,) + rest, dtype=np.int32)
        w = make(base.spec)
        w.parents[0] = par
        w.tree_mask[0] = tree_mask_from_parents(par, 5)
        check_node_is_path(w)


def test_node_is_path_sampled_large_trees():
    check_node_is_path(make(small(B=2, q_len=16, depth=6, ctx=(40, 90), seed=42)))
    check_node_is_path(make(small(B=1, q_len=32, depth=8, ctx=(50, 100), seed=43)))


def test_permutation_bit_identical():
    check_permutation_bit_identical(make(small(q_dtype="bf16", kv_dtype="bf16", q_len=4, seed=51)))
    check_permutation_bit_identical(make(small(q_dtype="bf16", kv_dtype="fp8", q_len=3, seed=52)))


@pytest.mark.parametrize("T", [16, 32, 48, 2048])
def test_split_identity(T):
    check_split_identity(make(small(q_len=4, ctx=(30, 140), seed=61)), T)


def test_split_single_partition_equals_unsplit():
    w = make(small(q_len=3, ctx=(20, 40), seed=62))
    s = w.spec
    O, LSE = oracle.paged_tree_attn_partials(w.q, w.k_cache, w.v_cache, w.block_tables, w.ctx_lens,
                                             w.q_lens, w.tree_mask, w.scale, 64, q_dtype=s.q_dtype,
                                             kv_dtype=s.kv_dtype)
    out, lse = run_oracle(w)
    assert O.shape[3] == 1
    assert np.array_equal(O[:, :, :, 0], out, equal_nan=True)
    assert np.array_equal(LSE[..., 0], lse, equal_nan=True)


def test_merge_closed_form():
    """Two partitions with equal LSE average their outputs; lse grows by ln 2."""
    O = np.zeros((1, 1, 1, 2, 3))
    O[0, 0, 0, 0] = [1, 2, 3]
    O[0, 0, 0, 1] = [3, 2, 1]
    LSE = np.array([[[[0.5, 0.5]]]])
    out, lse = oracle.merge_partials(O, LSE)
    assert np.allclose(out[0, 0, 0], [2, 2, 2], atol=1e-15)
    assert abs(lse[0, 0, 0] - (0.5 + math.log(2))) < 1e-15
    LSE = np.array([[[[0.0, -np.inf]]]])
    out, lse = oracle.merge_partials(O, LSE)
    assert np.array_equal(out[0, 0, 0], [1, 2, 3]) and lse[0, 0, 0] == 0.0


def test_closed_forms():
    check_closed_forms(make(small(q_len=4, seed=71)))
    check_constant_v(make(small(q_dtype="bf16", kv_dtype="bf16", q_len=3, seed=72)))


def test_one_hot_probe_exact():
    check_one_hot_probe(make(small(B=2, Hq=4, Hkv=2, D=64, q_len=6, ctx=(20, 60), seed=81)))


def test_mask_probe_exact():
    check_mask_probe(make(small(B=2, Hq=2, Hkv=1, D=32, q_len=12, depth=5, ctx=(20, 60), seed=91)))


def test_gqa_is_replicated_mha():
    check_gqa_is_replicated_mha(make(small(Hq=8, Hkv=2, q_len=3, seed=101)))
    check_gqa_is_replicated_mha(make(small(q_dtype="bf16", kv_dtype="fp8", Hq=8, Hkv=2, q_len=3,
                                           seed=102)))


def test_empty_visibility_row():
    """A candidate with no committed prefix and an all-zero mask row: out 0, lse -inf."""
    w = make(small(B=1, q_len=2, ctx=(2, 2), tree="chain", seed=111))
    w.tree_mask[0, 1, :] = 0
    out, lse = run_oracle(w)
    assert np.array_equal(out[0, 1], np.zeros_like(out[0, 1]))
    assert np.isneginf(lse[0, :, 1]).all()


# ---------------------------------------------------------------- planted mistakes
def _pins_fail(monkeypatch_target, attr, mutant, specs):
    """True if at least one pin raises with the mutant in place."""
    failed = False
    orig = getattr(monkeypatch_target, attr)
    setattr(monkeypatch_target, attr, mutant)
    try:
        for spec in specs:
            w = make(spec)
            for check in (check_bruteforce, check_node_is_path, check_mask_probe, check_one_hot_probe):
                try:
                    check(w)
                except (AssertionError, IndexError, ValueError):
                    failed = True
    finally:
        setattr(monkeypatch_target, attr, orig)
    return failed


MUT_SPECS = [small(q_dtype="bf16", kv_dtype="fp8", Hq=4, Hkv=2, D=16, ctx=(20, 60), q_len=5, seed=5),
             small(Hq=4, Hkv=2, D=16, ctx=(20, 60), q_len=5, seed=6)]


def test_mutant_transposed_mask_is_caught():
    orig = oatt.visibility

    def mut(C, Q, m):
        return orig(C, Q, np.asarray(m).T)
    assert _pins_fail(oatt, "visibility", mut, MUT_SPECS)


def test_mutant_prefix_off_by_one_is_caught():
    def mut(C, Q, m):
        # candidate j placed at L + 1 + j: the mask is applied one position late
        L = C - Q + 1
        vis = np.zeros((Q, C), dtype=bool)
        vis[:, :L] = True
        vis[:, L:] = np.asarray(m)[:Q, :Q - 1] != 0
        return vis
    assert _pins_fail(oatt, "visibility", mut, MUT_SPECS)


def test_mutant_page_slot_swapped_is_caught():
    def mut(cache, row, hk, C, dtype, scales=None, page_size=16):
        t = np.arange(C)
        phys = np.asarray(row)[np.minimum(t % page_size, len(row) - 1)]
        rows = oatt._decode(cache[phys, hk, np.minimum(t // page_size, 15), :], dtype)
        if dtype == "fp8":
            rows = rows * np.asarray(scales, np.float64)[phys, hk][:, None]
        return rows
    assert _pins_fail(oatt, "gather_page_rows", mut, MUT_SPECS)


def test_mutant_fp8_scale_dropped_is_caught():
    orig = oatt.gather_page_rows

    def mut(cache, row, hk, C, dtype, scales=None, page_size=16):
        if dtype == "fp8":
            return oatt._decode(cache[np.asarray(row)[np.arange(C) // 16], hk, np.arange(C) % 16], dtype)
        return orig(cache, row, hk, C, dtype, scales, page_size)
    assert _pins_fail(oatt, "gather_page_rows", mut, MUT_SPECS[:1])


def test_mutant_gqa_map_is_caught():
    assert _pins_fail(oatt, "kv_head_of", lambda h, g: h % 2, [small(Hq=4, Hkv=2, D=16, q_len=3, seed=7)])


def test_mutant_attend_without_normalisation_is_caught():
    orig = oatt._attend

    def mut(s, vis, v):
        o, l = orig(s, vis, v)
        return o * 1.01, l
    assert _pins_fail(oatt, "_attend", mut, MUT_SPECS[1:])
