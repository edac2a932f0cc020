"""CPU pins for the oracle's KV append and the pages' printed formulas."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests import golden, refs
from workload import Spec, make
from workload.gen import f32_to_bf16_bits


def test_decode_roofline_golden():
    g = golden.load("decode_roofline_a100.txt")
    io, comp = oracle.decode_io_compute_ms(g["params"], g["bytes_per_param"], g["hbm_bytes_per_s"],
                                           g["peak_flop_per_s"])
    assert abs(io - g["io_ms"]) <= g["io_ms_tol"]
    assert abs(comp - g["compute_ms"]) <= g["compute_ms_tol"]


def test_lookahead_speedup_golden():
    g = golden.load("lookahead_speedup.txt")
    s = oracle.lookahead_speedup(g["ceiling"], int(g["lookahead"]), g["accepted"])
    assert abs(s - g["speedup"]) <= g["speedup_tol"]


def _append_case(kv_dtype, new_dtype, seed=0):
    spec = Spec("ap", 3, 4, 2, 32, "bf16" if kv_dtype != "f32" else "f32", kv_dtype,
                ctx_range=(10, 60), q_len=4, tree="chain", seed=seed)
    w = make(spec)
    rng = np.random.default_rng(seed + 100)
    # new tokens: the last q_b logical positions of every sequence, plus one skipped slot
    pos = [(b, int(w.ctx_lens[b]) - int(w.q_lens[b]) + j) for b in range(3) for j in range(int(w.q_lens[b]))]
    slots = np.array([w.block_tables[b, t // 16] * 16 + t % 16 for b, t in pos] + [-1], dtype=np.int64)
    N = len(slots)
    x = rng.standard_normal((N, 2, 32)).astype(np.float32) * 3
    new = x if new_dtype == "f32" else f32_to_bf16_bits(x)
    return w, pos, slots, new


def test_kv_append_copy_exact():
    for dt in ("f32", "bf16"):
        w, pos, slots, new = _append_case(dt, dt)
        k2, v2 = oracle.kv_append(w.k_cache, w.v_cache, new, new[:, ::-1], slots, cache_dtype=dt,
                                  new_dtype=dt)
        for n, (b, t) in enumerate(pos):
            K = refs.unpage(k2, w.block_tables[b], int(w.ctx_lens[b]), dt)
            V = refs.unpage(v2, w.block_tables[b], int(w.ctx_lens[b]), dt)
            assert np.array_equal(K[:, t], refs.torch_decode(new[n], dt))
            assert np.array_equal(V[:, t], refs.torch_decode(new[n, ::-1], dt))
        # everything else untouched
        touched = np.zeros(w.k_cache.shape[0] * 16, bool)
        touched[slots[slots >= 0]] = True
        flat_old = w.k_cache.transpose(0, 2, 1, 3).reshape(-1, 2, 32)
        flat_new = k2.transpose(0, 2, 1, 3).reshape(-1, 2, 32)
        assert np.array_equal(flat_old[~touched].view(np.uint8), flat_new[~touched].view(np.uint8))


def test_kv_append_fp8_matches_library_cast():
    for new_dt in ("bf16", "f32"):
        w, pos, slots, new = _append_case("fp8", new_dt, seed=3)
        w.k_scale[...] = np.float32(0.0173)
        w.v_scale[...] = np.float32(0.5)
        k2, v2 = oracle.kv_append(w.k_cache, w.v_cache, new, new, slots, cache_dtype="fp8",
                                  new_dtype=new_dt, k_scale=w.k_scale, v_scale=w.v_scale)
        xs = refs.torch_decode(new, new_dt).astype(np.float32)
        for cache, scl in ((k2, 0.0173), (v2, 0.5)):
            quot = np.clip(xs / np.float32(scl), -448, 448).astype(np.float32)
            lib = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            for n, (b, t) in enumerate(pos):
                got = cache[w.block_tables[b, t // 16], :, t % 16, :]
                assert np.array_equal(got, lib[n])
