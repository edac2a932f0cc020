"""GPU parity of the quantized GEMMs (taco_gemm_w8a8, taco_gemm_w4a16; include/pta_gemm.h) against the
fp64 oracle.  W8A8:

Bound per output, from the arithmetic: the products of two e4m3fn values are exact in float32,
the matrix core adds them in float32 (K / 64 accumulator updates), the scales multiply the
float32 sum and the result is rounded to bf16:
    |y - y_ref| <= 2^-8 |y_ref| + 2^-14 * S,   S = a_scale[m] w_scale[n] sum_k |a_mk| |w_nk|
(2^-8 covers the bf16 rounding of the result and of the scale products with room; 2^-14 S is
far above K / 64 float32 roundings of partial sums bounded by S).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from oracle.formats import decode_fp8_e4m3fn
from workload.gemm import LLAMA70B_GATE_UP, make_w8a8

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


def run(torch, g, rows=None):
    import paged_speculative_verify_amd as psv
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = psv.taco_gemm_w8a8(T(g.a_codes), T(g.a_scale), T(g.w_codes), T(g.w_scale))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    return y if rows is None else y[rows]


def check(g, y, rows=None):
    sel = slice(None) if rows is None else rows
    ref = oracle.w8a8_gemm(g.a_codes[sel], g.a_scale[sel], g.w_codes, g.w_scale)
    S = (np.abs(decode_fp8_e4m3fn(g.a_codes[sel])) * g.a_scale[sel].astype(np.float64)[:, None]) @ \
        (np.abs(decode_fp8_e4m3fn(g.w_codes)) * g.w_scale.astype(np.float64)[:, None]).T
    err = np.abs(y - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S
    assert np.isfinite(y).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"
    return float((err / np.maximum(bound, 1e-30)).max())


CASES = [
    ("one_by_one", 1, 1, 64, 31),
    ("ragged_small", 37, 200, 128, 32),
    ("ragged_tiles", 130, 260, 320, 33),
    ("one_tile_long_k", 128, 128, 4096, 34),
    ("many_tiles", 300, 1100, 1024, 35),
    ("tall_three_row_tiles", 520, 600, 512, 37),
    ("decode_rows", 64, 2048, 8192, 36),
]


@pytest.mark.parametrize("cid,M,N,K,seed", CASES, ids=[c[0] for c in CASES])
def test_w8a8_parity(torch_cuda, cid, M, N, K, seed):
    g = make_w8a8(M, N, K, seed=seed)
    say(cid, M, N, K)
    y = run(torch_cuda, g)
    r = check(g, y)
    say(cid, "worst error / bound", r)


@pytest.mark.parametrize("cid,M,N,K,seed", CASES, ids=[c[0] for c in CASES])
def test_w8a8_tiled_equals_row_major(torch_cuda, cid, M, N, K, seed):
    """On weights rearranged by taco_gemm_w8a16_pack the W8A8 GEMM gives exactly the row-major
    entry's output (itself checked against the oracle above), for every tile width, 128-column
    tiles reading one block per stage and 256-column tiles two."""
    import torch
    import paged_speculative_verify_amd as psv
    g = make_w8a8(M, N, K, seed=seed)
    say("w8a8 tiled", cid, M, N, K)
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    a, sa, w, sw = T(g.a_codes), T(g.a_scale), T(g.w_codes), T(g.w_scale)
    y_r = psv.taco_gemm_w8a8(a, sa, w, sw)
    y_t = psv.taco_gemm_w8a8(a, sa, psv.taco_gemm_w8a16_pack(w), sw, tiled=(N, K))
    torch.cuda.synchronize()
    assert torch.equal(y_r.view(torch.int16), y_t.view(torch.int16))


def test_w8a8_full_size_sampled_rows(torch_cuda):
    """The benchmarked shape (Llama-3.1-70B gate+up, 512 verify tokens), sampled rows."""
    s = LLAMA70B_GATE_UP
    g = make_w8a8(s["M"], s["N"], s["K"], seed=7)
    rows = np.array([0, 127, 128, 300, 511])
    say("full size", s, "rows", rows.tolist())
    y = run(torch_cuda, g, rows)
    r = check(g, y, rows)
    say("full size worst error / bound", r)


@pytest.mark.parametrize("M,N,K", [(70, 90, 256), (200, 600, 512)], ids=["narrow_tiles", "wide_tiles"])
def test_w8a8_integer_exact(torch_cuda, M, N, K):
    """Small integers with power-of-two scales: every partial sum is exact in float32, so the
    output is the bf16 rounding of the exact integer result (both tile widths: up to 128 rows
    and beyond)."""
    import torch
    rng = np.random.default_rng(5)
    say("integer exact", M, N, K)
    from tests.test_oracle_gemm import fp8_codes_of
    ai, wi = rng.integers(-4, 5, (M, K)), rng.integers(-4, 5, (N, K))
    sa, sw = (2.0 ** rng.integers(-2, 3, M)).astype(np.float32), (2.0 ** rng.integers(-2, 3, N)).astype(np.float32)
    from workload.gemm import W8A8
    g = W8A8(fp8_codes_of(ai), sa, fp8_codes_of(wi), sw)
    y = run(torch_cuda, g)
    exact = (ai @ wi.T).astype(np.float64) * sa[:, None] * sw[None, :]
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, want)


def test_w8a8_nan_rows(torch_cuda):
    """A NaN code in a row of A makes that output row NaN and leaves the others finite."""
    g = make_w8a8(40, 130, 128, seed=9)
    g.a_codes[3, 17] = 0x7F
    y = run(torch_cuda, g)
    assert np.isnan(y[3]).all()
    assert np.isfinite(np.delete(y, 3, axis=0)).all()


def test_w8a8_argument_checks(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    a = torch.zeros((8, 100), dtype=torch.uint8, device="cuda")        # K not a multiple of 64
    w = torch.zeros((8, 100), dtype=torch.uint8, device="cuda")
    s = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(psv.PtaError):
        psv.taco_gemm_w8a8(a, s, w, s)


# ------------------------------------------------------------------ W4A16
# Bound per output, from the arithmetic: every int4 weight converts exactly to bf16, the products
# bf16 x bf16 are exact in float32, each group's sum is a float32 matrix-core sum of group / 16
# accumulator updates, the group scale multiplies it in float32 and the groups add in float32;
# the result is rounded to bf16:
#     |y - y_ref| <= 2^-8 |y_ref| + 2^-14 * S,   S = sum_k |a_mk| |q_nk| w_scale[n, k / group]
# (the same form as W8A8's: 2^-8 covers the bf16 result, 2^-14 S is far above the float32 sums).
from oracle.formats import decode_bf16  # noqa: E402
from workload.gemm import W4A16, make_w4a16, make_w4a16_device, pack_int4  # noqa: E402


def run4(torch, g, rows=None, tiled=False):
    import paged_speculative_verify_amd as psv
    a = torch.from_numpy(np.ascontiguousarray(g.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(g.w_packed)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(g.w_scale)).cuda()
    if tiled:
        N, K = w.shape[0], w.shape[1] * 2
        y = psv.taco_gemm_w4a16(a, psv.taco_gemm_w4a16_pack(w), s, g.group, tiled=(N, K))
    else:
        y = psv.taco_gemm_w4a16(a, w, s, g.group)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    return y if rows is None else y[rows]


def bound4(a_bits, w_packed, w_scale, group, y):
    """(reference, bound) of W4A16 outputs, column chunk by column chunk (the decoded weights of a
    full-size matrix would not fit in memory at once)."""
    K = a_bits.shape[1]
    A = np.abs(decode_bf16(a_bits))
    ref = np.empty(y.shape)
    S = np.empty(y.shape)
    for c0 in range(0, w_packed.shape[0], 4096):
        c1 = min(c0 + 4096, w_packed.shape[0])
        ref[:, c0:c1] = oracle.w4a16_gemm(a_bits, w_packed[c0:c1], w_scale[c0:c1], group)
        q = np.abs(oracle.decode_int4_packed(w_packed[c0:c1], K)).astype(np.float64)
        S[:, c0:c1] = A @ (q * np.repeat(w_scale[c0:c1].astype(np.float64), group, axis=1)).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def check4(g, y, rows=None):
    sel = slice(None) if rows is None else rows
    ref, bound = bound4(g.a_bits[sel], g.w_packed, g.w_scale, g.group, y)
    err = np.abs(y - ref)
    assert np.isfinite(y).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"
    return float((err / np.maximum(bound, 1e-30)).max())


W4_CASES = [
    ("one_by_one", 1, 1, 64, 64, 41),
    ("ragged_small", 37, 200, 256, 128, 42),
    ("ragged_tall", 130, 260, 384, 128, 43),
    ("group64_tall", 300, 1100, 1024, 64, 44),
    ("single_group", 70, 300, 512, 512, 45),
    ("decode_rows", 64, 2048, 8192, 128, 46),
]


@pytest.mark.parametrize("cid,M,N,K,G,seed", W4_CASES, ids=[c[0] for c in W4_CASES])
def test_w4a16_parity(torch_cuda, cid, M, N, K, G, seed):
    g = make_w4a16(M, N, K, G, seed=seed)
    say(cid, M, N, K, G)
    y = run4(torch_cuda, g)
    r = check4(g, y)
    say(cid, "worst error / bound", r)


def tiled_layout(w_packed):
    """The rearranged weight buffer as include/pta_gemm.h defines it, built with numpy loops over
    its blocks: block (t, s) at byte (t * K / 64 + s) * 4096 holds at byte 32 r + 16 p the 16
    bytes of column 128 t + r at k-bytes 32 s + 16 (p ^ ((r >> 3) & 1)), zero past N."""
    N, KB = w_packed.shape
    K = 2 * KB
    T, S = (N + 127) // 128, K // 64
    out = np.zeros(T * S * 4096, np.uint8)
    for t in range(T):
        for st in range(S):
            blk = out[(t * S + st) * 4096:(t * S + st + 1) * 4096].reshape(128, 2, 16)
            for r in range(128):
                n = 128 * t + r
                if n >= N:
                    continue
                for p in range(2):
                    u = p ^ ((r >> 3) & 1)
                    blk[r, p] = w_packed[n, 32 * st + 16 * u:32 * st + 16 * u + 16]
    return out


@pytest.mark.parametrize("cid,M,N,K,G,seed", W4_CASES[:5], ids=[c[0] for c in W4_CASES[:5]])
def test_w4a16_tiled_parity(torch_cuda, cid, M, N, K, G, seed):
    """The rearranged weights match the header's layout byte for byte, and the GEMM on them
    gives exactly the row-major GEMM's output (itself checked against the oracle above) and
    stays within the oracle's bound."""
    import torch
    import paged_speculative_verify_amd as psv
    g = make_w4a16(M, N, K, G, seed=seed)
    say("tiled", cid, M, N, K, G)
    w = torch.from_numpy(np.ascontiguousarray(g.w_packed)).cuda()
    wt = psv.taco_gemm_w4a16_pack(w)
    torch.cuda.synchronize()
    assert np.array_equal(wt.cpu().numpy(), tiled_layout(g.w_packed))
    y_t = run4(torch_cuda, g, tiled=True)
    y_r = run4(torch_cuda, g)
    assert np.array_equal(y_t, y_r)
    check4(g, y_t)


def test_w4a16_tiled_full_size(torch_cuda):
    """The timed shape (512 x 57344 x 8192, group 128) on rearranged weights: the whole output
    equals the row-major GEMM's bit for bit."""
    import torch
    import paged_speculative_verify_amd as psv
    s = LLAMA70B_GATE_UP
    M, N, K, G = s["M"], s["N"], s["K"], 128
    a, w, sc = make_w4a16_device(M, N, K, G, seed=8, torch=torch)
    say("tiled full size", s)
    y_r = psv.taco_gemm_w4a16(a, w, sc, G)
    y_t = psv.taco_gemm_w4a16(a, psv.taco_gemm_w4a16_pack(w), sc, G, tiled=(N, K))
    torch.cuda.synchronize()
    assert torch.equal(y_r.view(torch.int16), y_t.view(torch.int16))


def test_w4a16_full_size_sampled_rows(torch_cuda):
    """Llama-3.1-70B gate+up at the verify step's 512 rows, group 128 (the timed shape): operands
    drawn on the GPU, rows spanning both tile rows checked against the oracle."""
    import torch
    import paged_speculative_verify_amd as psv
    s = LLAMA70B_GATE_UP
    M, N, K, G = s["M"], s["N"], s["K"], 128
    a, w, sc = make_w4a16_device(M, N, K, G, seed=7, torch=torch)
    rows = np.array([0, 127, 128, 300, 511])
    say("full size", s, "group", G, "rows", rows.tolist())
    y = psv.taco_gemm_w4a16(a, w, sc, G)
    torch.cuda.synchronize()
    yr = y.float().cpu().numpy().astype(np.float64)[rows]
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref, bound = bound4(a_bits, w.cpu().numpy(), sc.cpu().numpy(), G, yr)
    err = np.abs(yr - ref)
    assert np.isfinite(yr).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"


@pytest.mark.parametrize("M,N,K,G", [(40, 90, 256, 128), (200, 300, 512, 64)], ids=["short_rows", "tall_rows"])
def test_w4a16_integer_exact(torch_cuda, M, N, K, G):
    """Small integer activations and power-of-two group scales: every product, group sum, scaled
    group and total is exact in float32, so the output is the bf16 rounding of the exact result."""
    import torch
    rng = np.random.default_rng(11)
    ai = rng.integers(-4, 5, (M, K))
    q = rng.integers(-8, 8, (N, K))
    sc = (2.0 ** rng.integers(-3, 3, (N, K // G))).astype(np.float32)
    from workload.gemm import bf16_bits_of
    g = W4A16(bf16_bits_of(ai.astype(np.float32)), pack_int4(q), sc, G)
    say("integer exact", M, N, K, G)
    y = run4(torch_cuda, g)
    exact = ai.astype(np.float64) @ (q.astype(np.float64) * np.repeat(sc.astype(np.float64), G, axis=1)).T
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, want)


def test_w4a16_nan_rows(torch_cuda):
    """A NaN activation makes its output row NaN and leaves the others finite."""
    g = make_w4a16(40, 130, 256, 128, seed=9)
    g.a_bits[3, 17] = 0x7FC0
    y = run4(torch_cuda, g)
    assert np.isnan(y[3]).all()
    assert np.isfinite(np.delete(y, 3, axis=0)).all()


def test_w4a16_argument_checks(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    a = torch.zeros((8, 192), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 96), dtype=torch.uint8, device="cuda")
    s = torch.ones((8, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(psv.PtaError):                     # group 32: not a multiple of 64
        psv.taco_gemm_w4a16(a, w, torch.ones((8, 6), dtype=torch.float32, device="cuda"), 32)
    y = psv.taco_gemm_w4a16(a, w, s, 64)                  # K = 192, group 64: served
    torch.cuda.synchronize()
    assert float(y.float().abs().max()) == 0.0
    with pytest.raises(ValueError):
        psv.taco_gemm_w4a16(a, w, s, 128)                 # 128 does not divide 192


# ------------------------------------------------------------------ W8A16
# Bound per output, from the arithmetic: every e4m3fn weight decodes exactly to bf16, the products
# bf16 x bf16 are exact in float32, the matrix core sums them in float32, the channel scale
# multiplies the float32 sum and the result is rounded to bf16:
#     |y - y_ref| <= 2^-8 |y_ref| + 2^-14 * S,   S = w_scale[n] sum_k |a_mk| |w_nk|
# (the W8A8 form: 2^-8 covers the bf16 result, 2^-14 S is far above the float32 sums).
from workload.gemm import W8A16, make_w8a16, make_w8a16_device  # noqa: E402


def run8(torch, g, rows=None, tiled=False):
    import paged_speculative_verify_amd as psv
    a = torch.from_numpy(np.ascontiguousarray(g.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(g.w_codes)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(g.w_scale)).cuda()
    if tiled:
        y = psv.taco_gemm_w8a16(a, psv.taco_gemm_w8a16_pack(w), s, tiled=tuple(w.shape))
    else:
        y = psv.taco_gemm_w8a16(a, w, s)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    return y if rows is None else y[rows]


def bound8(a_bits, w_codes, w_scale, y):
    """(reference, bound) of W8A16 outputs, column chunk by column chunk."""
    A = np.abs(decode_bf16(a_bits))
    ref = np.empty(y.shape)
    S = np.empty(y.shape)
    for c0 in range(0, w_codes.shape[0], 4096):
        c1 = min(c0 + 4096, w_codes.shape[0])
        ref[:, c0:c1] = oracle.w8a16_gemm(a_bits, w_codes[c0:c1], w_scale[c0:c1])
        S[:, c0:c1] = A @ (np.abs(decode_fp8_e4m3fn(w_codes[c0:c1])) *
                           w_scale[c0:c1].astype(np.float64)[:, None]).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def check8(g, y, rows=None):
    sel = slice(None) if rows is None else rows
    ref, bound = bound8(g.a_bits[sel], g.w_codes, g.w_scale, y)
    err = np.abs(y - ref)
    assert np.isfinite(y).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"
    return float((err / np.maximum(bound, 1e-30)).max())


W8_CASES = [
    ("one_by_one", 1, 1, 64, 51),
    ("ragged_small", 37, 200, 128, 52),
    ("ragged_tall", 130, 260, 384, 53),
    ("many_tiles", 300, 1100, 1024, 54),
    ("decode_rows", 64, 2048, 8192, 55),
]


@pytest.mark.parametrize("cid,M,N,K,seed", W8_CASES, ids=[c[0] for c in W8_CASES])
def test_w8a16_parity(torch_cuda, cid, M, N, K, seed):
    g = make_w8a16(M, N, K, seed=seed)
    say("w8a16", cid, M, N, K)
    y = run8(torch_cuda, g)
    r = check8(g, y)
    say("w8a16", cid, "worst error / bound", r)


def tiled_layout8(w_codes):
    """The rearranged W8A16 buffer as include/pta_gemm.h defines it, built with numpy loops over
    its blocks: block (t, s) at byte (t * K / 64 + s) * 8192 holds at byte 64 r + 16 p the 16
    bytes of column 128 t + r at k-bytes 64 s + 16 (p ^ ((r >> 2) & 3)), zero past N."""
    N, K = w_codes.shape
    T, S = (N + 127) // 128, K // 64
    out = np.zeros(T * S * 8192, np.uint8)
    for t in range(T):
        for st in range(S):
            blk = out[(t * S + st) * 8192:(t * S + st + 1) * 8192].reshape(128, 4, 16)
            for r in range(128):
                n = 128 * t + r
                if n >= N:
                    continue
                for p in range(4):
                    u = p ^ ((r >> 2) & 3)
                    blk[r, p] = w_codes[n, 64 * st + 16 * u:64 * st + 16 * u + 16]
    return out


@pytest.mark.parametrize("cid,M,N,K,seed", W8_CASES[:4], ids=[c[0] for c in W8_CASES[:4]])
def test_w8a16_tiled_parity(torch_cuda, cid, M, N, K, seed):
    """The rearranged weights match the header's layout byte for byte, and the GEMM on them
    gives exactly the row-major GEMM's output and stays within the oracle's bound."""
    import torch
    import paged_speculative_verify_amd as psv
    g = make_w8a16(M, N, K, seed=seed)
    say("w8a16 tiled", cid, M, N, K)
    wt = psv.taco_gemm_w8a16_pack(torch.from_numpy(np.ascontiguousarray(g.w_codes)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(wt.cpu().numpy(), tiled_layout8(g.w_codes))
    y_t = run8(torch_cuda, g, tiled=True)
    y_r = run8(torch_cuda, g)
    assert np.array_equal(y_t, y_r)
    check8(g, y_t)


def test_w8a16_full_size_sampled_rows(torch_cuda):
    """Llama-3.1-70B gate+up at the verify step's 512 rows (the timed shape): operands drawn on
    the GPU, rows spanning both row tiles and the ragged-free edge checked against the oracle."""
    import torch
    import paged_speculative_verify_amd as psv
    s = LLAMA70B_GATE_UP
    M, N, K = s["M"], s["N"], s["K"]
    a, w, sc = make_w8a16_device(M, N, K, seed=7, torch=torch)
    rows = np.array([0, 127, 128, 300, 511])
    say("w8a16 full size", s, "rows", rows.tolist())
    y = psv.taco_gemm_w8a16(a, w, sc)
    y_t = psv.taco_gemm_w8a16(a, psv.taco_gemm_w8a16_pack(w), sc, tiled=(N, K))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_t.view(torch.int16))     # the timed layout, whole output
    yr = y.float().cpu().numpy().astype(np.float64)[rows]
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref, bound = bound8(a_bits, w.cpu().numpy(), sc.cpu().numpy(), yr)
    err = np.abs(yr - ref)
    assert np.isfinite(yr).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"


@pytest.mark.parametrize("M,N,K", [(40, 90, 256), (200, 300, 512)], ids=["short_rows", "tall_rows"])
def test_w8a16_integer_exact(torch_cuda, M, N, K):
    """Small integer activations and weights with power-of-two channel scales: every product and
    partial sum is exact in float32, so the output is the bf16 rounding of the exact result."""
    import torch
    from tests.test_oracle_gemm import fp8_codes_of
    from workload.gemm import bf16_bits_of
    rng = np.random.default_rng(12)
    ai, wi = rng.integers(-4, 5, (M, K)), rng.integers(-4, 5, (N, K))
    sc = (2.0 ** rng.integers(-3, 3, N)).astype(np.float32)
    g = W8A16(bf16_bits_of(ai.astype(np.float32)), fp8_codes_of(wi), sc)
    say("w8a16 integer exact", M, N, K)
    y = run8(torch_cuda, g)
    exact = (ai @ wi.T).astype(np.float64) * sc[None, :].astype(np.float64)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, want)


def test_w8a16_nan_rows_and_columns(torch_cuda):
    """A NaN activation makes its output row NaN, a NaN weight code its output column; the other
    outputs stay finite."""
    g = make_w8a16(40, 130, 256, seed=13)
    g.a_bits[3, 17] = 0x7FC0
    g.w_codes[100, 200] = 0x7F
    y = run8(torch_cuda, g)
    assert np.isnan(y[3]).all() and np.isnan(y[:, 100]).all()
    rest = np.delete(np.delete(y, 3, axis=0), 100, axis=1)
    assert np.isfinite(rest).all()


def test_w8a16_argument_checks(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    a = torch.zeros((8, 100), dtype=torch.bfloat16, device="cuda")      # K not a multiple of 64
    w = torch.zeros((8, 100), dtype=torch.uint8, device="cuda")
    s = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(psv.PtaError):
        psv.taco_gemm_w8a16(a, w, s)
    with pytest.raises(ValueError):
        psv.taco_gemm_w8a16(a[:, :64].contiguous(), w[:, :64].contiguous(), s[:4].contiguous())


# ------------------------------------------------------------------ W4A8
# Bound per output, from the arithmetic: each group's products sum exactly in int32 (the weights
# widen exactly to int8), the group scale multiplies the group sum in float32, the groups add in
# float32, the activation scale multiplies the total and the result is rounded to bf16:
#     |y - y_ref| <= 2^-8 |y_ref| + 2^-14 * S,   S = a_scale[m] sum_k |a_mk| |q_nk| w_scale[n, k / group]
from workload.gemm import W4A8, make_w4a8, make_w4a8_device  # noqa: E402


def run48(torch, g, rows=None, tiled=False):
    import paged_speculative_verify_amd as psv
    a = torch.from_numpy(np.ascontiguousarray(g.a_codes).view(np.int8)).cuda()
    sa = torch.from_numpy(np.ascontiguousarray(g.a_scale)).cuda()
    w = torch.from_numpy(np.ascontiguousarray(g.w_packed)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(g.w_scale)).cuda()
    if tiled:
        N, K = w.shape[0], w.shape[1] * 2
        y = psv.taco_gemm_w4a8(a, sa, psv.taco_gemm_w4a16_pack(w), s, g.group, tiled=(N, K))
    else:
        y = psv.taco_gemm_w4a8(a, sa, w, s, g.group)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    return y if rows is None else y[rows]


def bound48(a_codes, a_scale, w_packed, w_scale, group, y):
    """(reference, bound) of W4A8 outputs, column chunk by column chunk."""
    K = a_codes.shape[1]
    A = np.abs(np.asarray(a_codes).view(np.int8).astype(np.float64)) * np.asarray(a_scale, np.float64)[:, None]
    ref = np.empty(y.shape)
    S = np.empty(y.shape)
    for c0 in range(0, w_packed.shape[0], 4096):
        c1 = min(c0 + 4096, w_packed.shape[0])
        ref[:, c0:c1] = oracle.w4a8_gemm(a_codes, a_scale, w_packed[c0:c1], w_scale[c0:c1], group)
        q = np.abs(oracle.decode_int4_packed(w_packed[c0:c1], K)).astype(np.float64)
        S[:, c0:c1] = A @ (q * np.repeat(w_scale[c0:c1].astype(np.float64), group, axis=1)).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def check48(g, y, rows=None):
    sel = slice(None) if rows is None else rows
    ref, bound = bound48(g.a_codes[sel], g.a_scale[sel], g.w_packed, g.w_scale, g.group, y)
    err = np.abs(y - ref)
    assert np.isfinite(y).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"
    return float((err / np.maximum(bound, 1e-30)).max())


W48_CASES = [
    ("one_by_one", 1, 1, 64, 64, 61),
    ("ragged_small", 37, 200, 256, 128, 62),
    ("ragged_tall", 130, 260, 384, 128, 63),
    ("group64_tall", 300, 1100, 1024, 64, 64),
    ("single_group", 70, 300, 512, 512, 65),
    ("decode_rows", 64, 2048, 8192, 128, 66),
]


@pytest.mark.parametrize("cid,M,N,K,G,seed", W48_CASES, ids=[c[0] for c in W48_CASES])
def test_w4a8_parity(torch_cuda, cid, M, N, K, G, seed):
    g = make_w4a8(M, N, K, G, seed=seed)
    say("w4a8", cid, M, N, K, G)
    y = run48(torch_cuda, g)
    r = check48(g, y)
    say("w4a8", cid, "worst error / bound", r)


@pytest.mark.parametrize("cid,M,N,K,G,seed", W48_CASES[:5], ids=[c[0] for c in W48_CASES[:5]])
def test_w4a8_tiled_parity(torch_cuda, cid, M, N, K, G, seed):
    """On weights rearranged by taco_gemm_w4a16_pack the W4A8 GEMM gives exactly the row-major
    GEMM's output (itself checked against the oracle above) and stays within the oracle's bound."""
    g = make_w4a8(M, N, K, G, seed=seed)
    say("w4a8 tiled", cid, M, N, K, G)
    y_t = run48(torch_cuda, g, tiled=True)
    y_r = run48(torch_cuda, g)
    assert np.array_equal(y_t, y_r)
    check48(g, y_t)


def test_w4a8_full_size_sampled_rows(torch_cuda):
    """Llama-3.1-70B gate+up at the verify step's 512 rows, group 128 (the timed shape): operands
    drawn on the GPU, rows spanning both row tiles checked against the oracle."""
    import torch
    import paged_speculative_verify_amd as psv
    s = LLAMA70B_GATE_UP
    M, N, K, G = s["M"], s["N"], s["K"], 128
    a, sa, w, sc = make_w4a8_device(M, N, K, G, seed=7, torch=torch)
    rows = np.array([0, 127, 128, 300, 511])
    say("w4a8 full size", s, "group", G, "rows", rows.tolist())
    y = psv.taco_gemm_w4a8(a, sa, w, sc, G)
    y_t = psv.taco_gemm_w4a8(a, sa, psv.taco_gemm_w4a16_pack(w), sc, G, tiled=(N, K))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_t.view(torch.int16))     # the timed layout, whole output
    yr = y.float().cpu().numpy().astype(np.float64)[rows]
    ac = a.cpu().numpy().view(np.uint8)[rows]
    ref, bound = bound48(ac, sa.cpu().numpy()[rows], w.cpu().numpy(), sc.cpu().numpy(), G, yr)
    err = np.abs(yr - ref)
    assert np.isfinite(yr).all()
    assert (err <= bound).all(), f"worst excess {float((err - bound).max())}"


@pytest.mark.parametrize("M,N,K,G", [(40, 90, 256, 128), (200, 300, 512, 64)], ids=["short_rows", "tall_rows"])
def test_w4a8_integer_exact(torch_cuda, M, N, K, G):
    """Full-range int8 activations (-128 included), every int4 code, power-of-two scales: every
    group sum is exact in int32 and every scaled sum exact in float32, so the output is the bf16
    rounding of the exact result."""
    import torch
    from workload.gemm import pack_int4
    rng = np.random.default_rng(14)
    ai = rng.integers(-128, 128, (M, K))
    q = rng.integers(-8, 8, (N, K))
    sa = (2.0 ** rng.integers(-3, 3, M)).astype(np.float32)
    sc = (2.0 ** rng.integers(-3, 3, (N, K // G))).astype(np.float32)
    g = W4A8(ai.astype(np.int8).view(np.uint8), sa, pack_int4(q), sc, G)
    say("w4a8 integer exact", M, N, K, G)
    y = run48(torch_cuda, g)
    exact = np.zeros((M, N))
    for gi in range(K // G):
        ks = slice(gi * G, (gi + 1) * G)
        exact += (ai[:, ks] @ q[:, ks].T).astype(np.float64) * sc[None, :, gi].astype(np.float64)
    exact *= sa[:, None].astype(np.float64)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, want)


def test_w4a8_argument_checks(torch_cuda):
    import torch
    import paged_speculative_verify_amd as psv
    a = torch.zeros((8, 192), dtype=torch.int8, device="cuda")
    sa = torch.ones(8, dtype=torch.float32, device="cuda")
    w = torch.zeros((8, 96), dtype=torch.uint8, device="cuda")
    s = torch.ones((8, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(psv.PtaError):                     # group 32: not a multiple of 64
        psv.taco_gemm_w4a8(a, sa, w, torch.ones((8, 6), dtype=torch.float32, device="cuda"), 32)
    y = psv.taco_gemm_w4a8(a, sa, w, s, 64)               # K = 192, group 64: served
    torch.cuda.synchronize()
    assert float(y.float().abs().max()) == 0.0
    with pytest.raises(ValueError):
        psv.taco_gemm_w4a8(a.to(torch.bfloat16), sa, w, s, 64)
