"""GPU parity of the W8A8 GEMM (taco_gemm_w8a8, include/pta_gemm.h) against the fp64 oracle.

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
    ("decode_rows", 64, 2048, 8192, 36),
]


@pytest.mark.parametrize("cid,M,N,K,seed", CASES, ids=[c[0] for c in CASES])
def test_w8a8_parity(torch_cuda, cid, M, N, K, seed):
    g = make_w8a8(M, N, K, seed=seed)
    say(cid, M, N, K)
    y = run(torch_cuda, g)
    r = check(g, y)
    say(cid, "worst error / bound", r)


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
