"""The allocation-free balanced entry (taco_paged_tree_attn_balanced_noalloc, for callers that
cannot allocate device memory) called through the C ABI with ctypes.

Two calls in a row per kernel family, the second on a smaller input than the first, so the
second call runs on a scratch array that still holds the first call's partials.  Each output must
be bit-identical to taco_paged_tree_attn_balanced with a caller workspace (same kernels, same
slices) and within the oracle tolerance.  A request whose workspace exceeds the scratch array
fails with PTA_ERR_WORKSPACE_TOO_SMALL before anything is launched.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import oracle
from workload import Spec, make
from workload.device import out_to_f64, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 3e-2}


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


def noalloc_c(torch, d, out, lse):
    """taco_paged_tree_attn_balanced_noalloc through the raw C symbol."""
    import paged_speculative_verify_amd as psv
    lib = psv.load()
    dims = psv.make_dims(d.q, d.k_cache, d.block_tables, d.max_ctx_len)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.taco_paged_tree_attn_balanced_noalloc(
        ctypes.byref(dims), p(d.q), p(d.k_cache), p(d.v_cache), p(d.k_scale), p(d.v_scale), p(d.block_tables),
        p(d.ctx_lens), p(d.q_lens), p(d.tree_mask), ctypes.c_float(d.scale), p(out), p(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def both(torch, w):
    """(out, lse) of the noalloc entry and of the workspace entry on the same inputs."""
    import paged_speculative_verify_amd as psv
    d = to_device(w)
    B, Qmax, Hq, D = w.q.shape
    res = []
    for which in ("noalloc", "workspace"):
        out = torch.full_like(d.q, float("nan"))
        lse = torch.full((B, Hq, Qmax), float("nan"), dtype=torch.float32, device=d.q.device)
        if which == "noalloc":
            assert noalloc_c(torch, d, out, lse) == 0
        else:
            psv.taco_paged_tree_attn_balanced(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens,
                                              d.tree_mask, d.scale, out=out, lse=lse, k_scale=d.k_scale,
                                              v_scale=d.v_scale, max_ctx_len=d.max_ctx_len)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def check(torch, w, cid):
    (o1, l1), (o2, l2) = both(torch, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "out differs from the workspace entry"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs from the workspace entry"
    s = w.spec
    ref, _ = oracle.paged_tree_attn(w.q, w.k_cache, w.v_cache, w.block_tables, w.ctx_lens, w.q_lens, w.tree_mask,
                                    w.scale, q_dtype=s.q_dtype, kv_dtype=s.kv_dtype, k_scale=w.k_scale,
                                    v_scale=w.v_scale)
    out = out_to_f64(o1)
    v = ~np.isnan(ref)
    assert np.isnan(out[~v]).all(), "padding rows were written"
    err = float(np.abs(out[v] - ref[v]).max())
    key = "fp8" if s.kv_dtype == "fp8" else "bf16"
    assert err <= TOL[key], f"{cid}: max abs err {err}"
    say(cid, "bit-identical to the workspace entry; max abs err vs oracle", err)


# (family, first call, second call on a smaller input)
PAIRS = [
    ("tile_tree16",
     Spec("na", 12, 64, 8, 128, "bf16", "bf16", ctx_range=(300, 3000), q_len=16, tree="random", depth_cap=6,
          seed=301),
     Spec("na", 5, 64, 8, 128, "bf16", "bf16", ctx_range=(20, 700), q_len=8, q_len_ragged=True, tree="random",
          seed=302)),
    ("stream_decode",
     Spec("na", 40, 32, 8, 128, "bf16", "bf16", ctx_range=(100, 4000), q_len=1, tree="chain", seed=303),
     Spec("na", 7, 32, 8, 128, "bf16", "bf16", ctx_range=(1, 300), q_len=1, tree="chain", seed=304)),
    ("stream_fp8_chain8",
     Spec("na", 24, 32, 8, 128, "bf16", "fp8", ctx_range=(200, 3000), q_len=8, tree="chain", seed=305),
     Spec("na", 6, 32, 8, 128, "bf16", "fp8", ctx_range=(8, 400), q_len=8, tree="chain", seed=306)),
]


@pytest.mark.parametrize("cid,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_two_calls_in_a_row(torch_cuda, cid, first, second):
    w1, w2 = make(first, poison=True), make(second, poison=True)
    say(cid, "first call B", w1.q.shape[0], "then B", w2.q.shape[0])
    check(torch_cuda, w1, cid + " first")
    check(torch_cuda, w2, cid + " second (smaller)")


def test_noalloc_rejects_workspace_beyond_scratch(torch_cuda):
    """100 sequences x 8 KV heads of 128 rows: the balanced workspace exceeds the scratch array,
    so the call fails on the host with PTA_ERR_WORKSPACE_TOO_SMALL (real inputs all the same)."""
    import paged_speculative_verify_amd as psv
    w = make(Spec("na", 100, 64, 8, 128, "bf16", "bf16", ctx_range=(16, 64), q_len=16, tree="random", seed=307))
    d = to_device(w)
    need = psv.taco_paged_tree_attn_balanced_workspace_size(d.q, d.k_cache, d.block_tables,
                                                            max_ctx_len=d.max_ctx_len)
    assert need > psv.NOALLOC_SCRATCH_BYTES
    out = torch_cuda.full_like(d.q, float("nan"))
    assert noalloc_c(torch_cuda, d, out, None) == 5          # PTA_ERR_WORKSPACE_TOO_SMALL
    torch_cuda.cuda.synchronize()
    assert torch_cuda.isnan(out).all(), "nothing may be written"
    with pytest.raises(psv.PtaError):
        psv.taco_paged_tree_attn_balanced_noalloc(d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens,
                                                  d.q_lens, d.tree_mask, d.scale, out=out,
                                                  max_ctx_len=d.max_ctx_len)
