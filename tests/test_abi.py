"""C-ABI checks that need no GPU: the library loads, exports every function
include/pta.h declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes."""
from __future__ import annotations

import ctypes

import pytest

import paged_speculative_verify_amd as psv
from paged_speculative_verify_amd._lib import PtaDims

OK, NULLP, DIMS, DTYPE, UNSUP, WS = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails host checks


@pytest.fixture(scope="module")
def lib():
    return psv.load()


def dims(**kw):
    base = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, max_q_len=1,
                max_blocks_per_seq=256, max_ctx_len=4096, num_blocks=20000, q_dtype=1, kv_dtype=1,
                path=0, flags=0)
    base.update(kw)
    return PtaDims(**base)


def attn(lib, d, mask=FAKE, ks=None, vs=None, out=FAKE, scale=0.1):
    return lib.taco_paged_tree_attn(ctypes.byref(d) if d is not None else None, FAKE, FAKE, FAKE, ks, vs,
                                    FAKE, FAKE, FAKE, mask, scale, out, None, None)


def test_exports_every_declared_function(lib):
    names = psv.declared_functions()
    assert set(names) >= {"taco_paged_tree_attn", "taco_paged_tree_attn_splitk",
                          "taco_paged_tree_attn_splitk_workspace_size", "taco_kv_append",
                          "taco_pta_validate", "taco_pta_status_string", "taco_pta_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert psv.taco_pta_version() == 100
    for st in range(7):
        assert psv.taco_pta_status_string(st)
    assert psv.taco_pta_status_string(99) == "unknown status"


def test_dims_struct_layout():
    assert ctypes.sizeof(PtaDims) == 56
    assert PtaDims.num_blocks.offset == 32


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), DIMS),                 # Hq % Hkv != 0
    (dict(head_dim=96), DIMS),
    (dict(page_size=32), DIMS),
    (dict(max_q_len=0), DIMS),
    (dict(max_q_len=65), DIMS),
    (dict(max_ctx_len=4097), DIMS),               # > page * max_blocks
    (dict(num_blocks=0), DIMS),
    (dict(num_seqs=-1), DIMS),
    (dict(flags=2), DIMS),                        # only PTA_FLAG_SHARED_PAGES is defined
    (dict(num_seqs=0, flags=1), OK),
    (dict(path=5), DIMS),                        # past PTA_PATH_TILE16
    (dict(q_dtype=0, kv_dtype=0, path=3), UNSUP),  # the shared-tile family needs bf16 q
    (dict(q_dtype=0, kv_dtype=1), DTYPE),         # fp32 q with bf16 KV
    (dict(q_dtype=0, kv_dtype=2), DTYPE),
    (dict(q_dtype=2, kv_dtype=2), DTYPE),
    (dict(q_dtype=0, kv_dtype=0, path=2), UNSUP),  # MFMA needs bf16 q
    (dict(max_q_len=16, num_q_heads=64, path=1), UNSUP),   # 128 rows on the VALU path
    (dict(max_q_len=64, num_q_heads=64), UNSUP),   # 512 rows per KV head
])
def test_host_validation(lib, kw, status):
    assert attn(lib, dims(**kw)) == status


def test_null_pointers(lib):
    assert attn(lib, None) == NULLP
    assert attn(lib, dims(), out=None) == NULLP
    assert attn(lib, dims(max_q_len=4), mask=None) == NULLP
    assert attn(lib, dims(kv_dtype=2)) == NULLP                    # fp8 without scales
    assert attn(lib, dims(), scale=float("nan")) == DIMS


def test_zero_batch_is_a_noop(lib):
    assert attn(lib, dims(num_seqs=0)) == OK


def test_splitk_workspace(lib):
    d = dims(num_seqs=4, max_q_len=32, num_q_heads=64, max_ctx_len=131072, max_blocks_per_seq=8192)
    n = lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(d), 2048)
    rows = 4 * 64 * 32 * 64
    assert n >= rows * 129 * 4 and n % 256 == 0
    assert lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(d), 100) == 0   # not a multiple of 32
    assert lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims(head_dim=80)), 2048) == 0
    st = lib.taco_paged_tree_attn_splitk(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                         FAKE, 0.1, FAKE, None, 2048, FAKE, n - 1, None)
    assert st == WS
    st = lib.taco_paged_tree_attn_splitk(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                         FAKE, 0.1, FAKE, None, 2048, None, n, None)
    assert st == NULLP
    st = lib.taco_paged_tree_attn_splitk(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                         FAKE, 0.1, FAKE, None, 48, FAKE, n, None)
    assert st == DIMS


def test_kv_append_validation(lib):
    d = dims()
    f = lambda new_dt, n=8, dd=d, **kw: lib.taco_kv_append(
        ctypes.byref(dd), kw.get("k", FAKE), FAKE, new_dt, FAKE, n, FAKE, FAKE,
        kw.get("ks"), kw.get("vs"), None)
    assert f(0) == DTYPE            # f32 rows into a bf16 cache
    assert f(1, n=-1) == DIMS
    assert f(1, n=0) == OK
    assert f(1, k=None) == NULLP
    assert f(1, dd=dims(kv_dtype=2)) == NULLP     # fp8 cache without scales
    assert f(1, dd=dims(head_dim=32)) == DIMS


def test_validate_host_checks(lib):
    assert lib.taco_pta_validate(ctypes.byref(dims()), FAKE, FAKE, FAKE, None, None) == NULLP
    assert lib.taco_pta_validate(ctypes.byref(dims(page_size=8)), FAKE, FAKE, FAKE, FAKE, None) == DIMS


def test_accept_commit_host_checks(lib):
    f = lambda dd, **kw: lib.taco_accept_commit(
        None if dd is None else ctypes.byref(dd), kw.get("cand", FAKE), FAKE, FAKE, FAKE, FAKE,
        kw.get("mask", FAKE), FAKE, FAKE, FAKE, kw.get("ks"), kw.get("vs"), FAKE, FAKE, FAKE,
        kw.get("ctx", FAKE), None)
    assert f(None) == NULLP
    assert f(dims(num_seqs=0)) == OK
    assert f(dims(), cand=None) == NULLP
    assert f(dims(), ctx=None) == NULLP
    assert f(dims(max_q_len=4), mask=None) == NULLP
    assert f(dims(kv_dtype=2)) == NULLP                 # fp8 cache without scales
    assert f(dims(head_dim=96)) == DIMS


def test_attn_append_host_checks(lib):
    """taco_paged_tree_attn_append: row dtype, kernel family, pointers and alignment are checked
    on the host."""
    def f(dd, new_dt=1, k=FAKE, v=FAKE, ks=None, vs=None, scale=0.1):
        return lib.taco_paged_tree_attn_append(ctypes.byref(dd), FAKE, k, v, new_dt, FAKE, FAKE, ks, vs, FAKE,
                                               FAKE, FAKE, FAKE, scale, FAKE, None, None)
    assert f(dims(), new_dt=0) == DTYPE                              # f32 rows into a bf16 cache
    assert f(dims(kv_dtype=2), new_dt=2, ks=FAKE, vs=FAKE) == DTYPE  # fp8 rows: f32 or bf16 only
    assert f(dims(max_q_len=16, num_q_heads=64)) == UNSUP            # 128 rows: not the stream kernel
    assert f(dims(path=1)) == UNSUP                                  # forced VALU path
    assert f(dims(num_seqs=0)) == OK
    assert f(dims(), k=None) == NULLP
    assert f(dims(kv_dtype=2), new_dt=0) == NULLP                    # fp8 cache without scales
    assert f(dims(), v=ctypes.c_void_p(0x10008)) == DIMS             # rows move in 16-byte chunks
    assert f(dims(), scale=float("inf")) == DIMS


def test_balanced_append_host_checks(lib):
    """taco_paged_tree_attn_balanced_append: row dtype, pointers, alignment and the kernel family
    (the 32x32x16 shared-tile grid only) are checked on the host."""
    def f(dd, new_dt=1, k=FAKE, v=FAKE, scale=0.1):
        return lib.taco_paged_tree_attn_balanced_append(
            ctypes.byref(dd) if dd is not None else None, FAKE, k, v, new_dt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            scale, FAKE, None, FAKE, 1 << 30, None)
    wide = dict(max_q_len=16, num_q_heads=64)                        # 128 rows per KV head
    assert f(None) == NULLP
    assert f(dims(**wide), new_dt=0) == DTYPE                        # bf16 rows only
    assert f(dims(**wide), k=None) == NULLP
    assert f(dims(**wide), v=ctypes.c_void_p(0x10008)) == DIMS       # rows move in 16-byte chunks
    assert f(dims(**wide), scale=float("inf")) == DIMS
    assert f(dims()) == UNSUP                                        # 4 rows: streaming balanced grid
    assert f(dims(kv_dtype=2, **wide)) == UNSUP                      # fp8 cache
    assert f(dims(path=4, **wide)) == UNSUP                          # 16x16x32 grid
    assert f(dims(num_seqs=0, **wide)) == OK


def test_shared_prefix_host_checks(lib):
    def f(dd, leader=FAKE, group=8, shared=2048, ws=FAKE, nbytes=1 << 30):
        return lib.taco_paged_tree_attn_shared_prefix(ctypes.byref(dd), FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                                      FAKE, FAKE, leader, group, shared, 0.1, FAKE, None, ws,
                                                      nbytes, None)
    assert f(dims(), group=0) == DIMS
    assert f(dims(), shared=100) == DIMS                             # not a multiple of 32 tokens
    assert f(dims(), group=9) == UNSUP                               # 9 members x 4 rows > 32
    assert f(dims(num_seqs=0)) == OK
    assert f(dims(), leader=None) == NULLP
    assert f(dims(), ws=None) == NULLP
    assert f(dims(), ws=ctypes.c_void_p(0x10010)) == DIMS            # workspace 256-byte aligned
    assert f(dims(), nbytes=16) == WS


def test_noalloc_host_checks(lib):
    """The allocation-free balanced entry rejects bad arguments on the host, before any HIP call,
    and the scratch size the binding states is the header's."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(psv._lib.HEADER), "pta.h"), encoding="utf-8").read()
    m = re.search(r"#define PTA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == psv.NOALLOC_SCRATCH_BYTES
    f = lib.taco_paged_tree_attn_balanced_noalloc
    call = lambda d, q=FAKE, out=FAKE, mask=FAKE, scale=0.1: f(
        ctypes.byref(d) if d is not None else None, q, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, mask, scale,
        out, None, None)
    assert call(None) == NULLP
    assert call(dims(head_dim=96)) == DIMS
    assert call(dims(), scale=float("inf")) == DIMS
    assert call(dims(q_dtype=0, kv_dtype=1)) == DTYPE
    assert call(dims(), q=None) == NULLP
    assert call(dims(), out=None) == NULLP
    assert call(dims(max_q_len=4), mask=None) == NULLP
    assert call(dims(q_dtype=0, kv_dtype=0, path=1)) == UNSUP      # vector-ALU rows: no balanced grid
    assert call(dims(num_seqs=0)) == OK


def test_gemm_host_checks(lib):
    """taco_gemm_w8a8 rejects bad arguments on the host, before any HIP call."""
    f = lib.taco_gemm_w8a8
    ok = dict(a=FAKE, sa=FAKE, w=FAKE, sw=FAKE, y=FAKE, M=4, N=4, K=128)
    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["sa"], d["w"], d["sw"], d["y"], d["M"], d["N"], d["K"], None)
    assert call(a=None) == NULLP and call(sw=None) == NULLP and call(y=None) == NULLP
    assert call(K=100) == DIMS and call(K=0) == DIMS and call(M=0) == DIMS and call(N=-1) == DIMS
    assert call(a=ctypes.c_void_p(0x10008)) == DIMS                 # not 16-byte aligned
    assert call(M=1 << 20, K=1 << 13) == DIMS                       # rows x K past 32-bit offsets
    # 66817 rows pad to 67072 in 256-row tiles: 67072 x 64064 passes 2^32 (66944 x 64064 would not)
    assert call(M=66817, K=64064) == DIMS
    t = lib.taco_gemm_w8a8_tiled
    assert t(FAKE, FAKE, None, FAKE, FAKE, 4, 4, 128, None) == NULLP
    assert t(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 100, None) == DIMS


def test_gemm_w8a16_host_checks(lib):
    """taco_gemm_w8a16 rejects bad arguments on the host, before any HIP call."""
    f = lib.taco_gemm_w8a16
    ok = dict(a=FAKE, w=FAKE, s=FAKE, y=FAKE, M=4, N=4, K=256)
    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["w"], d["s"], d["y"], d["M"], d["N"], d["K"], None)
    assert call(a=None) == NULLP and call(w=None) == NULLP and call(s=None) == NULLP and call(y=None) == NULLP
    assert call(K=100) == DIMS and call(K=0) == DIMS and call(M=0) == DIMS and call(N=-1) == DIMS
    assert call(a=ctypes.c_void_p(0x10008)) == DIMS and call(w=ctypes.c_void_p(0x10004)) == DIMS
    assert call(s=ctypes.c_void_p(0x10002)) == DIMS                         # scales not 4-byte aligned
    # 65409 columns pad to 65536 in 128-column tiles: 65536 x 65536 bytes reach 2^32
    assert call(N=65409, K=65536) == DIMS
    # 32769 rows pad to 32896: 32896 x 2 x 65536 bytes pass 2^32
    assert call(M=32769, K=65536) == DIMS
    assert lib.taco_gemm_w8a16_tiled_bytes(0, 64) == 0 and lib.taco_gemm_w8a16_tiled_bytes(4, 100) == 0
    assert lib.taco_gemm_w8a16_tiled_bytes(4, 128) == 128 * 128           # N padded to 128 columns
    assert lib.taco_gemm_w8a16_tiled_bytes(57344, 8192) == 57344 * 8192
    assert lib.taco_gemm_w8a16_tiled_bytes(1 << 19, 1 << 13) == 0         # 2^32 bytes
    pack = lib.taco_gemm_w8a16_pack
    assert pack(None, FAKE, 4, 128, None) == NULLP and pack(FAKE, None, 4, 128, None) == NULLP
    assert pack(FAKE, FAKE, 4, 100, None) == DIMS and pack(FAKE, FAKE, 0, 128, None) == DIMS
    assert pack(ctypes.c_void_p(0x10008), FAKE, 4, 128, None) == DIMS
    t = lib.taco_gemm_w8a16_tiled
    assert t(FAKE, None, FAKE, FAKE, 4, 4, 128, None) == NULLP and t(FAKE, FAKE, FAKE, FAKE, 4, 4, 100, None) == DIMS


def test_gemm_w4a8_host_checks(lib):
    """taco_gemm_w4a8 rejects bad arguments on the host, before any HIP call."""
    f = lib.taco_gemm_w4a8
    ok = dict(a=FAKE, sa=FAKE, w=FAKE, s=FAKE, y=FAKE, M=4, N=4, K=256, G=128)
    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["sa"], d["w"], d["s"], d["y"], d["M"], d["N"], d["K"], d["G"], None)
    assert call(a=None) == NULLP and call(sa=None) == NULLP and call(w=None) == NULLP
    assert call(s=None) == NULLP and call(y=None) == NULLP
    assert call(K=100) == DIMS and call(K=0) == DIMS and call(M=0) == DIMS and call(N=-1) == DIMS
    assert call(G=96) == DIMS and call(G=32) == DIMS and call(K=192, G=128) == DIMS
    assert call(a=ctypes.c_void_p(0x10008)) == DIMS and call(w=ctypes.c_void_p(0x10004)) == DIMS
    assert call(sa=ctypes.c_void_p(0x10002)) == DIMS and call(s=ctypes.c_void_p(0x10001)) == DIMS
    # 65537 rows pad to 65664: 65664 x 65536 bytes pass 2^32
    assert call(M=65537, K=65536, G=64) == DIMS
    t = lib.taco_gemm_w4a8_tiled
    assert t(FAKE, FAKE, None, FAKE, FAKE, 4, 4, 256, 128, None) == NULLP
    assert t(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 256, 96, None) == DIMS


def test_gemm_w4a16_tiled_host_checks(lib):
    """Rearranged-weight entries: sizes, pointers and alignment checked on the host."""
    assert lib.taco_gemm_w4a16_tiled_bytes(0, 64) == 0 and lib.taco_gemm_w4a16_tiled_bytes(4, 100) == 0
    assert lib.taco_gemm_w4a16_tiled_bytes(4, 128) == 128 * 64           # N padded to 128 columns
    assert lib.taco_gemm_w4a16_tiled_bytes(57344, 8192) == 57344 * 4096
    assert lib.taco_gemm_w4a16_tiled_bytes(1 << 20, 1 << 13) == 0         # 2^32 bytes
    pack = lib.taco_gemm_w4a16_pack
    assert pack(None, FAKE, 4, 128, None) == NULLP and pack(FAKE, None, 4, 128, None) == NULLP
    assert pack(FAKE, FAKE, 4, 100, None) == DIMS and pack(FAKE, FAKE, 0, 128, None) == DIMS
    assert pack(ctypes.c_void_p(0x10008), FAKE, 4, 128, None) == DIMS
    f = lib.taco_gemm_w4a16_tiled
    assert f(FAKE, None, FAKE, FAKE, 4, 4, 128, 64, None) == NULLP
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 128, 96, None) == DIMS       # group not a multiple of 64


def test_gemm_w4a16_host_checks(lib):
    """taco_gemm_w4a16 rejects bad arguments on the host, before any HIP call."""
    f = lib.taco_gemm_w4a16
    ok = dict(a=FAKE, w=FAKE, s=FAKE, y=FAKE, M=4, N=4, K=256, G=128)
    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["w"], d["s"], d["y"], d["M"], d["N"], d["K"], d["G"], None)
    assert call(a=None) == NULLP and call(w=None) == NULLP and call(s=None) == NULLP and call(y=None) == NULLP
    assert call(K=100) == DIMS and call(K=0) == DIMS and call(M=0) == DIMS and call(N=-1) == DIMS
    assert call(G=96) == DIMS and call(G=32) == DIMS and call(G=0) == DIMS   # group: a multiple of 64
    assert call(K=192, G=128) == DIMS                                       # group must divide K
    assert call(a=ctypes.c_void_p(0x10008)) == DIMS                         # not 16-byte aligned
    assert call(s=ctypes.c_void_p(0x10002)) == DIMS                         # scales not 4-byte aligned
    assert call(M=1 << 20, K=1 << 12) == DIMS                               # 2 K bytes x rows past 2^32
