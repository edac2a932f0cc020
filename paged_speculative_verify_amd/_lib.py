"""ctypes binding of libpta.so (argument marshalling only).

Every function here validates tensor placement, dtype and shape, fills the
C dims struct, passes raw device pointers and the current HIP stream, and
turns a non-zero status into an exception.  All arithmetic runs in the
library's HIP kernels; there is no fallback path.  If libpta.so is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpta.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADER = os.path.join(INCLUDE, "pta.h")

PTA_F32, PTA_BF16, PTA_FP8_E4M3FN = 0, 1, 2
PATHS = {"auto": 0, "valu": 1, "mfma": 2, "tile": 3, "tile16": 4}
STATUS = {0: "PTA_OK", 1: "PTA_ERR_NULL_PTR", 2: "PTA_ERR_BAD_DIMS", 3: "PTA_ERR_BAD_DTYPE",
          4: "PTA_ERR_UNSUPPORTED", 5: "PTA_ERR_WORKSPACE_TOO_SMALL", 6: "PTA_ERR_HIP"}


class PtaDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class PtaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def declared_functions() -> list:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            with open(os.path.join(INCLUDE, h), encoding="utf-8") as f:
                names |= set(re.findall(r"\b(taco_\w+)\s*\(", f.read()))
    return sorted(names)


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_speculative_verify_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(PtaDims)
    lib.taco_paged_tree_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, F, P, P, P]
    lib.taco_paged_tree_attn.restype = ctypes.c_int
    lib.taco_paged_tree_attn_splitk_workspace_size.argtypes = [D, I32]
    lib.taco_paged_tree_attn_splitk_workspace_size.restype = SZ
    lib.taco_paged_tree_attn_splitk.argtypes = [D, P, P, P, P, P, P, P, P, P, F, P, P, I32, P, SZ, P]
    lib.taco_paged_tree_attn_splitk.restype = ctypes.c_int
    lib.taco_paged_tree_attn_append.argtypes = [D, P, P, P, I32, P, P, P, P, P, P, P, P, F, P, P, P]
    lib.taco_paged_tree_attn_append.restype = ctypes.c_int
    lib.taco_paged_tree_attn_balanced_append.argtypes = [D, P, P, P, I32, P, P, P, P, P, P, F, P, P, P, SZ, P]
    lib.taco_paged_tree_attn_balanced_append.restype = ctypes.c_int
    lib.taco_paged_tree_attn_shared_prefix.argtypes = [D, P, P, P, P, P, P, P, P, P, P, I32, I32, F, P, P, P,
                                                       SZ, P]
    lib.taco_paged_tree_attn_shared_prefix.restype = ctypes.c_int
    lib.taco_paged_tree_attn_balanced_workspace_size.argtypes = [D]
    lib.taco_paged_tree_attn_balanced_workspace_size.restype = SZ
    lib.taco_paged_tree_attn_balanced.argtypes = [D, P, P, P, P, P, P, P, P, P, F, P, P, P, SZ, P]
    lib.taco_paged_tree_attn_balanced.restype = ctypes.c_int
    lib.taco_paged_tree_attn_balanced_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, F, P, P, P]
    lib.taco_paged_tree_attn_balanced_noalloc.restype = ctypes.c_int
    lib.taco_kv_append.argtypes = [D, P, P, I32, P, I32, P, P, P, P, P]
    lib.taco_kv_append.restype = ctypes.c_int
    lib.taco_accept_commit.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.taco_accept_commit.restype = ctypes.c_int
    lib.taco_pta_validate.argtypes = [D, P, P, P, P, P]
    lib.taco_pta_validate.restype = ctypes.c_int
    lib.taco_pta_status_string.argtypes = [ctypes.c_int]
    lib.taco_pta_status_string.restype = ctypes.c_char_p
    lib.taco_pta_version.argtypes = []
    lib.taco_pta_version.restype = I32
    lib.taco_pta_calib_stream_read.argtypes = [P, SZ, P, I32, P]
    lib.taco_pta_calib_stream_read.restype = ctypes.c_int
    lib.taco_pta_calib_mfma_bf16.argtypes = [I32, I32, P, P]
    lib.taco_pta_calib_mfma_bf16.restype = ctypes.c_int
    lib.taco_gemm_w8a8.argtypes = [P, P, P, P, P, I32, I32, I32, P]
    lib.taco_gemm_w8a8.restype = ctypes.c_int
    lib.taco_gemm_w4a16.argtypes = [P, P, P, P, I32, I32, I32, I32, P]
    lib.taco_gemm_w4a16.restype = ctypes.c_int
    lib.taco_gemm_w8a16.argtypes = [P, P, P, P, I32, I32, I32, P]
    lib.taco_gemm_w8a16.restype = ctypes.c_int
    lib.taco_gemm_w8a16_tiled_bytes.argtypes = [I32, I32]
    lib.taco_gemm_w8a16_tiled_bytes.restype = SZ
    lib.taco_gemm_w8a16_pack.argtypes = [P, P, I32, I32, P]
    lib.taco_gemm_w8a16_pack.restype = ctypes.c_int
    lib.taco_gemm_w8a16_tiled.argtypes = [P, P, P, P, I32, I32, I32, P]
    lib.taco_gemm_w8a16_tiled.restype = ctypes.c_int
    lib.taco_gemm_w8a8_tiled.argtypes = [P, P, P, P, P, I32, I32, I32, P]
    lib.taco_gemm_w8a8_tiled.restype = ctypes.c_int
    lib.taco_gemm_w4a8.argtypes = [P, P, P, P, P, I32, I32, I32, I32, P]
    lib.taco_gemm_w4a8.restype = ctypes.c_int
    lib.taco_gemm_w4a8_tiled.argtypes = [P, P, P, P, P, I32, I32, I32, I32, P]
    lib.taco_gemm_w4a8_tiled.restype = ctypes.c_int
    lib.taco_gemm_w4a16_tiled_bytes.argtypes = [I32, I32]
    lib.taco_gemm_w4a16_tiled_bytes.restype = SZ
    lib.taco_gemm_w4a16_pack.argtypes = [P, P, I32, I32, P]
    lib.taco_gemm_w4a16_pack.restype = ctypes.c_int
    lib.taco_gemm_w4a16_tiled.argtypes = [P, P, P, P, I32, I32, I32, I32, P]
    lib.taco_gemm_w4a16_tiled.restype = ctypes.c_int
    lib.taco_la_create.argtypes = [I32, I32]
    lib.taco_la_create.restype = P
    lib.taco_la_destroy.argtypes = [P]
    lib.taco_la_destroy.restype = None
    lib.taco_la_set_threads.argtypes = [P, I32]
    lib.taco_la_set_threads.restype = ctypes.c_int
    lib.taco_la_threads.argtypes = [P]
    lib.taco_la_threads.restype = I32
    lib.taco_la_append.argtypes = [P, I32, P, I32]
    lib.taco_la_append.restype = ctypes.c_int
    lib.taco_la_append_batch.argtypes = [P, I32, P, P, P]
    lib.taco_la_append_batch.restype = ctypes.c_int
    lib.taco_la_release.argtypes = [P, I32]
    lib.taco_la_release.restype = ctypes.c_int
    lib.taco_la_propose.argtypes = [P, I32, P, P, I32, P, P, P]
    lib.taco_la_propose.restype = ctypes.c_int
    lib.taco_la_update_budgets.argtypes = [P, I32, P, P, P, I32, I32, I32, P]
    lib.taco_la_update_budgets.restype = ctypes.c_int
    lib.taco_la_tree_mask.argtypes = [I32, I32, P, P, P]
    lib.taco_la_tree_mask.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(st: int) -> None:
    if st != 0:
        msg = load().taco_pta_status_string(st).decode()
        raise PtaError(st, msg)


# ---------------------------------------------------------------- tensor helpers
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _q_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PTA_F32
    if t.dtype == torch.bfloat16:
        return PTA_BF16
    raise ValueError(f"q/new-token dtype must be float32 or bfloat16, got {t.dtype}")


def _kv_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PTA_F32
    if t.dtype == torch.bfloat16:
        return PTA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PTA_FP8_E4M3FN
    raise ValueError(f"cache dtype must be float32, bfloat16 or fp8 e4m3fn/uint8, got {t.dtype}")


def _need(t, name, ndim=None, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


PTA_FLAG_SHARED_PAGES = 1


def make_dims(q, k_cache, block_tables, max_ctx_len=None, path="auto", shared_pages=False) -> PtaDims:
    """shared_pages: the block tables may name one physical page for several sequences
    (PTA_FLAG_SHARED_PAGES: page tiles then keep the default cache policy)."""
    B, Qmax, Hq, D = q.shape
    NB, Hkv, page, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim of q and the caches differ")
    MBS = block_tables.shape[1]
    return PtaDims(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=page,
                   max_q_len=Qmax, max_blocks_per_seq=MBS,
                   max_ctx_len=int(max_ctx_len) if max_ctx_len is not None else MBS * page,
                   num_blocks=NB, q_dtype=_q_code(q), kv_dtype=_kv_code(k_cache),
                   path=PATHS[path], flags=PTA_FLAG_SHARED_PAGES if shared_pages else 0)


def _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale, scales=True):
    torch = _torch()
    _need(q, "q", 4)
    dev = q.device
    _need(k_cache, "k_cache", 4, device=dev)
    _need(v_cache, "v_cache", 4, dtype=k_cache.dtype, device=dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(ctx_lens, "ctx_lens", 1, torch.int32, dev)
    _need(q_lens, "q_lens", 1, torch.int32, dev)
    B, Qmax = q.shape[0], q.shape[1]
    if block_tables.shape[0] != B or ctx_lens.shape[0] != B or q_lens.shape[0] != B:
        raise ValueError("batch sizes of q, block_tables, ctx_lens, q_lens differ")
    if tree_mask is not None:
        _need(tree_mask, "tree_mask", 3, torch.uint8, dev)
        if tuple(tree_mask.shape) != (B, Qmax, Qmax):
            raise ValueError(f"tree_mask must be [{B}, {Qmax}, {Qmax}]")
    if scales and _kv_code(k_cache) == PTA_FP8_E4M3FN:
        for nm, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{nm} is required for an fp8 cache")
            _need(s, nm, 2, torch.float32, dev)
            if tuple(s.shape) != tuple(k_cache.shape[:2]):
                raise ValueError(f"{nm} must be [num_blocks, num_kv_heads]")


def _alloc_out(q, out, lse):
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", 4, q.dtype, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is not None:
        _need(lse, "lse", 3, torch.float32, q.device)
        B, Qmax, Hq, _ = q.shape
        if tuple(lse.shape) != (B, Hq, Qmax):
            raise ValueError(f"lse must be [{B}, {Hq}, {Qmax}]")
    return out, lse


# ---------------------------------------------------------------- entry points
def taco_paged_tree_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, scale,
                         out=None, lse=None, k_scale=None, v_scale=None, max_ctx_len=None,
                         path="auto", stream=None, shared_pages=False):
    """Paged tree attention over each sequence's whole context (see include/pta.h)."""
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    _check(lib.taco_paged_tree_attn(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(ctx_lens),
                                    _ptr(q_lens), _ptr(tree_mask), float(scale), _ptr(out), _ptr(lse),
                                    _stream(stream)))
    return out


def taco_paged_tree_attn_splitk_workspace_size(q, k_cache, block_tables, partition_tokens,
                                               max_ctx_len=None, path="auto", shared_pages=False) -> int:
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    return int(load().taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims), int(partition_tokens)))


def taco_paged_tree_attn_splitk(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                                scale, partition_tokens, out=None, lse=None, k_scale=None,
                                v_scale=None, workspace=None, max_ctx_len=None, path="auto",
                                stream=None, shared_pages=False):
    """Split-K paged tree attention with a log-sum-exp merge (see include/pta.h).

    workspace: a caller-owned uint8 device tensor of at least
    taco_paged_tree_attn_splitk_workspace_size(...) bytes whose arrival-counter
    region is zero before its first use (torch.zeros does it; every call leaves
    the counters zero again); allocated zero-filled here if None.
    """
    torch = _torch()
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    need = int(lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims), int(partition_tokens)))
    if workspace is None:
        if need == 0:
            raise ValueError("invalid dims or partition_tokens for split-K")
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", device=q.device)
    _check(lib.taco_paged_tree_attn_splitk(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale), _ptr(out),
        _ptr(lse), int(partition_tokens), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def taco_paged_tree_attn_append(q, k_new, v_new, k_cache, v_cache, block_tables, ctx_lens, q_lens,
                                tree_mask, scale, out=None, lse=None, k_scale=None, v_scale=None,
                                max_ctx_len=None, path="auto", stream=None, shared_pages=False):
    """KV append fused into the whole-context attention call (see include/pta.h).

    k_new, v_new: [B, Qmax, Hkv, D] device tensors, the candidates' K/V rows, written into their
    paged slots (positions ctx_lens - q_lens .. ctx_lens - 1) before attention reads the cache.
    """
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    B, Qmax, Hq, D = q.shape
    _need(k_new, "k_new", 4, device=q.device)
    _need(v_new, "v_new", 4, k_new.dtype, q.device)
    if tuple(k_new.shape) != (B, Qmax, k_cache.shape[1], D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, Qmax, Hkv, D]")
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    _check(lib.taco_paged_tree_attn_append(
        ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask),
        float(scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def taco_paged_tree_attn_balanced_append(q, k_new, v_new, k_cache, v_cache, block_tables, ctx_lens, q_lens,
                                         tree_mask, scale, out=None, lse=None, workspace=None, max_ctx_len=None,
                                         path="auto", stream=None, shared_pages=False):
    """KV append fused into the balanced entry (see include/pta.h): bf16 k_new, v_new
    [B, Qmax, Hkv, D] written into their paged slots by the grid before it reads them.

    workspace: as taco_paged_tree_attn_balanced (allocated zero-filled here if None).
    """
    torch = _torch()
    lib = load()
    # no scales: an fp8 cache is passed through, for the library to refuse (bf16 caches only)
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, None, None, scales=False)
    B, Qmax, Hq, D = q.shape
    _need(k_new, "k_new", 4, torch.bfloat16, q.device)
    _need(v_new, "v_new", 4, torch.bfloat16, q.device)
    if tuple(k_new.shape) != (B, Qmax, k_cache.shape[1], D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, Qmax, Hkv, D]")
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    need = int(lib.taco_paged_tree_attn_balanced_workspace_size(ctypes.byref(dims)))
    if workspace is None:
        if need == 0:
            raise PtaError(4, "the balanced mode does not serve these dims")
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", device=q.device)
    _check(lib.taco_paged_tree_attn_balanced_append(
        ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale), _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def taco_paged_tree_attn_shared_prefix(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                                       prefix_leader, max_group, shared_tokens, scale, out=None, lse=None,
                                       k_scale=None, v_scale=None, workspace=None, max_ctx_len=None,
                                       path="auto", stream=None, shared_pages=False):
    """Shared-prefix paged tree attention (see include/pta.h): partition 0 of every group of
    consecutive sequences that alias their first shared_tokens / 16 pages is worked once.

    prefix_leader: int32 device tensor [B], the first sequence of each sequence's group.
    workspace: as taco_paged_tree_attn_splitk with partition_tokens = shared_tokens
    (allocated zero-filled here if None).
    """
    torch = _torch()
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    _need(prefix_leader, "prefix_leader", 1, torch.int32, q.device)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    need = int(lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims), int(shared_tokens)))
    if workspace is None:
        if need == 0:
            raise ValueError("invalid dims or shared_tokens")
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", device=q.device)
    _check(lib.taco_paged_tree_attn_shared_prefix(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), _ptr(prefix_leader),
        int(max_group), int(shared_tokens), float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def taco_paged_tree_attn_balanced_workspace_size(q, k_cache, block_tables, max_ctx_len=None,
                                                 path="auto", shared_pages=False) -> int:
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    return int(load().taco_paged_tree_attn_balanced_workspace_size(ctypes.byref(dims)))


def taco_paged_tree_attn_balanced(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                                  scale, out=None, lse=None, k_scale=None, v_scale=None,
                                  workspace=None, max_ctx_len=None, path="auto", stream=None, shared_pages=False):
    """Work-balanced paged tree attention (see include/pta.h).

    workspace: a caller-owned uint8 device tensor of at least
    taco_paged_tree_attn_balanced_workspace_size(...) bytes whose arrival-counter
    region is zero before its first use; allocated zero-filled here if None.
    """
    torch = _torch()
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    need = int(lib.taco_paged_tree_attn_balanced_workspace_size(ctypes.byref(dims)))
    if workspace is None:
        if need == 0:
            raise PtaError(4, "the balanced mode does not serve these dims")
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", device=q.device)
    _check(lib.taco_paged_tree_attn_balanced(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


# PTA_NOALLOC_SCRATCH_BYTES of include/pta.h
NOALLOC_SCRATCH_BYTES = 64 << 20


def taco_paged_tree_attn_balanced_noalloc(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                                          scale, out=None, lse=None, k_scale=None, v_scale=None,
                                          max_ctx_len=None, path="auto", stream=None, shared_pages=False):
    """taco_paged_tree_attn_balanced with the library's own per-GPU scratch array as the workspace
    (no allocation by the library; see include/pta.h for the size limit and the rule that calls
    overlapping on one GPU race).  Allocates out/lse here only when they are not given."""
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    _check(lib.taco_paged_tree_attn_balanced_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale), _ptr(out),
        _ptr(lse), _stream(stream)))
    return out


def taco_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
                   stream=None):
    """Write new tokens' K/V rows into their paged cache slots (see include/pta.h)."""
    torch = _torch()
    lib = load()
    _need(k_new, "k_new", 3)
    dev = k_new.device
    _need(v_new, "v_new", 3, k_new.dtype, dev)
    _need(slot_mapping, "slot_mapping", 1, torch.int64, dev)
    _need(k_cache, "k_cache", 4, device=dev)
    _need(v_cache, "v_cache", 4, k_cache.dtype, dev)
    N, Hkv, D = k_new.shape
    if v_new.shape != k_new.shape or slot_mapping.shape[0] != N:
        raise ValueError("k_new, v_new and slot_mapping disagree on the token count")
    if k_cache.shape[1] != Hkv or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("new rows and caches disagree on heads / head_dim")
    dims = PtaDims(num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D, page_size=k_cache.shape[2],
                   max_q_len=1, max_blocks_per_seq=1, max_ctx_len=1, num_blocks=k_cache.shape[0],
                   q_dtype=PTA_BF16, kv_dtype=_kv_code(k_cache), path=0, flags=0)
    _check(lib.taco_kv_append(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _q_code(k_new),
                              _ptr(slot_mapping), N, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                              _ptr(v_scale), _stream(stream)))


def taco_accept_commit(cand_tokens, target_tokens, target_prev, ctx_lens, q_lens, tree_mask, block_tables,
                       k_cache, v_cache, k_scale=None, v_scale=None, n_accepted=None, accepted_path=None,
                       bonus_tokens=None, new_ctx_lens=None, stream=None):
    """Greedy acceptance of verified candidates and commit of the path's K/V
    rows (see include/pta.h).  Returns (n_accepted, accepted_path, bonus_tokens,
    new_ctx_lens), int32 device tensors; the caches are updated in place."""
    torch = _torch()
    lib = load()
    _need(cand_tokens, "cand_tokens", 2, torch.int32)
    dev = cand_tokens.device
    B, Qmax = cand_tokens.shape
    _need(target_tokens, "target_tokens", 2, torch.int32, dev)
    _need(target_prev, "target_prev", 1, torch.int32, dev)
    _need(ctx_lens, "ctx_lens", 1, torch.int32, dev)
    _need(q_lens, "q_lens", 1, torch.int32, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(k_cache, "k_cache", 4, device=dev)
    _need(v_cache, "v_cache", 4, k_cache.dtype, dev)
    if target_tokens.shape != (B, Qmax) or target_prev.shape[0] != B or ctx_lens.shape[0] != B \
            or q_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("per-sequence inputs disagree on the batch or max_q_len")
    if Qmax > 1:
        _need(tree_mask, "tree_mask", 3, torch.uint8, dev)
        if tree_mask.shape != (B, Qmax, Qmax):
            raise ValueError("tree_mask must be [num_seqs, max_q_len, max_q_len]")
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if accepted_path is None:
        accepted_path = torch.empty(B, Qmax, dtype=torch.int32, device=dev)
    if bonus_tokens is None:
        bonus_tokens = torch.empty(B, dtype=torch.int32, device=dev)
    if new_ctx_lens is None:
        new_ctx_lens = torch.empty(B, dtype=torch.int32, device=dev)
    NB, Hkv, page, D = k_cache.shape
    dims = PtaDims(num_seqs=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D, page_size=page,
                   max_q_len=Qmax, max_blocks_per_seq=block_tables.shape[1],
                   max_ctx_len=block_tables.shape[1] * page, num_blocks=NB,
                   q_dtype=PTA_BF16 if _kv_code(k_cache) != 0 else 0, kv_dtype=_kv_code(k_cache),
                   path=0, flags=0)
    _check(lib.taco_accept_commit(ctypes.byref(dims), _ptr(cand_tokens), _ptr(target_tokens),
                                  _ptr(target_prev), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask),
                                  _ptr(block_tables), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                  _ptr(v_scale), _ptr(n_accepted), _ptr(accepted_path), _ptr(bonus_tokens),
                                  _ptr(new_ctx_lens), _stream(stream)))
    return n_accepted, accepted_path, bonus_tokens, new_ctx_lens


def taco_pta_validate(block_tables, ctx_lens, q_lens, max_q_len, num_blocks, max_ctx_len=None,
                      flags=None, stream=None) -> int:
    """Device-side contract check; returns the flag bits (synchronises the stream)."""
    torch = _torch()
    lib = load()
    dev = block_tables.device
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(ctx_lens, "ctx_lens", 1, torch.int32, dev)
    _need(q_lens, "q_lens", 1, torch.int32, dev)
    B, MBS = block_tables.shape
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=dev)
    dims = PtaDims(num_seqs=B, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=16,
                   max_q_len=int(max_q_len), max_blocks_per_seq=MBS,
                   max_ctx_len=int(max_ctx_len) if max_ctx_len is not None else MBS * 16,
                   num_blocks=int(num_blocks), q_dtype=PTA_BF16, kv_dtype=PTA_BF16, path=0, flags=0)
    _check(lib.taco_pta_validate(ctypes.byref(dims), _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens),
                                 _ptr(flags), _stream(stream)))
    return int(flags.item())


def taco_pta_calib_stream_read(buf, sink, workgroups: int, stream=None) -> None:
    """Streaming read of every byte of buf (a contiguous device tensor; its size a multiple of
    16 KiB) by `workgroups` workgroups; sink: int32 device tensor of at least `workgroups`."""
    torch = _torch()
    _need(buf, "buf")
    _need(sink, "sink", dtype=torch.int32, device=buf.device)
    if sink.numel() < workgroups:
        raise ValueError("sink needs one word per workgroup")
    _check(load().taco_pta_calib_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                             workgroups, _stream(stream)))


def taco_pta_calib_mfma_bf16(workgroups: int, iters: int, sink, stream=None) -> int:
    """bf16 matrix-core loop; returns the flops one launch performs.  sink: float32 device
    tensor of at least `workgroups`."""
    torch = _torch()
    _need(sink, "sink", dtype=torch.float32)
    if sink.numel() < workgroups:
        raise ValueError("sink needs one word per workgroup")
    _check(load().taco_pta_calib_mfma_bf16(workgroups, iters, sink.data_ptr(), _stream(stream)))
    return workgroups * 4 * iters * 4 * 32 * 32 * 16 * 2


def taco_gemm_w8a8(a, a_scale, w, w_scale, y=None, stream=None, tiled=None):
    """W8A8 GEMM (include/pta_gemm.h): a uint8 [M, K] and w uint8 [N, K] e4m3fn codes (or
    float8_e4m3fn tensors), float32 scales [M] and [N]; returns y bf16 [M, N].  tiled=(N, K): w
    is the 1-D output of taco_gemm_w8a16_pack (taco_gemm_w8a8_tiled)."""
    torch = _torch()
    _need(a, "a", 2)
    if a.element_size() != 1:
        raise ValueError("a must hold 1-byte fp8 codes")
    M, K = a.shape
    if tiled is not None:
        N, Kt = (int(v) for v in tiled)
        _need(w, "w", 1, torch.uint8, a.device)
        if Kt != K or w.numel() != int(load().taco_gemm_w8a16_tiled_bytes(N, K)):
            raise ValueError("tiled weights must come from taco_gemm_w8a16_pack of an [N, K] matrix")
    else:
        _need(w, "w", 2)
        if w.element_size() != 1:
            raise ValueError("w must hold 1-byte fp8 codes")
        N = w.shape[0]
        if w.shape[1] != K:
            raise ValueError("a and w disagree on K")
    _need(a_scale, "a_scale", 1, torch.float32, a.device)
    _need(w_scale, "w_scale", 1, torch.float32, a.device)
    if a_scale.numel() != M or w_scale.numel() != N:
        raise ValueError("one scale per row of a and of w")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(y, "y", 2, torch.bfloat16, a.device)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    fn = load().taco_gemm_w8a8_tiled if tiled is not None else load().taco_gemm_w8a8
    _check(fn(a.data_ptr(), a_scale.data_ptr(), w.data_ptr(), w_scale.data_ptr(), y.data_ptr(), M, N, K,
              _stream(stream)))
    return y


def taco_gemm_w8a16_pack(w, stream=None):
    """Weights of taco_gemm_w8a16 (uint8 [N, K] e4m3fn codes) rearranged into the GEMM's load
    order (taco_gemm_w8a16_pack, include/pta_gemm.h); returns the new uint8 buffer: pass it to
    taco_gemm_w8a16 with tiled=(N, K)."""
    torch = _torch()
    _need(w, "w", 2)
    if w.element_size() != 1:
        raise ValueError("w must hold 1-byte fp8 codes")
    N, K = w.shape
    lib = load()
    nbytes = int(lib.taco_gemm_w8a16_tiled_bytes(N, K))
    if nbytes == 0:
        raise ValueError("N and K out of range for the rearranged layout")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check(lib.taco_gemm_w8a16_pack(w.data_ptr(), out.data_ptr(), N, K, _stream(stream)))
    return out


def taco_gemm_w8a16(a, w, w_scale, y=None, stream=None, tiled=None):
    """W8A16 GEMM (include/pta_gemm.h): a bf16 [M, K], w uint8 [N, K] e4m3fn codes (or a
    float8_e4m3fn tensor), w_scale float32 [N]; returns y bf16 [M, N] =
    w_scale[n] * sum_k a[m, k] dec(w[n, k]).  tiled=(N, K): w is the 1-D output of
    taco_gemm_w8a16_pack (taco_gemm_w8a16_tiled)."""
    torch = _torch()
    _need(a, "a", 2, torch.bfloat16)
    M, K = a.shape
    if tiled is not None:
        N, Kt = (int(v) for v in tiled)
        _need(w, "w", 1, torch.uint8, a.device)
        if Kt != K or w.numel() != int(load().taco_gemm_w8a16_tiled_bytes(N, K)):
            raise ValueError("tiled weights must come from taco_gemm_w8a16_pack of an [N, K] matrix")
    else:
        _need(w, "w", 2, device=a.device)
        if w.element_size() != 1:
            raise ValueError("w must hold 1-byte fp8 codes")
        N = w.shape[0]
        if w.shape[1] != K:
            raise ValueError("a and w disagree on K")
    _need(w_scale, "w_scale", 1, torch.float32, a.device)
    if w_scale.numel() != N:
        raise ValueError("one scale per row of w")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(y, "y", 2, torch.bfloat16, a.device)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    fn = load().taco_gemm_w8a16_tiled if tiled is not None else load().taco_gemm_w8a16
    _check(fn(a.data_ptr(), w.data_ptr(), w_scale.data_ptr(), y.data_ptr(), M, N, K, _stream(stream)))
    return y


def taco_gemm_w4a8(a, a_scale, w_packed, w_scale, group, y=None, stream=None, tiled=None):
    """W4A8 GEMM (include/pta_gemm.h): a int8 [M, K] (or uint8 holding two's complement
    codes), a_scale float32 [M], w_packed uint8 [N, K / 2] (as taco_gemm_w4a16), w_scale float32
    [N, K / group]; returns y bf16 [M, N] = a_scale[m] sum_k a[m, k] q[n, k] w_scale[n, k // group].
    tiled=(N, K): w_packed is the 1-D output of taco_gemm_w4a16_pack (taco_gemm_w4a8_tiled)."""
    torch = _torch()
    _need(a, "a", 2)
    if a.dtype not in (torch.int8, torch.uint8):
        raise ValueError("a must hold int8 codes")
    M, K = a.shape
    _need(a_scale, "a_scale", 1, torch.float32, a.device)
    if a_scale.numel() != M:
        raise ValueError("one scale per row of a")
    if tiled is not None:
        N, Kt = (int(v) for v in tiled)
        _need(w_packed, "w_packed", 1, torch.uint8, a.device)
        if Kt != K or w_packed.numel() != int(load().taco_gemm_w4a16_tiled_bytes(N, K)):
            raise ValueError("tiled weights must come from taco_gemm_w4a16_pack of an [N, K / 2] matrix")
    else:
        _need(w_packed, "w_packed", 2, torch.uint8, a.device)
        N = w_packed.shape[0]
        if w_packed.shape[1] * 2 != K:
            raise ValueError("w_packed must hold K / 2 bytes per row")
    group = int(group)
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    _need(w_scale, "w_scale", 2, torch.float32, a.device)
    if tuple(w_scale.shape) != (N, K // group):
        raise ValueError("w_scale must be [N, K / group]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(y, "y", 2, torch.bfloat16, a.device)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    fn = load().taco_gemm_w4a8_tiled if tiled is not None else load().taco_gemm_w4a8
    _check(fn(a.data_ptr(), a_scale.data_ptr(), w_packed.data_ptr(), w_scale.data_ptr(), y.data_ptr(), M, N, K,
              group, _stream(stream)))
    return y


def taco_gemm_w4a16_pack(w_packed, stream=None):
    """Weights of taco_gemm_w4a16 (uint8 [N, K / 2]) rearranged into the GEMM's load order
    (taco_gemm_w4a16_pack, include/pta_gemm.h); returns the new uint8 buffer, whose use
    needs N and K: pass it to taco_gemm_w4a16 with tiled=(N, K)."""
    torch = _torch()
    _need(w_packed, "w_packed", 2, torch.uint8)
    N, K = w_packed.shape[0], w_packed.shape[1] * 2
    lib = load()
    nbytes = int(lib.taco_gemm_w4a16_tiled_bytes(N, K))
    if nbytes == 0:
        raise ValueError("N and K out of range for the rearranged layout")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_packed.device)
    _check(lib.taco_gemm_w4a16_pack(w_packed.data_ptr(), out.data_ptr(), N, K, _stream(stream)))
    return out


def taco_gemm_w4a16(a, w_packed, w_scale, group, y=None, stream=None, tiled=None):
    """W4A16 GEMM (include/pta_gemm.h): a bf16 [M, K], w_packed uint8 [N, K / 2] (two's
    complement int4, k = 2 j in the low nibble of byte j), w_scale float32 [N, K / group];
    returns y bf16 [M, N] = sum_k a[m, k] q[n, k] w_scale[n, k // group].  tiled=(N, K):
    w_packed is the 1-D output of taco_gemm_w4a16_pack (taco_gemm_w4a16_tiled)."""
    torch = _torch()
    _need(a, "a", 2, torch.bfloat16)
    M, K = a.shape
    if tiled is not None:
        N, Kt = (int(v) for v in tiled)
        _need(w_packed, "w_packed", 1, torch.uint8, a.device)
        if Kt != K or w_packed.numel() != int(load().taco_gemm_w4a16_tiled_bytes(N, K)):
            raise ValueError("tiled weights must come from taco_gemm_w4a16_pack of an [N, K / 2] matrix")
    else:
        _need(w_packed, "w_packed", 2, torch.uint8, a.device)
        N = w_packed.shape[0]
        if w_packed.shape[1] * 2 != K:
            raise ValueError("w_packed must hold K / 2 bytes per row")
    group = int(group)
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    _need(w_scale, "w_scale", 2, torch.float32, a.device)
    if tuple(w_scale.shape) != (N, K // group):
        raise ValueError("w_scale must be [N, K / group]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(y, "y", 2, torch.bfloat16, a.device)
    if tuple(y.shape) != (M, N):
        raise ValueError("y must be [M, N]")
    fn = load().taco_gemm_w4a16_tiled if tiled is not None else load().taco_gemm_w4a16
    _check(fn(a.data_ptr(), w_packed.data_ptr(), w_scale.data_ptr(), y.data_ptr(), M, N, K, group,
              _stream(stream)))
    return y


def taco_pta_status_string(status: int) -> str:
    return load().taco_pta_status_string(int(status)).decode()


def taco_pta_version() -> int:
    return int(load().taco_pta_version())


# ---------------------------------------------------------------- prepared calls
class PreparedCall:
    """A library call whose arguments were validated and marshalled once.

    Calling it re-issues the same C call (same tensors, same stream) with no
    per-call Python checks, for tight loops where the host must stay ahead of
    the GPU.  The tensors passed to the preparing function must stay alive and
    keep their storage for as long as the prepared call is used.
    """

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep           # references that keep the tensors alive

    def __call__(self) -> None:
        _check(self._fn(*self._args))


def prepare_paged_tree_attn(mode, q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask,
                            scale, out, lse=None, k_scale=None, v_scale=None, partition_tokens=None,
                            workspace=None, max_ctx_len=None, path="auto", stream=None, prefix_leader=None,
                            max_group=None, k_new=None, v_new=None, shared_pages=False) -> PreparedCall:
    """Validate once and return a PreparedCall for one of the attention entry points.

    mode: "whole" (taco_paged_tree_attn), "whole_append" (taco_paged_tree_attn_append with k_new,
    v_new), "split" (taco_paged_tree_attn_splitk with
    partition_tokens), "shared" (taco_paged_tree_attn_shared_prefix with partition_tokens =
    shared tokens, prefix_leader and max_group), "balanced" (taco_paged_tree_attn_balanced) or
    "balanced_append" (taco_paged_tree_attn_balanced_append with k_new, v_new).  out (and, for
    split/balanced, a zero-initialised workspace of sufficient size) must be given.
    """
    torch = _torch()
    lib = load()
    _check_attn(q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, k_scale, v_scale)
    out, lse = _alloc_out(q, out, lse)
    dims = make_dims(q, k_cache, block_tables, max_ctx_len, path, shared_pages)
    common = (ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
              _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale),
              _ptr(out), _ptr(lse))
    keep = (dims, q, k_cache, v_cache, block_tables, ctx_lens, q_lens, tree_mask, out, lse, k_scale,
            v_scale, workspace)
    st = _stream(stream)
    if mode == "whole":
        return PreparedCall(lib.taco_paged_tree_attn, common + (st,), keep)
    if mode == "whole_append":
        _need(k_new, "k_new", 4, device=q.device)
        _need(v_new, "v_new", 4, k_new.dtype, q.device)
        args = (ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(k_cache),
                _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens),
                _ptr(tree_mask), float(scale), _ptr(out), _ptr(lse), st)
        return PreparedCall(lib.taco_paged_tree_attn_append, args, keep + (k_new, v_new))
    if workspace is None:
        raise ValueError("prepared split/balanced calls need a caller-owned workspace")
    _need(workspace, "workspace", device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    if mode == "split":
        need = int(lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims), int(partition_tokens)))
        if need == 0 or need > wbytes:
            raise ValueError(f"split-K workspace must hold {need} bytes")
        return PreparedCall(lib.taco_paged_tree_attn_splitk,
                            common + (int(partition_tokens), _ptr(workspace), wbytes, st), keep)
    if mode == "shared":
        _need(prefix_leader, "prefix_leader", 1, torch.int32, q.device)
        need = int(lib.taco_paged_tree_attn_splitk_workspace_size(ctypes.byref(dims), int(partition_tokens)))
        if need == 0 or need > wbytes:
            raise ValueError(f"shared-prefix workspace must hold {need} bytes")
        args = (ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), _ptr(prefix_leader),
                int(max_group), int(partition_tokens), float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                wbytes, st)
        return PreparedCall(lib.taco_paged_tree_attn_shared_prefix, args, keep + (prefix_leader,))
    if mode in ("balanced", "balanced_append"):
        need = int(lib.taco_paged_tree_attn_balanced_workspace_size(ctypes.byref(dims)))
        if need == 0 or need > wbytes:
            raise ValueError(f"balanced workspace must hold {need} bytes (0: dims not served)")
        if mode == "balanced":
            return PreparedCall(lib.taco_paged_tree_attn_balanced, common + (_ptr(workspace), wbytes, st), keep)
        _need(k_new, "k_new", 4, torch.bfloat16, q.device)
        _need(v_new, "v_new", 4, torch.bfloat16, q.device)
        args = (ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(k_cache),
                _ptr(v_cache), _ptr(block_tables), _ptr(ctx_lens), _ptr(q_lens), _ptr(tree_mask), float(scale),
                _ptr(out), _ptr(lse), _ptr(workspace), wbytes, st)
        return PreparedCall(lib.taco_paged_tree_attn_balanced_append, args, keep + (k_new, v_new))
    raise ValueError(f"unknown mode {mode!r}")


def prepare_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
                      stream=None) -> PreparedCall:
    """Validate once and return a PreparedCall of taco_kv_append."""
    torch = _torch()
    lib = load()
    _need(k_new, "k_new", 3)
    dev = k_new.device
    _need(v_new, "v_new", 3, k_new.dtype, dev)
    _need(slot_mapping, "slot_mapping", 1, torch.int64, dev)
    _need(k_cache, "k_cache", 4, device=dev)
    _need(v_cache, "v_cache", 4, k_cache.dtype, dev)
    N, Hkv, D = k_new.shape
    dims = PtaDims(num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D, page_size=k_cache.shape[2],
                   max_q_len=1, max_blocks_per_seq=1, max_ctx_len=1, num_blocks=k_cache.shape[0],
                   q_dtype=PTA_BF16, kv_dtype=_kv_code(k_cache), path=0, flags=0)
    args = (ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(slot_mapping), N,
            _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _stream(stream))
    return PreparedCall(lib.taco_kv_append, args,
                        (dims, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale))


# ---------------------------------------------------------------- lookahead cache (host)
def _i32(a) -> "np.ndarray":
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class LookaheadCache:
    """The lookahead cache of include/pta_lookahead.h (host memory, numpy int32 arrays)."""

    def __init__(self, window: int = 16, max_match: int = 8, threads: int = 1):
        self._lib = load()
        self._h = self._lib.taco_la_create(int(window), int(max_match))
        if not self._h:
            raise PtaError(2, "taco_la_create: window 2..64 and max_match 1..window-1")
        self.window, self.max_match = int(window), int(max_match)
        if threads != 1:
            self.set_threads(threads)

    def set_threads(self, n: int) -> None:
        """Batch calls run on n threads (the caller and n - 1 workers of the cache)."""
        _check(self._lib.taco_la_set_threads(self._h, int(n)))

    @property
    def threads(self) -> int:
        return int(self._lib.taco_la_threads(self._h))

    def close(self):
        if self._h:
            self._lib.taco_la_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def append(self, seq: int, tokens) -> None:
        t = _i32(tokens).reshape(-1)
        _check(self._lib.taco_la_append(self._h, int(seq), _np_ptr(t), int(t.size)))

    def append_batch(self, seqs, chunks) -> None:
        """chunks[i] (a token sequence) appended to seqs[i], in one library call."""
        import numpy as np
        sq = _i32(seqs).reshape(-1)
        lens = _i32([len(c) for c in chunks]).reshape(-1)
        if sq.size != lens.size:
            raise ValueError("seqs and chunks differ in length")
        toks = _i32(np.concatenate([np.asarray(c, np.int32).reshape(-1) for c in chunks]) if len(chunks)
                    else np.zeros(0, np.int32))
        _check(self._lib.taco_la_append_batch(self._h, sq.size, _np_ptr(sq), _np_ptr(lens), _np_ptr(toks)))

    def append_packed(self, seqs, lens, tokens) -> None:
        """append_batch with the tokens already packed: int32 arrays seqs [n], lens [n] and
        tokens [sum(lens)] (no per-call conversion beyond a dtype check)."""
        sq, ln, tk = _i32(seqs).reshape(-1), _i32(lens).reshape(-1), _i32(tokens).reshape(-1)
        if sq.size != ln.size or int(ln.sum()) != tk.size:
            raise ValueError("lens must match seqs and sum to the token count")
        _check(self._lib.taco_la_append_batch(self._h, sq.size, _np_ptr(sq), _np_ptr(ln), _np_ptr(tk)))

    def release(self, seq: int) -> None:
        _check(self._lib.taco_la_release(self._h, int(seq)))

    def propose(self, seqs, budgets, max_q: int):
        """(tokens [n, max_q], parents [n, max_q], counts [n]) as int32 arrays."""
        import numpy as np
        sq, bu = _i32(seqs).reshape(-1), _i32(budgets).reshape(-1)
        if sq.size != bu.size:
            raise ValueError("seqs and budgets differ in length")
        n = sq.size
        tok = np.empty((n, max_q), np.int32)
        par = np.empty((n, max_q), np.int32)
        cnt = np.empty(n, np.int32)
        _check(self._lib.taco_la_propose(self._h, n, _np_ptr(sq), _np_ptr(bu), int(max_q), _np_ptr(tok),
                                         _np_ptr(par), _np_ptr(cnt)))
        return tok, par, cnt

    def update_budgets(self, seqs, proposed, accepted, min_len: int, max_len: int, batch_cap: int = 0):
        import numpy as np
        sq, pr, ac = _i32(seqs).reshape(-1), _i32(proposed).reshape(-1), _i32(accepted).reshape(-1)
        if not (sq.size == pr.size == ac.size):
            raise ValueError("seqs, proposed and accepted differ in length")
        out = np.empty(sq.size, np.int32)
        _check(self._lib.taco_la_update_budgets(self._h, sq.size, _np_ptr(sq), _np_ptr(pr), _np_ptr(ac),
                                                int(min_len), int(max_len), int(batch_cap), _np_ptr(out)))
        return out


def taco_la_tree_mask(parents, counts):
    """Ancestor-or-self tree_mask [n, max_q, max_q] uint8 from parent arrays [n, max_q]."""
    import numpy as np
    par = _i32(parents)
    cnt = _i32(counts).reshape(-1)
    n, max_q = par.shape
    mask = np.empty((n, max_q, max_q), np.uint8)
    _check(load().taco_la_tree_mask(n, max_q, _np_ptr(par), _np_ptr(cnt), _np_ptr(mask)))
    return mask
