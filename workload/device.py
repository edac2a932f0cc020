"""Move a Workload's host arrays into torch device tensors (copies only)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class DeviceWorkload:
    q: "object"
    k_cache: "object"
    v_cache: "object"
    k_scale: Optional["object"]
    v_scale: Optional["object"]
    block_tables: "object"
    ctx_lens: "object"
    q_lens: "object"
    tree_mask: Optional["object"]
    scale: float
    max_ctx_len: int


def _t(torch, a: np.ndarray, device, dtype_view=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return t.view(dtype_view) if dtype_view is not None else t


def to_device(w, device="cuda:0") -> DeviceWorkload:
    import torch
    s = w.spec
    qv = torch.bfloat16 if s.q_dtype == "bf16" else None
    kvv = {"f32": None, "bf16": torch.bfloat16, "fp8": None}[s.kv_dtype]
    return DeviceWorkload(
        q=_t(torch, w.q, device, qv),
        k_cache=_t(torch, w.k_cache, device, kvv),
        v_cache=_t(torch, w.v_cache, device, kvv),
        k_scale=_t(torch, w.k_scale, device) if w.k_scale is not None else None,
        v_scale=_t(torch, w.v_scale, device) if w.v_scale is not None else None,
        block_tables=_t(torch, w.block_tables, device),
        ctx_lens=_t(torch, w.ctx_lens, device),
        q_lens=_t(torch, w.q_lens, device),
        tree_mask=_t(torch, w.tree_mask, device) if w.q.shape[1] > 1 else None,
        scale=float(w.scale),
        max_ctx_len=int(w.ctx_lens.max()),
    )


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
