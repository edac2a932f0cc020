"""Seeded synthetic operands for the quantized GEMM (inputs only).

Weights and activations are float32 N(0, 1) draws quantized the way an offline
quantizer would store them: one float32 scale per row (max |x| / 448, 1.0 for an
all-zero row) and OCP e4m3fn codes of x / scale from torch's float8_e4m3fn cast.
No GEMM arithmetic lives here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

FP8_MAX = 448.0


@dataclass
class W8A8:
    a_codes: np.ndarray    # uint8 [M, K]
    a_scale: np.ndarray    # float32 [M]
    w_codes: np.ndarray    # uint8 [N, K]
    w_scale: np.ndarray    # float32 [N]


def _rowwise_fp8(x: np.ndarray):
    import torch
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    q = np.clip(x / scale[:, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def make_w8a8(M: int, N: int, K: int, seed: int = 0) -> W8A8:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    ac, asc = _rowwise_fp8(a)
    wc, wsc = _rowwise_fp8(w)
    return W8A8(ac, asc, wc, wsc)


# Llama-3.1-70B's MLP gate and up projections side by side (N = 2 x 28672, K = 8192), with the
# verify step's tokens as rows: 32 sequences x 16 candidates
LLAMA70B_GATE_UP = dict(M=512, N=57344, K=8192)


def make_w8a8_device(M: int, N: int, K: int, seed: int, torch, device="cuda"):
    """The same recipe drawn on the GPU (torch's generator), for operand sizes where a host
    draw would take long: returns (a_codes, a_scale, w_codes, w_scale) device tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for rows in (M, N):
        x = torch.randn((rows, K), generator=g, device=device, dtype=torch.float32)
        amax = x.abs().amax(dim=1)
        scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        q = (x / scale[:, None]).clamp(-FP8_MAX, FP8_MAX)
        out += [q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), scale.contiguous()]
        del x, q
    return tuple(out)
