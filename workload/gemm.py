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


@dataclass
class W4A16:
    a_bits: np.ndarray     # uint16 [M, K] bf16 bit patterns
    w_packed: np.ndarray   # uint8 [N, K / 2]: k = 2 j in the low nibble of byte j, 2 j + 1 in the high
    w_scale: np.ndarray    # float32 [N, K / group]
    group: int


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's cast)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int [N, K] in -8..7 -> uint8 [N, K / 2], two's complement nibbles, low nibble first."""
    u = (np.asarray(q, np.int64) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def quantize_int4_groups(w: np.ndarray, group: int):
    """Symmetric group quantization of float32 [N, K]: scale = max |x| / 7 over each group of
    `group` consecutive k (1.0 for an all-zero group), q = round-half-even(x / scale) clipped to
    -8..7.  Returns (q int8 [N, K], scale float32 [N, K / group])."""
    N, K = w.shape
    g = w.reshape(N, K // group, group)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / 7.0, 1.0).astype(np.float32)
    q = np.clip(np.rint(g / scale[:, :, None]), -8, 7).astype(np.int8).reshape(N, K)
    return q, scale


def make_w4a16(M: int, N: int, K: int, group: int = 128, seed: int = 0) -> W4A16:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    q, scale = quantize_int4_groups(w, group)
    return W4A16(bf16_bits_of(a), pack_int4(q), scale, group)


def make_w4a16_device(M: int, N: int, K: int, group: int, seed: int, torch, device="cuda"):
    """The same recipe drawn on the GPU: returns (a bf16 [M, K], w_packed uint8 [N, K / 2],
    w_scale float32 [N, K / group]) device tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    a = torch.randn((M, K), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16).contiguous()
    w = torch.randn((N, K // group, group), generator=g, device=device, dtype=torch.float32)
    amax = w.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax))
    q = torch.round(w / scale[:, :, None]).clamp(-8, 7).to(torch.int32).reshape(N, K)
    del w
    u = (q & 0xF).to(torch.uint8)
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).contiguous()
    return a, packed, scale.contiguous()


@dataclass
class W8A16:
    a_bits: np.ndarray     # uint16 [M, K] bf16 bit patterns
    w_codes: np.ndarray    # uint8 [N, K] e4m3fn codes
    w_scale: np.ndarray    # float32 [N]


def make_w8a16(M: int, N: int, K: int, seed: int = 0) -> W8A16:
    """bf16 N(0, 1) activations; N(0, 1) weights quantized to e4m3fn with one scale per row
    (the W8A8 weight recipe)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    wc, wsc = _rowwise_fp8(w)
    return W8A16(bf16_bits_of(a), wc, wsc)


def make_w8a16_device(M: int, N: int, K: int, seed: int, torch, device="cuda"):
    """The same recipe drawn on the GPU: returns (a bf16 [M, K], w_codes uint8 [N, K],
    w_scale float32 [N]) device tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    a = torch.randn((M, K), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16).contiguous()
    x = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x / scale[:, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    del x
    return a, codes, scale.contiguous()


@dataclass
class W4A8:
    a_codes: np.ndarray    # uint8 [M, K] two's complement int8 codes
    a_scale: np.ndarray    # float32 [M]
    w_packed: np.ndarray   # uint8 [N, K / 2], as W4A16
    w_scale: np.ndarray    # float32 [N, K / group]
    group: int


def _rowwise_int8(x: np.ndarray):
    """Symmetric per-row int8 quantization: scale = max |x| / 127 (1.0 for an all-zero row),
    code = round-half-even(x / scale) (|x / scale| <= 127 already)."""
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / 127.0, 1.0).astype(np.float32)
    q = np.clip(np.rint(x / scale[:, None]), -127, 127).astype(np.int8)
    return q.view(np.uint8), scale


def make_w4a8(M: int, N: int, K: int, group: int = 128, seed: int = 0) -> W4A8:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    ac, asc = _rowwise_int8(a)
    q, scale = quantize_int4_groups(w, group)
    return W4A8(ac, asc, pack_int4(q), scale, group)


def make_w4a8_device(M: int, N: int, K: int, group: int, seed: int, torch, device="cuda"):
    """The same recipe drawn on the GPU: returns (a int8 [M, K], a_scale float32 [M], w_packed
    uint8 [N, K / 2], w_scale float32 [N, K / group]) device tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    amax = x.abs().amax(dim=1)
    a_scale = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    a = torch.round(x / a_scale[:, None]).clamp(-127, 127).to(torch.int8).contiguous()
    del x
    w = torch.randn((N, K // group, group), generator=g, device=device, dtype=torch.float32)
    wmax = w.abs().amax(dim=2)
    w_scale = torch.where(wmax > 0, wmax / 7.0, torch.ones_like(wmax))
    q = torch.round(w / w_scale[:, :, None]).clamp(-8, 7).to(torch.int32).reshape(N, K)
    del w
    u = (q & 0xF).to(torch.uint8)
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).contiguous()
    return a, a_scale.contiguous(), packed, w_scale.contiguous()
