"""Quantized GEMM, written out plainly in float64 (TEST INFRASTRUCTURE).

The TACO-LLM pages list quantized GEMM operators (W4A8, W4A16, W8A16, W8A8)
among the engine's operators (17173xz.com article, section
"TACO-LLM如何实现降本增效?"; 618zxw.cn article, section "LLM量子化技術による
推論コストの削減", which names fast dequantisation and integer scales for the
GEMM and attention operators; design talk "大模型倍速推理引擎 TACO-LLM 的设计与
实践", section "5. 支持 Quantization（模型量化）": fp32 weights stored as
INT8/FP8 to cut storage and bandwidth).  The pages fix no formats, layouts or
scale granularity; these readings are taken:

  * Y = A . W^T with A [M, K] (activations, one row per token) and W [N, K]
    (one row per output channel), output bf16 rounded to nearest even.
  * W8A8: both operands OCP fp8 e4m3fn codes (the 8-bit float format of the
    KV cache), one float32 scale per activation row and one per weight row:
        Y[m, n] = a_scale[m] * w_scale[n] * sum_k dec(A[m, k]) * dec(W[n, k]).
  * W4A16: A bf16; W signed 4-bit integers (two's complement, -8 .. 7) packed
    two per byte along k (byte j of a row: k = 2 j in the low nibble,
    k = 2 j + 1 in the high nibble), one float32 scale per (row n, group of G
    consecutive k):
        Y[m, n] = sum_k A[m, k] * q[n, k] * w_scale[n, k // G].
  * W8A16: A bf16; W fp8 e4m3fn codes (the W8A8 weight format, which carries
    its own exponent), one float32 scale per weight row:
        Y[m, n] = w_scale[n] * sum_k A[m, k] * dec(W[n, k]).
  * W4A8: A signed 8-bit integers (-128 .. 127) with one float32 scale per
    activation row; W the W4A16 int4 codes and group scales:
        Y[m, n] = a_scale[m] * sum_k A[m, k] * q[n, k] * w_scale[n, k // G].
    (8-bit integers rather than fp8 on the activation side: int4 weights widen
    to int8 exactly, so the products run on integer matrix cores.)

Nothing here is shared with the library.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_fp8_e4m3fn


def decode_int4_packed(packed: np.ndarray, k: int) -> np.ndarray:
    """uint8 [N, k / 2] -> int64 [N, k]: low nibble first, two's complement."""
    p = np.asarray(packed, dtype=np.uint8)
    assert k % 2 == 0 and p.shape[-1] == k // 2
    lo = (p & 0x0F).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    q = np.empty(p.shape[:-1] + (k,), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return np.where(q >= 8, q - 16, q)


def w8a8_gemm(a_codes, a_scale, w_codes, w_scale) -> np.ndarray:
    """fp8 x fp8 GEMM with per-row activation and per-output-channel weight scales, fp64 [M, N]."""
    a = decode_fp8_e4m3fn(a_codes) * np.asarray(a_scale, np.float64)[:, None]
    w = decode_fp8_e4m3fn(w_codes) * np.asarray(w_scale, np.float64)[:, None]
    return a @ w.T


def w4a16_gemm(a_bits, w_packed, w_scale, group: int) -> np.ndarray:
    """bf16 activations x group-scaled int4 weights, fp64 [M, N]."""
    a = decode_bf16(a_bits)
    k = a.shape[1]
    assert k % group == 0
    q = decode_int4_packed(w_packed, k).astype(np.float64)
    s = np.repeat(np.asarray(w_scale, np.float64), group, axis=1)
    assert s.shape == q.shape
    return a @ (q * s).T


def w8a16_gemm(a_bits, w_codes, w_scale) -> np.ndarray:
    """bf16 activations x fp8 e4m3fn weights with one scale per output channel, fp64 [M, N]."""
    a = decode_bf16(a_bits)
    w = decode_fp8_e4m3fn(w_codes) * np.asarray(w_scale, np.float64)[:, None]
    return a @ w.T


def w4a8_gemm(a_codes, a_scale, w_packed, w_scale, group: int) -> np.ndarray:
    """int8 activations (per-row scales) x group-scaled int4 weights, fp64 [M, N]."""
    a = np.asarray(a_codes).astype(np.int8).astype(np.float64) * np.asarray(a_scale, np.float64)[:, None]
    k = a.shape[1]
    assert k % group == 0
    q = decode_int4_packed(w_packed, k).astype(np.float64)
    s = np.repeat(np.asarray(w_scale, np.float64), group, axis=1)
    assert s.shape == q.shape
    return a @ (q * s).T
