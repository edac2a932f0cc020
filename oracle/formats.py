"""Element formats used by the KV cache, decoded exactly into float64.

The design talk (大模型倍速推理引擎 TACO-LLM 的设计与实践, section
"5. 支持 Quantization") motivates 8-bit floating point storage for bandwidth.
The KV cache here stores OCP FP8 E4M3 ("e4m3fn": 4 exponent bits with bias 7,
3 mantissa bits, no infinities, the all-ones codes 0x7F/0xFF are NaN, largest
finite magnitude 448).  The decoding below is the closed form of that format.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 is the upper 16 bits of an IEEE-754 binary32 pattern.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _fp8_value(code: int) -> float:
    """Closed form of one e4m3fn code: s.eeee.mmm."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * 2.0 ** -6 * (m / 8.0)
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


_TABLE = np.array([_fp8_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3fn_table() -> np.ndarray:
    """All 256 e4m3fn codes decoded to float64 (copy)."""
    return _TABLE.copy()


def decode_fp8_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float64, exactly."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_fp8_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Round values to e4m3fn codes: nearest, ties to even, saturating to +-448.

    NaN maps to 0x7F.  The input is taken as exact float64 values (typically
    float32 quotients); every step below is exact in float64 except the one
    rounding to 3 mantissa bits, which np.rint does half-to-even.
    """
    a = np.asarray(x, dtype=np.float64)
    out = np.zeros(a.shape, dtype=np.uint8)
    sign = np.where(np.signbit(a), 0x80, 0x00).astype(np.uint8)
    mag = np.abs(a)
    nan = np.isnan(a)
    with np.errstate(invalid="ignore", divide="ignore"):
        # subnormal range: multiples of 2^-9 below 2^-6
        sub = mag < 2.0 ** -6
        m_sub = np.rint(np.where(sub, mag, 0.0) / 2.0 ** -9)           # 0..8; 8 == 2^-6, the first normal
        code_sub = m_sub.astype(np.int64)                              # code = m (e = 0), 8 -> 0x08 (e = 1, m = 0)
        # normal range
        safe = np.where(sub | nan, 1.0, np.minimum(mag, 2.0 ** 10))
        e = np.floor(np.log2(safe)).astype(np.int64)
        # guard against log2 landing one off at exact powers of two
        e = np.where(safe < np.ldexp(1.0, e), e - 1, e)
        e = np.where(safe >= np.ldexp(1.0, e + 1), e + 1, e)
        frac = safe / np.ldexp(1.0, e) - 1.0                            # [0, 1), exact
        m = np.rint(frac * 8.0).astype(np.int64)                        # 0..8
        e = np.where(m == 8, e + 1, e)
        m = np.where(m == 8, 0, m)
        code_norm = ((e + 7) << 3) | m
        code_norm = np.minimum(code_norm, 0x7E)                         # saturate at 448
    code = np.where(sub, code_sub, code_norm)
    out[...] = code.astype(np.uint8) | sign
    out[nan] = 0x7F
    return out
