"""KV append: write new tokens' K/V rows into their paged cache slots.

Physical blocks are handed out on demand as new tokens are generated (design
talk 大模型倍速推理引擎 TACO-LLM 的设计与实践, section
"4. 支持 Paged Attention"); before a verify step the candidates' K/V rows are
written into the slots of the blocks that hold their logical positions.

Reading adopted: a slot id is physical_block * page_size + offset; a negative
slot means "skip this token".  f32 and bf16 caches take a bit-exact copy of a
row of the same format.  An fp8 cache stores code = RNE_sat(x / scale), the
quotient taken in float32 (the precision the kernel computes it in) with the
caller's per-(block, KV head) scale, rounded to nearest-even e4m3fn and
saturated at +-448 (the fast low-precision storage of the talk's section
"5. 支持 Quantization").
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, encode_fp8_e4m3fn

PAGE = 16


def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, *, cache_dtype: str, new_dtype: str,
              k_scale=None, v_scale=None, page_size: int = PAGE):
    """Return updated copies of (k_cache, v_cache).

    k_new, v_new: [N, Hkv, D] in new_dtype storage (f32 array or bf16 bits).
    slot_mapping: int64 [N].
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for src, dst, scl in ((k_new, k_out, k_scale), (v_new, v_out, v_scale)):
        src = np.asarray(src)
        for n, slot in enumerate(slots):
            if slot < 0:
                continue
            phys, off = int(slot) // page_size, int(slot) % page_size
            if cache_dtype in ("f32", "bf16"):
                if new_dtype != cache_dtype:
                    raise ValueError("f32/bf16 caches take rows of their own format")
                dst[phys, :, off, :] = src[n]
            elif cache_dtype == "fp8":
                if new_dtype == "bf16":
                    x32 = decode_bf16(src[n]).astype(np.float32)
                elif new_dtype == "f32":
                    x32 = np.asarray(src[n], dtype=np.float32)
                else:
                    raise ValueError(new_dtype)
                s32 = np.asarray(scl, dtype=np.float32)[phys][:, None]
                quot = (x32 / s32).astype(np.float32)         # IEEE float32 division
                dst[phys, :, off, :] = encode_fp8_e4m3fn(quot.astype(np.float64))
            else:
                raise ValueError(cache_dtype)
    return k_out, v_out
