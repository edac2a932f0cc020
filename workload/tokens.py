"""Seeded synthetic token streams for the lookahead cache (no real text is available).

Stand-in for the workloads the pages name for the cache (summaries, reviews, code: generated
text that repeats phrases from the prompt and from other requests): every stream is built from
pieces chosen at random among
  * a phrase of a pool shared by all streams (cross-request repetition, global cache),
  * a span copied from the stream's own earlier tokens (in-request repetition, local cache),
  * a few fresh random tokens (novel text).
"""
from __future__ import annotations

import numpy as np


def synthetic_streams(n: int, length: int, vocab: int = 1000, seed: int = 0, p_shared: float = 0.45,
                      p_self: float = 0.25, pool: int = 64):
    rng = np.random.default_rng(seed)
    phrases = [list(rng.integers(0, vocab, int(rng.integers(4, 13)))) for _ in range(pool)]
    out = []
    for _ in range(n):
        s = []
        while len(s) < length:
            u = rng.random()
            if u < p_shared:
                s += phrases[int(rng.integers(0, pool))]
            elif u < p_shared + p_self and len(s) >= 8:
                k = int(rng.integers(3, 11))
                i = int(rng.integers(0, len(s) - 2))
                s += s[i:i + k]
            else:
                s += list(rng.integers(0, vocab, int(rng.integers(1, 5))))
        out.append([int(t) for t in s[:length]])
    return out
