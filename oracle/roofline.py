"""The pages' own back-of-envelope formulas, used to check the report helpers.

* Decode-bound analysis (design talk 大模型倍速推理引擎 TACO-LLM 的设计与实践,
  section "TACO-LLM 如何解决大模型推理瓶颈?"): a model with N parameters in
  fp16 moves 2N bytes and does about 2N flop per generated token; the time
  of each is bytes / bandwidth and flop / peak.
* Lookahead speedup (same talk, "TACO-LLM 性能效果" item 2): with a ceiling
  speedup S for a verify step of k candidates plus the bonus token, and a
  accepted candidates on average, the speedup is S * (a + 1) / (k + 1).
"""
from __future__ import annotations


def decode_io_compute_ms(params: float, bytes_per_param: float, hbm_bytes_per_s: float,
                         peak_flop_per_s: float):
    """(IO time ms, compute time ms) for one single-token decode step."""
    io = params * bytes_per_param / hbm_bytes_per_s * 1e3
    compute = 2.0 * params / peak_flop_per_s * 1e3
    return io, compute


def lookahead_speedup(ceiling: float, lookahead: int, accepted: float) -> float:
    return ceiling * (accepted + 1.0) / (lookahead + 1.0)
