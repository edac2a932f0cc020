"""Plain fp64 CPU oracle for paged tree attention (TEST INFRASTRUCTURE).

Only the test suite, the smoke check of the package entry file and the CPU
baseline leg of the benchmark may import this package.  The library itself
never calls it, and this package never imports the library: the two share no
code, headers, tables or helpers.

Every function states the passage of the TACO-LLM pages it follows; where the
pages are silent the reading adopted is stated in the docstring.
"""
from .formats import (  # noqa: F401
    decode_bf16,
    decode_fp8_e4m3fn,
    encode_fp8_e4m3fn,
    fp8_e4m3fn_table,
)
from .attention import (  # noqa: F401
    gather_page_rows,
    visibility,
    paged_tree_attn,
    paged_tree_attn_partials,
    merge_partials,
)
from .kv_append import kv_append  # noqa: F401
from .accept import accept_commit, accept_path, tree_parents  # noqa: F401
from .roofline import decode_io_compute_ms, lookahead_speedup  # noqa: F401
from .lookahead import LookaheadOracle, tree_mask_from_parents  # noqa: F401
from .quant_gemm import decode_int4_packed, w4a8_gemm, w4a16_gemm, w8a8_gemm, w8a16_gemm  # noqa: F401
