"""Seeded synthetic inputs for paged tree attention.

This package builds the inputs only: context lengths, a paged KV pool with its
block tables, candidate trees and their masks, Q/K/V values and fp8 codes with
their per-page scales. It holds none of the attention arithmetic; both the GPU
path and the CPU oracle consume what it produces.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Spec,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make,
    make_tokens,
    permute_pool,
    sample_tree_parents,
    tree_mask_from_parents,
)
