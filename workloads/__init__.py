"""Seeded synthetic inputs for DDTree MLA verify attention.

This package only draws and lays out input data (trees, prefix lengths,
page_size=1 token indices, bf16 query and latent-KV values). It holds none of
the attention arithmetic, so the CPU oracle and the HIP library can both be fed
from it without sharing any part of the method.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    LATENT_DIM,
    V_DIM,
    bf16_bits_to_f32,
    chain_tree,
    f32_to_bf16_bits,
    make_config,
    random_tree,
    tiny_tree,
    tree_depths,
)
