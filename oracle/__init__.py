"""CPU fp64 oracle for DDTree MLA verify attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg, never by the library.
"""

from .mla_tree_oracle import (  # noqa: F401
    ancestor_masks,
    ancestors_with_self,
    attention_over_slots,
    attention_weights,
    bf16_to_f64,
    brute_force_verify_attention,
    lse_merge,
    node_offsets,
    request_offsets,
    validate_parents,
    verify_attention,
    verify_attention_ragged,
    visible_slots,
)
