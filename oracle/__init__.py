"""CPU oracle for the prune-then-graft step (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library and its binding never depend on it.
"""
from .graft_oracle import (  # noqa: F401
    accept, accept_sample, append_kv, append_kv_rope, as_f64, bf16_bits_to_f64, build_tree,
    build_tree_one, gather_prefix, mask_words, rope, transitions, tree_attention,
    tree_attention_rope, tree_transitions, update_adjacency, update_adjacency_tree,
)
