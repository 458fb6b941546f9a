"""Float64 CPU oracle for absorbed-MLA tree-verify attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .kv_compact_oracle import kv_compact
from .tree_accept_oracle import tree_accept, tree_accept_batch, tree_accept_packed
from .mla_verify_oracle import (brute_force_verify, chunk_partial, merge_partials, node_scores,
                                tree_ancestors, tree_mask_words, verify_attention,
                                visible_positions)

__all__ = ["brute_force_verify", "chunk_partial", "kv_compact", "merge_partials", "node_scores",
           "tree_accept", "tree_accept_batch", "tree_accept_packed", "tree_ancestors", "tree_mask_words", "verify_attention",
           "visible_positions"]
