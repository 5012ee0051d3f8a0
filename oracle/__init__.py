"""fp64 CPU oracle of the XAttention prefill path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the library.
"""
from .xattn_oracle import (Selection, antidiagonal_sums, approx_attention, block_mass,
                           block_scores, block_sparse_attention, dit_attention, dit_run_density,
                           dit_step_is_dense, find_blocks, find_blocks_topk, find_blocks_topratio,
                           full_attention, head_rel_sq_error, pattern_sums, select_all, tau_dp,
                           tau_levels, to_mask, topratio_count)

__all__ = ["Selection", "antidiagonal_sums", "approx_attention", "block_mass",
           "block_scores", "block_sparse_attention", "dit_attention", "dit_run_density",
           "dit_step_is_dense", "find_blocks", "find_blocks_topk",
           "find_blocks_topratio", "full_attention", "head_rel_sq_error", "pattern_sums",
           "select_all", "tau_dp", "tau_levels", "to_mask", "topratio_count"]
