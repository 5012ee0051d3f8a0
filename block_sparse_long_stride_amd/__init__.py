"""MI355X (gfx950) library for XAttention's prefill path: block scoring,
threshold block selection (and its Top-K / Top-Ratio variants) and
block-sparse attention (libxattn.so, C-ABI in include/xattn.h) with a thin
Python binding."""
from .xattn import (XattnError, lib, xattn_dit_attention, xattn_dit_workspace_bytes, xattn_full,
                    xattn_head_error, xattn_score, xattn_score_noalloc, xattn_score_select,
                    xattn_score_workspace_bytes,
                    xattn_select, xattn_select_topk, xattn_select_topratio, xattn_sparse_prefill,
                    xattn_tau_dp)

__all__ = ["XattnError", "lib", "xattn_dit_attention", "xattn_dit_workspace_bytes", "xattn_full",
           "xattn_head_error", "xattn_score", "xattn_score_noalloc", "xattn_score_select",
           "xattn_score_workspace_bytes",
           "xattn_select", "xattn_select_topk", "xattn_select_topratio", "xattn_sparse_prefill",
           "xattn_tau_dp"]
