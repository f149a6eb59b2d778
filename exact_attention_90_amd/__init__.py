"""exact_attention_90_amd: FlashAttention forward and backward for MI355X (gfx950).

A C-ABI library (libfa.so, declared in include/fa.h) of hand-written HIP kernels
plus a thin Python binding.  See ``api`` for the entry points.
"""
from .api import (bwd, bwd_split, bwd_split_suggest, bwd_split_workspace_bytes,  # noqa: F401
                  bwd_workspace_bytes, fwd, fwd_split, fwd_stats, naive_fwd,
                  naive_workspace_bytes, split_suggest, split_workspace_bytes, version)
from ._lib import FAError  # noqa: F401

__all__ = ["fwd", "fwd_stats", "fwd_split", "bwd_split", "bwd_split_suggest", "bwd_split_workspace_bytes", "split_suggest", "split_workspace_bytes", "bwd", "bwd_workspace_bytes", "naive_fwd",
           "naive_workspace_bytes", "version", "FAError"]
