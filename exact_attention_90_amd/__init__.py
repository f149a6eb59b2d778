"""exact_attention_90_amd: FlashAttention forward for MI355X (gfx950).

A C-ABI library (libfa.so, declared in include/fa.h) of hand-written HIP kernels
plus a thin Python binding.  See ``api`` for the entry points.
"""
from .api import fwd, naive_fwd, naive_workspace_bytes, version  # noqa: F401
from ._lib import FAError  # noqa: F401

__all__ = ["fwd", "naive_fwd", "naive_workspace_bytes", "version", "FAError"]
